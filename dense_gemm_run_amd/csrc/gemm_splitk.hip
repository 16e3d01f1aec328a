// Second pass of the split-K schedule: C = round(sum over s of P[s]), where
// P[s] is split s's M x N slice of fp32 sums in the workspace (written by the
// split variants of the 16x16x32 and 8-bit kernels).  The slices are added in
// split order in fp32, so a configuration and split count give one bitwise
// result, and the sum is rounded once to the output type (round to nearest
// even), as the single-pass epilogue rounds its accumulator.  Each thread
// takes 4 consecutive elements (one 16-byte load per slice, one 8-byte
// store); M*N is a multiple of 4 because N is.  The loads of all slices (of
// 16 at a time beyond 16 splits) are issued together before they are added,
// so a thread waits for memory once, not once per slice.  The pass streams splits*M*N*4
// bytes in and M*N*2 out, most of it from the caches the first pass just
// wrote.
#include "gemm_internal.h"
#include "gemm_device.h"

namespace dgr {
namespace {

constexpr int kSliceBatch = 16;

// S > 0: exactly S slices (straight-line code); S = 0: `splits` slices, in
// batches of kSliceBatch.
template <typename T, int S>
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* ws, T* C, long long mn, int splits)
{
    const long long stride = (long long)gridDim.x * 256 * 4;
    for (long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4; i < mn; i += stride) {
        f32x4 acc;
        if constexpr (S > 0) {
            f32x4 v[S];
#pragma unroll
            for (int j = 0; j < S; ++j) v[j] = *(const f32x4*)(ws + (long long)j * mn + i);
            acc = v[0];
#pragma unroll
            for (int j = 1; j < S; ++j) acc += v[j];
        } else {
            acc = *(const f32x4*)(ws + i);
            for (int s0 = 1; s0 < splits; s0 += kSliceBatch) {
                f32x4 v[kSliceBatch];
#pragma unroll
                for (int j = 0; j < kSliceBatch; ++j)
                    if (s0 + j < splits) v[j] = *(const f32x4*)(ws + (long long)(s0 + j) * mn + i);
#pragma unroll
                for (int j = 0; j < kSliceBatch; ++j)
                    if (s0 + j < splits) acc += v[j];
            }
        }
        u32x2 o;
        o[0] = pack2<T>(acc[0], acc[1]);
        o[1] = pack2<T>(acc[2], acc[3]);
        __builtin_nontemporal_store(o, (u32x2*)(C + i));   // C is not read again
    }
}

template <typename T>
hipError_t launch_reduce_t(const LaunchArgs& a, long long mn, dim3 grid)
{
    T* C = static_cast<T*>(a.C);
    const dim3 block(256);
    switch (a.splits) {
#define DGR_S(S_)                                                                                     \
    case S_:                                                                                           \
        hipLaunchKernelGGL((reduce_splits_kernel<T, S_>), grid, block, 0, a.stream, a.ws, C, mn, S_); \
        break;
        DGR_S(2) DGR_S(3) DGR_S(4) DGR_S(5) DGR_S(6) DGR_S(7) DGR_S(8) DGR_S(9)
        DGR_S(10) DGR_S(11) DGR_S(12) DGR_S(13) DGR_S(14) DGR_S(15) DGR_S(16)
#undef DGR_S
    default:
        hipLaunchKernelGGL((reduce_splits_kernel<T, 0>), grid, block, 0, a.stream, a.ws, C, mn, a.splits);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce_splits(const LaunchArgs& a)
{
    const long long mn = (long long)a.M * a.N;
    if (mn % 4 || a.splits < 1 || !a.ws) return hipErrorInvalidValue;
    const long long groups = (mn / 4 + 255) / 256;
    const dim3 grid((unsigned)(groups < 4096 ? groups : 4096));
    if (a.dtype == kF16) return launch_reduce_t<_Float16>(a, mn, grid);
    if (a.dtype == kBF16 || a.dtype == kFP8E4M3 || a.dtype == kFP8E5M2)   // 8-bit inputs: bf16 C
        return launch_reduce_t<__bf16>(a, mn, grid);
    return hipErrorInvalidValue;
}

}  // namespace dgr
