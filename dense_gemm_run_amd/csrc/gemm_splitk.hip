// Second pass of the split-K schedule: C = round(sum over s of P[s]), where
// P[s] is split s's M x N slice of fp32 sums in the workspace (written by the
// split variants of the 16x16x32 and 8-bit kernels).  The slices are added in split order
// in fp32, so a configuration and split count give one bitwise result, and
// the sum is rounded once to the output type (round to nearest even), as the
// single-pass epilogue rounds its accumulator.  Each thread takes 8
// consecutive elements (two 16-byte loads per slice, one 16-byte store); M*N
// is a multiple of 8 because N is.  The pass streams splits*M*N*4 bytes in
// and M*N*2 out, most of it from the caches the first pass just wrote.
#include "gemm_internal.h"
#include "gemm_device.h"

namespace dgr {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* ws, T* C, long long mn, int splits)
{
    const long long stride = (long long)gridDim.x * 256 * 8;
    for (long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 8; i < mn; i += stride) {
        f32x4 lo = *(const f32x4*)(ws + i), hi = *(const f32x4*)(ws + i + 4);
        for (int s = 1; s < splits; ++s) {
            const float* p = ws + (long long)s * mn + i;
            lo += *(const f32x4*)p;
            hi += *(const f32x4*)(p + 4);
        }
        u32x4 v;
        v[0] = pack2<T>(lo[0], lo[1]);
        v[1] = pack2<T>(lo[2], lo[3]);
        v[2] = pack2<T>(hi[0], hi[1]);
        v[3] = pack2<T>(hi[2], hi[3]);
        *(u32x4*)(C + i) = v;
    }
}

}  // namespace

hipError_t launch_reduce_splits(const LaunchArgs& a)
{
    const long long mn = (long long)a.M * a.N;
    if (mn % 8 || a.splits < 1 || !a.ws) return hipErrorInvalidValue;
    const long long groups = (mn / 8 + 255) / 256;
    const dim3 grid((unsigned)(groups < 2048 ? groups : 2048)), block(256);
    if (a.dtype == kF16)
        hipLaunchKernelGGL(reduce_splits_kernel<_Float16>, grid, block, 0, a.stream, a.ws,
                           static_cast<_Float16*>(a.C), mn, a.splits);
    else if (a.dtype == kBF16 || a.dtype == kFP8E4M3 || a.dtype == kFP8E5M2)   // 8-bit inputs: bf16 C
        hipLaunchKernelGGL(reduce_splits_kernel<__bf16>, grid, block, 0, a.stream, a.ws,
                           static_cast<__bf16*>(a.C), mn, a.splits);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace dgr
