// Matrix-vector kernel for C = A·B with few columns (N <= 4): decode-time
// y = W·x, W = A [M, K] row-major, x = B [K, N] (chapter "Fast matrix
// multiplication", section "Decode is a different problem: GEMV").
//
// Every weight is used once, so there is nothing to tile: the kernel streams
// A at HBM bandwidth, as that section prescribes:
//  * coalesced 16-byte loads: lane l of a wavefront reads elements
//    8l .. 8l+7 of a 512-element chunk of a row, so a wavefront instruction
//    covers 1 KB of one row;
//  * enough parallelism: each wavefront owns R consecutive rows and keeps
//    U chunks of each in flight (U*R loads of 16 bytes per lane) before it
//    multiplies; the matching 8 x N values of B are loaded once per chunk and
//    shared by the R rows (B is small and stays in the caches);
//  * the per-lane fp32 partial sums of each output are combined with a
//    butterfly of cross-lane adds, and one lane rounds (nearest even) and
//    stores each output.
// K positions >= K read zeros: A pieces are switched to an offset past the
// buffer end per chunk, and B's buffer ends at row K.  Rows >= M are skipped
// whole (a wavefront's rows are uniform).
#include "gemm_internal.h"
#include "gemm_device.h"

namespace dgr {
namespace {

constexpr int kWaves = 4;   // wavefronts per workgroup

template <typename T> struct Widen;
template <> struct Widen<_Float16> {
    static __device__ __forceinline__ float lo(unsigned u) { return (float)__builtin_bit_cast(_Float16, (unsigned short)(u & 0xffffu)); }
    static __device__ __forceinline__ float hi(unsigned u) { return (float)__builtin_bit_cast(_Float16, (unsigned short)(u >> 16)); }
};
template <> struct Widen<__bf16> {
    // bf16 -> fp32 is exact: the 16 bits are the high half of the fp32 word
    static __device__ __forceinline__ float lo(unsigned u) { return __builtin_bit_cast(float, u << 16); }
    static __device__ __forceinline__ float hi(unsigned u) { return __builtin_bit_cast(float, u & 0xffff0000u); }
};

template <typename T> __device__ __forceinline__ T round_out(float x);
template <> __device__ __forceinline__ _Float16 round_out<_Float16>(float x) { return (_Float16)x; }
template <> __device__ __forceinline__ __bf16 round_out<__bf16>(float x) { return (__bf16)x; }

// Element i of a 16-byte piece, widened to fp32.
template <typename T> __device__ __forceinline__ float elem(const u32x4& v, int i)
{
    const unsigned u = v[i >> 1];
    return (i & 1) ? Widen<T>::hi(u) : Widen<T>::lo(u);
}

template <typename T, int NV, int R, int U>
__global__ __launch_bounds__(64 * kWaves) void gemv_kernel(const T* A, const T* B, T* C, int M, int K,
                                                           Batch bt)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tiles_m = cdiv_i(M, kWaves * R);
    int b, tm, tn;
    tile_of_block(blockIdx.x, tiles_m, 1, bt.count, 1, false, b, tm, tn);
    A += b * bt.sa;
    B += b * bt.sb;
    C += b * bt.sc;
    const int row0 = (tm * kWaves + wave) * R;
    if (row0 >= M) return;   // uniform per wavefront; the kernel has no barrier

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (unsigned)M * (unsigned)K * 2u);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B, (unsigned)K * (unsigned)NV * 2u);
    unsigned row_off[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        row_off[r] = row0 + r < M ? (unsigned)(row0 + r) * (unsigned)K * 2u : kOOB;

    float acc[R][NV];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[r][v] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += 512 * U) {
        u32x4 w[U][R], x[U][NV];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k0 + 512 * u + 8 * lane;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const unsigned ro = row_off[r];
                const unsigned off = (k < K && ro != kOOB) ? ro + (unsigned)k * 2u : kOOB;
                w[u][r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
            }
            // B rows k .. k+7 are 8*NV contiguous elements; rows >= K lie past the buffer
#pragma unroll
            for (int v = 0; v < NV; ++v)
                x[u][v] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, (unsigned)k * NV * 2u + 16u * v, 0, 0));
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float xe[NV];
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const int i = e * NV + v;   // element of the 8*NV-element run of B
                    xe[v] = elem<T>(x[u][i / 8], i % 8);
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float we = elem<T>(w[u][r], e);
#pragma unroll
                    for (int v = 0; v < NV; ++v) acc[r][v] = __builtin_fmaf(we, xe[v], acc[r][v]);
                }
            }
    }

    // butterfly over the 64 lanes: every lane ends with the full sums
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float s = acc[r][v];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
            acc[r][v] = s;
        }
    // lane r*NV + v stores output (row0 + r, v)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int v = 0; v < NV; ++v)
            if (lane == r * NV + v && row0 + r < M) C[(size_t)(row0 + r) * NV + v] = round_out<T>(acc[r][v]);
}

template <typename T, int NV>
hipError_t launch_nv(const Config& cfg, const LaunchArgs& a)
{
    const T* A = static_cast<const T*>(a.A);
    const T* B = static_cast<const T*>(a.B);
    T* C = static_cast<T*>(a.C);
    // cfg.bm = rows per workgroup = kWaves * R
    const int tiles = cdiv_i(a.M, cfg.bm);
    const dim3 grid(tiles * a.batch.count), block(64 * kWaves);
    if (cfg.bm == kWaves * 2)
        hipLaunchKernelGGL((gemv_kernel<T, NV, 2, 4>), grid, block, 0, a.stream, A, B, C, a.M, a.K, a.batch);
    else if (cfg.bm == kWaves * 4)
        hipLaunchKernelGGL((gemv_kernel<T, NV, 4, 2>), grid, block, 0, a.stream, A, B, C, a.M, a.K, a.batch);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const Config& cfg, const LaunchArgs& a)
{
    switch (a.N) {
    case 1: return launch_nv<T, 1>(cfg, a);
    case 2: return launch_nv<T, 2>(cfg, a);
    case 3: return launch_nv<T, 3>(cfg, a);
    case 4: return launch_nv<T, 4>(cfg, a);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemv(const Config& cfg, const LaunchArgs& a)
{
    if (a.dtype == kF16) return launch_t<_Float16>(cfg, a);
    if (a.dtype == kBF16) return launch_t<__bf16>(cfg, a);
    return hipErrorInvalidValue;
}

}  // namespace dgr
