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
//  * the products run as 2-element dot products (v_dot2_f32_{bf16,f16}:
//    two exact 16-bit products added to an fp32 accumulator): each 32-bit
//    word of an A piece is a pair of adjacent K positions, and the matching
//    pairs of B (one per column) are gathered once per chunk and shared by
//    the wavefront's rows, so a piece of 8 A elements costs 4*N operations;
//  * the per-lane fp32 partial sums of the wavefront's R*N outputs are
//    combined across the 64 lanes by a halving exchange: at each step the
//    two partner lanes split the outputs still held, each sending the half
//    it gives up and adding the half it keeps, so P outputs (P = R*N rounded
//    up to a power of two) cost P - 1 + 6 - log2(P) cross-lane moves instead
//    of 6 per output; one lane then rounds (nearest even) and stores each
//    output.
// A second schedule (KS) splits K instead of rows over the workgroup's
// wavefronts: the workgroup owns R rows, wavefront w takes chunks w, w+4, ...
// of the K range, and the four partial sums of each output are added in LDS
// in wavefront order.  Each wavefront then owns R rows at the same wavefront
// count, so each 16-byte piece of B it loads serves more A rows: with
// several columns, B's loads (NV per chunk against R of A) no longer
// outnumber A's.
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

// acc + a[0]*b[0] + a[1]*b[1] for packed pairs of 16-bit values.
template <typename T> struct Dot2;
template <> struct Dot2<_Float16> {
    typedef _Float16 v2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ float fma(v2 a, v2 b, float acc) { return __builtin_amdgcn_fdot2(a, b, acc, false); }
};
template <> struct Dot2<__bf16> {
    typedef __bf16 v2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ float fma(v2 a, v2 b, float acc)
    {
        return __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false);
    }
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

constexpr int pow2_ceil(int x) { return x <= 1 ? 1 : 2 * pow2_ceil((x + 1) / 2); }
constexpr int log2_exact(int p) { return p <= 1 ? 0 : 1 + log2_exact(p / 2); }

// Sum of each of the O values over the 64 lanes.  Returns, on every lane,
// the full sum of value number lane >> (6 - log2(P)) (P = O rounded up to a
// power of two; numbers >= O are padding that sums to zero).
template <int O>
__device__ __forceinline__ float lane_sums(const float (&in)[O], int lane)
{
    constexpr int P = pow2_ceil(O), LG = log2_exact(P);
    static_assert(P <= 64, "at most one value per lane");
    float v[P];
#pragma unroll
    for (int i = 0; i < P; ++i) v[i] = i < O ? in[i] : 0.0f;
    // step s pairs lanes 32 >> s apart: the lane with that bit set keeps
    // the upper half of the values still held (renumbered from 0)
#pragma unroll
    for (int s = 0; s < LG; ++s) {
        const int d = 32 >> s, h = P >> (s + 1);
        // all ones on the lanes that keep the upper half; the halves are
        // chosen with bit masks on values already read (a conditional
        // expression over the two array elements can be turned into one read
        // at a lane-dependent index, which the compiler expands into a chain
        // of compares over the whole array)
        const unsigned m = (lane & d) ? ~0u : 0u;
#pragma unroll
        for (int i = 0; i < h; ++i) {
            const unsigned lo = __builtin_bit_cast(unsigned, v[i]), hi = __builtin_bit_cast(unsigned, v[i + h]);
            const float give = __builtin_bit_cast(float, (lo & m) | (hi & ~m));
            const float keep = __builtin_bit_cast(float, (hi & m) | (lo & ~m));
            v[i] = keep + __shfl_xor(give, d, 64);
        }
    }
    // the lanes that hold the same value number add their partial sums
    float t = v[0];
#pragma unroll
    for (int d = 32 >> LG; d >= 1; d >>= 1) t += __shfl_xor(t, d, 64);
    return t;
}

template <typename T, int NV, int R, int U, bool KS>
__global__ __launch_bounds__(64 * kWaves) void gemv_kernel(const T* A, const T* B, T* C, int M, int K,
                                                           Batch bt)
{
    static_assert(R * NV <= 64, "one lane per output");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tiles_m = cdiv_i(M, KS ? R : kWaves * R);
    int b, tm, tn;
    tile_of_block(blockIdx.x, tiles_m, 1, bt.count, 1, false, b, tm, tn);
    A += b * bt.sa;
    B += b * bt.sb;
    C += b * bt.sc;
    const int row0 = KS ? tm * R : (tm * kWaves + wave) * R;
    // uniform per wavefront, and with KS per workgroup (before its one barrier)
    if (row0 >= M) return;

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

    for (int k0 = KS ? wave * 512 * U : 0; k0 < K; k0 += (KS ? kWaves : 1) * 512 * U) {
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
        // keep every load of the step issued before the first product: left to
        // itself the scheduler may sink loads next to their uses to save
        // registers, which leaves one or two loads in flight
        __builtin_amdgcn_sched_barrier(0);
        typedef typename Dot2<T>::v2 v2;
        typedef T v8 __attribute__((ext_vector_type(8)));
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // B pairs (row k+2j, row k+2j+1) of column v, j = 0..3: elements
            // 2j*NV+v and (2j+1)*NV+v of the 8*NV-element run
            v2 xp[NV][4];
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i0 = 2 * j * NV + v, i1 = (2 * j + 1) * NV + v;
                    const v8 h0 = __builtin_bit_cast(v8, x[u][i0 / 8]);
                    const v8 h1 = __builtin_bit_cast(v8, x[u][i1 / 8]);
                    xp[v][j] = v2{h0[i0 % 8], h1[i1 % 8]};
                }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // A elements 2j, 2j+1 (word j, copied out of the vector first:
                    // a bit cast of a vector-element expression reads word 0)
                    const unsigned wj = w[u][r][j];
                    const v2 wp = __builtin_bit_cast(v2, wj);
#pragma unroll
                    for (int v = 0; v < NV; ++v) acc[r][v] = Dot2<T>::fma(wp, xp[v][j], acc[r][v]);
                }
        }
    }

    // output o = r*NV + v of the wavefront ends on the lanes o*G .. o*G+G-1
    constexpr int G = 64 / pow2_ceil(R * NV);
    float flat[R * NV];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int v = 0; v < NV; ++v) flat[r * NV + v] = acc[r][v];
    const float sum = lane_sums<R * NV>(flat, lane);
    const int o = lane / G;
    const bool holder = lane % G == 0 && o < R * NV;
    if constexpr (KS) {
        // lane o of wavefront 0 adds the four partial sums of output o in
        // wavefront order and stores it
        __shared__ float part[kWaves][R * NV];
        if (holder) part[wave][o] = sum;
        __syncthreads();
        if (wave == 0 && lane < R * NV) {
            float s = part[0][lane];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) s += part[w][lane];
            const int r = lane / NV, v = lane - r * NV;
            if (row0 + r < M) C[(size_t)(row0 + r) * NV + v] = round_out<T>(s);
        }
        return;
    }
    const int r = o / NV, v = o - r * NV;
    if (holder && row0 + r < M) C[(size_t)(row0 + r) * NV + v] = round_out<T>(sum);
}

template <typename T, int NV>
hipError_t launch_nv(const Config& cfg, const LaunchArgs& a)
{
    const T* A = static_cast<const T*>(a.A);
    const T* B = static_cast<const T*>(a.B);
    T* C = static_cast<T*>(a.C);
    // cfg.bm = rows per workgroup: kWaves * R, or R when the wavefronts split K
    const int tiles = cdiv_i(a.M, cfg.bm);
    const dim3 grid(tiles * a.batch.count), block(64 * kWaves);
    if (cfg.sched == 0 && cfg.bm == kWaves * 2)
        hipLaunchKernelGGL((gemv_kernel<T, NV, 2, 4, false>), grid, block, 0, a.stream, A, B, C, a.M, a.K, a.batch);
    else if (cfg.sched == 0 && cfg.bm == kWaves * 4)
        hipLaunchKernelGGL((gemv_kernel<T, NV, 4, 2, false>), grid, block, 0, a.stream, A, B, C, a.M, a.K, a.batch);
    else if (cfg.sched == 1 && cfg.bm == 4)
        hipLaunchKernelGGL((gemv_kernel<T, NV, 4, 4, true>), grid, block, 0, a.stream, A, B, C, a.M, a.K, a.batch);
    else if (cfg.sched == 1 && cfg.bm == 8)
        hipLaunchKernelGGL((gemv_kernel<T, NV, 8, 2, true>), grid, block, 0, a.stream, A, B, C, a.M, a.K, a.batch);
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
