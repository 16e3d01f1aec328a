// Generic tiled kernels: any M, N, K, any pointer alignment, fp32/fp16/bf16,
// and the 8-bit inputs (E4M3, E5M2) with a bf16 result.
//
// One workgroup of 256 lanes (4 wavefronts in a 2x2 grid) owns a 64x64 tile
// of C and walks K in steps of BK (the tiled loop of kernels-book chapter
// "Matrix Multiplication", section "Tiles", and lesson "Matrix
// multiplication", section "Tiles are small rectangles of work").  Every
// input element is fetched with its own bounds check, so out-of-range rows,
// columns and K positions read as zero; the tiles pass through LDS with a
// barrier after filling and a barrier before the next overwrite (chapter
// "Fast matrix multiplication", section "The CUDA kernel": the two-barrier
// rule, and every lane reaches every barrier).  Each wavefront owns a 32x32
// block of C held in 16 fp32 accumulator registers per lane and multiplies
// with one MFMA per K-slice.  This path exists for ragged and unaligned
// shapes; the aligned large shapes run the pipelined kernel instead.
//
// 8-bit inputs are widened to bf16 as they are staged: every finite E4M3
// value (3 significand bits, exponents 2^-9 .. 2^8) and E5M2 value (2 bits,
// 2^-16 .. 2^15) is a bf16 value, so the widening is exact and the bf16 MFMA
// forms the same exact products and fp32 sums.
#include "gemm_internal.h"

namespace dgr {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 64, kBN = 64, kThreads = 256;

template <typename T> struct Vec8;
template <> struct Vec8<_Float16> { typedef f16x8 type; };
template <> struct Vec8<__bf16> { typedef bf16x8 type; };

__device__ inline f32x16 mfma16(f16x8 a, f16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ inline f32x16 mfma16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One-byte storage types of the 8-bit formats (OCP FP8).
struct E4M3 { unsigned char bits; };
struct E5M2 { unsigned char bits; };

// Value of an input element as the MFMA's operand type T.
template <typename T> __device__ inline T widen(T x) { return x; }
// E4M3: sign, 4 exponent bits (bias 7), 3 significand bits; exponent 0 is
// subnormal (m * 2^-9); S.1111.111 is NaN; no infinities.
__device__ inline __bf16 widen(E4M3 x)
{
    const unsigned b = x.bits, e = (b >> 3) & 15u, m = b & 7u;
    unsigned f;
    if (e == 0) f = __builtin_bit_cast(unsigned, (float)m * 0x1p-9f);
    else if (e == 15 && m == 7) f = 0x7fc00000u;
    else f = ((e + 120u) << 23) | (m << 20);
    return (__bf16)__builtin_bit_cast(float, f | ((b & 0x80u) << 24));
}
// E5M2: sign, 5 exponent bits (bias 15), 2 significand bits; exponent 0 is
// subnormal (m * 2^-16); exponent 31 is infinity (m = 0) or NaN.
__device__ inline __bf16 widen(E5M2 x)
{
    const unsigned b = x.bits, e = (b >> 2) & 31u, m = b & 3u;
    unsigned f;
    if (e == 0) f = __builtin_bit_cast(unsigned, (float)m * 0x1p-16f);
    else if (e == 31) f = m ? 0x7fc00000u : 0x7f800000u;
    else f = ((e + 112u) << 23) | (m << 21);
    return (__bf16)__builtin_bit_cast(float, f | ((b & 0x80u) << 24));
}

// 32x32 MFMA result layout: lane l holds column (l % 32); register r holds
// row 8*(r/4) + 4*(l/32) + r%4.
__device__ inline int acc_row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// ------------------------------------------------- fp16/bf16 (and 8-bit in)
// TI: storage type of A and B; T: the MFMA operand type and C's type.
template <typename TI, typename T>
__global__ __launch_bounds__(kThreads) void gemm_generic16_kernel(
    const TI* __restrict__ A, const TI* __restrict__ B, T* __restrict__ C,
    int M, int N, int K, int group_m, Batch bt)
{
    constexpr int BK = 32;
    constexpr int LDK = BK + 8;   // row pitch in elements: 80 bytes, keeps 16-byte alignment
    typedef typename Vec8<T>::type V8;
    __shared__ __attribute__((aligned(16))) T As[kBM * LDK];   // [m][k]
    __shared__ __attribute__((aligned(16))) T Bs[kBN * LDK];   // [n][k]: B tile stored transposed

    int b, tm, tn;
    tile_of_block(blockIdx.x, cdiv_i(M, kBM), cdiv_i(N, kBN), bt.count, group_m, false, b, tm, tn);
    A += b * bt.sa;
    B += b * bt.sb;
    C += b * bt.sc;
    const int m0 = tm * kBM, n0 = tn * kBN;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // fill mapping: A lane -> (row t/4, 8 consecutive k); B lane -> (column t%64, 8 consecutive k)
    const int a_row = t >> 2, a_k = (t & 3) * 8;
    const int b_col = t & 63, b_k = (t >> 6) * 8;
    const int gm = m0 + a_row, gn = n0 + b_col;

    f32x16 acc;
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    // this lane's share of the A and B tiles of the K-step at k0
    auto fetch = [&](int k0, V8& av, V8& bv) __attribute__((always_inline)) {
        for (int e = 0; e < 8; ++e) {
            const int ka = k0 + a_k + e;
            av[e] = (gm < M && ka < K) ? widen(A[(size_t)gm * K + ka]) : T(0.0f);
            const int kb = k0 + b_k + e;
            bv[e] = (kb < K && gn < N) ? widen(B[(size_t)kb * N + gn]) : T(0.0f);
        }
    };
    // fill the LDS tiles, multiply them, and free them for the next fill
    auto step = [&](const V8& av, const V8& bv) __attribute__((always_inline)) {
        *reinterpret_cast<V8*>(&As[a_row * LDK + a_k]) = av;
        *reinterpret_cast<V8*>(&Bs[b_col * LDK + b_k]) = bv;
        __syncthreads();   // tile complete before anyone reads it
        for (int kk = 0; kk < BK; kk += 16) {
            const int ko = kk + 8 * (lane >> 5);
            const V8 a = *reinterpret_cast<const V8*>(&As[(wm * 32 + (lane & 31)) * LDK + ko]);
            const V8 b = *reinterpret_cast<const V8*>(&Bs[(wn * 32 + (lane & 31)) * LDK + ko]);
            acc = mfma16(a, b, acc);
        }
        __syncthreads();   // all reads done before the next fill overwrites the tile
    };

    constexpr int PRE = 4;
    if (K <= PRE * BK) {
        // short K: every K-step's share is fetched at once, so the product
        // waits for memory once rather than once per K-step (K is the same
        // for all lanes: every lane takes the same steps and barriers)
        V8 av[PRE], bv[PRE];
#pragma unroll
        for (int s = 0; s < PRE; ++s)
            if (s * BK < K) fetch(s * BK, av[s], bv[s]);
#pragma unroll
        for (int s = 0; s < PRE; ++s)
            if (s * BK < K) step(av[s], bv[s]);
    } else {
        for (int k0 = 0; k0 < K; k0 += BK) {
            V8 av, bv;
            fetch(k0, av, bv);
            step(av, bv);
        }
    }

    const int col = n0 + wn * 32 + (lane & 31);
    for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 32 + acc_row(lane, r);
        if (row < M && col < N) C[(size_t)row * N + col] = T(acc[r]);
    }
}

// ---------------------------------------------------------------- fp32
// v_mfma_f32_32x32x2_f32: lane l supplies A[l%32][l/32] and B[l/32][l%32];
// products and sums are fp32.
__global__ __launch_bounds__(kThreads) void gemm_generic32_kernel(
    const float* __restrict__ A, const float* __restrict__ B, float* __restrict__ C,
    int M, int N, int K, int group_m, Batch bt)
{
    constexpr int BK = 16;
    constexpr int LDA = BK + 1;    // odd pitch: the 32 rows a wavefront reads land in 32 banks
    __shared__ float As[kBM * LDA];        // [m][k]
    __shared__ float Bs[BK * kBN];         // [k][n]

    int b, tm, tn;
    tile_of_block(blockIdx.x, cdiv_i(M, kBM), cdiv_i(N, kBN), bt.count, group_m, false, b, tm, tn);
    A += b * bt.sa;
    B += b * bt.sb;
    C += b * bt.sc;
    const int m0 = tm * kBM, n0 = tn * kBN;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    const int a_row = t >> 2, a_k = (t & 3) * 4;    // 64 rows x 16 k
    const int b_k = t >> 4, b_col = (t & 15) * 4;   // 16 k x 64 columns
    const int gm = m0 + a_row;

    f32x16 acc;
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += BK) {
        for (int e = 0; e < 4; ++e) {
            const int ka = k0 + a_k + e;
            As[a_row * LDA + a_k + e] = (gm < M && ka < K) ? A[(size_t)gm * K + ka] : 0.0f;
            const int kb = k0 + b_k, gn = n0 + b_col + e;
            Bs[b_k * kBN + b_col + e] = (kb < K && gn < N) ? B[(size_t)kb * N + gn] : 0.0f;
        }
        __syncthreads();
        for (int kk = 0; kk < BK; kk += 2) {
            const float a = As[(wm * 32 + (lane & 31)) * LDA + kk + (lane >> 5)];
            const float b = Bs[(kk + (lane >> 5)) * kBN + wn * 32 + (lane & 31)];
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
        }
        __syncthreads();
    }

    const int col = n0 + wn * 32 + (lane & 31);
    for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 32 + acc_row(lane, r);
        if (row < M && col < N) C[(size_t)row * N + col] = acc[r];
    }
}

}  // namespace

hipError_t launch_generic(const Config& cfg, const LaunchArgs& a)
{
    const int tiles = cdiv_i(a.M, kBM) * cdiv_i(a.N, kBN);
    const dim3 grid(tiles * a.batch.count), block(kThreads);
    switch (a.dtype) {
    case kF32:
        hipLaunchKernelGGL(gemm_generic32_kernel, grid, block, 0, a.stream,
                           static_cast<const float*>(a.A), static_cast<const float*>(a.B),
                           static_cast<float*>(a.C), a.M, a.N, a.K, cfg.group_m, a.batch);
        break;
    case kF16:
        hipLaunchKernelGGL((gemm_generic16_kernel<_Float16, _Float16>), grid, block, 0, a.stream,
                           static_cast<const _Float16*>(a.A), static_cast<const _Float16*>(a.B),
                           static_cast<_Float16*>(a.C), a.M, a.N, a.K, cfg.group_m, a.batch);
        break;
    case kBF16:
        hipLaunchKernelGGL((gemm_generic16_kernel<__bf16, __bf16>), grid, block, 0, a.stream,
                           static_cast<const __bf16*>(a.A), static_cast<const __bf16*>(a.B),
                           static_cast<__bf16*>(a.C), a.M, a.N, a.K, cfg.group_m, a.batch);
        break;
    case kFP8E4M3:
        hipLaunchKernelGGL((gemm_generic16_kernel<E4M3, __bf16>), grid, block, 0, a.stream,
                           static_cast<const E4M3*>(a.A), static_cast<const E4M3*>(a.B),
                           static_cast<__bf16*>(a.C), a.M, a.N, a.K, cfg.group_m, a.batch);
        break;
    case kFP8E5M2:
        hipLaunchKernelGGL((gemm_generic16_kernel<E5M2, __bf16>), grid, block, 0, a.stream,
                           static_cast<const E5M2*>(a.A), static_cast<const E5M2*>(a.B),
                           static_cast<__bf16*>(a.C), a.M, a.N, a.K, cfg.group_m, a.batch);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dgr
