// Pipelined MFMA kernel for fp16/bf16 problems whose rows are 16-byte aligned
// (K and N multiples of 8 elements, A, B, C 16-byte aligned).
//
// Structure (the tiled loop of kernels-book chapter "Matrix Multiplication",
// section "Tiles"; one program per BM x BN output tile with an fp32
// accumulator that lives across the whole K walk):
//
//  * Tile order: 1-D grid, XCD-aware remap + grouped band order
//    (tile_of_block in gemm_internal.h).
//  * Staging: the BM x 64 A tile and 64 x BN B tile of K-step i+1 are copied
//    global -> LDS by buffer loads that write LDS directly (16 bytes per lane,
//    no VGPR round trip) while K-step i is being multiplied; two LDS stages.
//    Out-of-range 16-byte pieces (rows >= M, columns >= N, K positions >= K)
//    are given an offset past the buffer's end, which the buffer unit
//    returns as zeros: the zero padding of the pages' tensor descriptors
//    (chapter "Matrix Multiplication", section "The real tiled loop").
//  * LDS layout: A tile [BM][64] and B tile [64][BN], both with their 16-byte
//    pieces XOR-swizzled by row so the MFMA operand reads spread over the
//    banks (the pages pad rows for the same purpose; chapter "Fast matrix
//    multiplication", section "Shared-memory bank conflicts").
//  * Math: 4 wavefronts in a 2x2 grid, each owning a (BM/2) x (BN/2) block
//    of 32x32 MFMA tiles (v_mfma_f32_32x32x16_{f16,bf16}) whose fp32
//    accumulators stay in registers for the whole K walk.  A operands are
//    read with 16-byte LDS reads; B is stored N-contiguous (as it is in
//    memory) and read with the gfx950 LDS transpose read, which hands each
//    lane 4 consecutive K values of one column.
//  * The MFMA is issued with its operands swapped (B fragment first), which
//    computes the transposed 32x32 block; each lane then holds 4 consecutive
//    columns of one row and the epilogue writes 8-byte pieces, rounding the
//    fp32 sums to the output type (round to nearest even) and skipping rows
//    >= M and columns >= N.
#include "gemm_internal.h"

namespace dgr {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) unsigned char lds_byte;

constexpr int kBK = 64;            // K-step (elements)
constexpr int kRowBytesA = kBK * 2; // one A tile row: 128 bytes = 8 pieces of 16 bytes
constexpr int kThreads = 256;
constexpr unsigned kOOB = 0x80000000u;   // byte offset past any buffer (< 2^31 bytes)

template <typename T> struct Op;
template <> struct Op<_Float16> {
    typedef f16x8 V8;
    static __device__ inline f32x16 mfma(V8 a, V8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Op<__bf16> {
    typedef bf16x8 V8;
    static __device__ inline f32x16 mfma(V8 a, V8 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

// 16-byte piece swizzles.  A rows hold 8 pieces; B rows hold BN/8 pieces and
// the B swizzle moves whole 64-byte groups so an LDS transpose read (which
// covers 64 contiguous bytes of 4 rows per half-wavefront) hits 4 different
// bank groups.
__device__ __forceinline__ int swz_a(int row) { return row & 7; }
template <int BN> __device__ __forceinline__ int swz_b(int k) { return ((k & 7) << 2) & (BN / 8 - 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

template <typename T, int BM, int BN>
__global__ __launch_bounds__(kThreads, 1) void gemm_mfma16_kernel(
    const T* __restrict__ A, const T* __restrict__ B, T* __restrict__ C,
    int M, int N, int K, int group_m)
{
    typedef typename Op<T>::V8 V8;
    constexpr int WM = BM / 2, WN = BN / 2;   // per-wavefront block
    constexpr int FM = WM / 32, FN = WN / 32; // 32x32 MFMA tiles per wavefront
    constexpr int A_BYTES = BM * kRowBytesA;
    constexpr int ROW_B = BN * 2;             // bytes in one B tile row
    constexpr int B_BYTES = kBK * ROW_B;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int A_LOADS = A_BYTES / 1024 / 4;   // 1 KB direct-to-LDS loads per wavefront
    constexpr int B_LOADS = B_BYTES / 1024 / 4;
    static_assert(A_LOADS >= 1 && B_LOADS >= 1, "tile too small");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];

    const int tiles_m = cdiv_i(M, BM), tiles_n = cdiv_i(N, BN);
    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, group_m, true, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform per wavefront
    const int wm = wave >> 1, wn = wave & 1;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (unsigned)M * (unsigned)K * 2u);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B, (unsigned)K * (unsigned)N * 2u);

    // ---- per-lane load geometry (fixed across K-steps)
    // A: load j of this wavefront fills tile rows 8*(wave*A_LOADS + j) .. +8;
    //    lane -> row +lane/8, physical piece lane%8, logical piece p ^ swz.
    // Rows >= M get a base offset of kOOB, so every piece of theirs reads zero.
    unsigned a_row_off[A_LOADS];
    int a_kpiece[A_LOADS];
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
        const int row = 8 * (wave * A_LOADS + j) + (lane >> 3);
        const int piece = (lane & 7) ^ swz_a(row);
        a_row_off[j] = (m0 + row) < M ? (unsigned)(m0 + row) * (unsigned)K * 2u : kOOB;
        a_kpiece[j] = piece * 8;
    }
    // B: 1 KB covers 1024/ROW_B rows of the B tile.
    constexpr int B_ROWS_PER_LOAD = 1024 / ROW_B;
    // Columns >= N get a base offset of kOOB (k*N*2 < 2^31 keeps the sum in range).
    int b_krow[B_LOADS];
    unsigned b_col_off[B_LOADS];
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
        const int byte = lane * 16;
        const int krow = B_ROWS_PER_LOAD * (wave * B_LOADS + j) + byte / ROW_B;
        const int piece = ((byte % ROW_B) / 16) ^ swz_b<BN>(krow);
        const int col = n0 + piece * 8;
        b_krow[j] = krow;
        b_col_off[j] = col < N ? (unsigned)col * 2u : kOOB;
    }

    auto issue_loads = [&](int stage, int k0) {
        lds_byte* base = (lds_byte*)smem + stage * STAGE;
#pragma unroll
        for (int j = 0; j < A_LOADS; ++j) {
            const int k = k0 + a_kpiece[j];
            const unsigned in_row = a_row_off[j] + (unsigned)k * 2u;
            const unsigned off = k < K ? in_row : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (void __attribute__((address_space(3)))*)(base + (wave * A_LOADS + j) * 1024),
                                                     16, off, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < B_LOADS; ++j) {
            const int k = k0 + b_krow[j];
            const unsigned in_col = (unsigned)k * (unsigned)N * 2u + b_col_off[j];
            const unsigned off = k < K ? in_col : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (void __attribute__((address_space(3)))*)(base + A_BYTES + (wave * B_LOADS + j) * 1024),
                                                     16, off, 0, 0, 0);
        }
    };

    // ---- per-lane LDS read geometry
    // A fragment (tile bi, K-slice s): row wm*WM + 32*bi + lane%32, logical piece 2s + lane/32.
    int a_rd[FM];
#pragma unroll
    for (int bi = 0; bi < FM; ++bi) a_rd[bi] = (wm * WM + 32 * bi + (lane & 31)) * kRowBytesA;
    const int a_sel = lane >> 5;
    // B fragment via transpose reads: within each 16-lane group, lane 4r+q
    // points at row r, columns 4q..4q+3 of a 4 x 16 block; the read returns
    // to lane i the 4 rows of column i.  Lanes 0-31 cover K rows 0..7 of the
    // slice, lanes 32-63 rows 8..15; lanes 16-31 / 48-63 the upper 16 columns.
    const int g16 = lane & 15;
    const int b_kr = 8 * (lane >> 5) + (g16 >> 2);          // + 16*s + 4*h
    const int b_cn = 16 * ((lane >> 4) & 1) + 4 * (g16 & 3); // + wn*WN + 32*bj

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = cdiv_i(K, kBK);
    if (nk > 0) issue_loads(0, 0);

    for (int it = 0; it < nk; ++it) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();                       // stage it%2 complete; stage (it+1)%2 free
        if (it + 1 < nk) issue_loads((it + 1) & 1, (it + 1) * kBK);
        const lds_byte* sa = (const lds_byte*)smem + (it & 1) * STAGE;
        const lds_byte* sb = sa + A_BYTES;
#pragma unroll
        for (int s = 0; s < kBK / 16; ++s) {
            V8 af[FM], bf[FN];
#pragma unroll
            for (int bi = 0; bi < FM; ++bi) {
                const int row = wm * WM + 32 * bi + (lane & 31);
                const int piece = (2 * s + a_sel) ^ swz_a(row);
                af[bi] = *(const V8*)(sa + a_rd[bi] + piece * 16);
            }
#pragma unroll
            for (int bj = 0; bj < FN; ++bj) {
                s16x4 h[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int k = 16 * s + 4 * hh + b_kr;
                    const int n = wn * WN + 32 * bj + b_cn;
                    const int piece = (n >> 3) ^ swz_b<BN>(k);
                    const lds_byte* p = sb + k * ROW_B + piece * 16 + (n & 7) * 2;
                    h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)p);
                }
                const s16x8 v = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
                bf[bj] = __builtin_bit_cast(V8, v);
            }
#pragma unroll
            for (int bi = 0; bi < FM; ++bi)
#pragma unroll
                for (int bj = 0; bj < FN; ++bj)
                    acc[bi][bj] = Op<T>::mfma(bf[bj], af[bi], acc[bi][bj]);
        }
    }

    // ---- epilogue: lane holds C[row][col .. col+3] for 4 groups per tile
#pragma unroll
    for (int bi = 0; bi < FM; ++bi) {
        const int row = m0 + wm * WM + 32 * bi + (lane & 31);
        if (row >= M) continue;
        T* crow = C + (size_t)row * N;
#pragma unroll
        for (int bj = 0; bj < FN; ++bj) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = n0 + wn * WN + 32 * bj + 8 * g + 4 * (lane >> 5);
                if (col < N) {
                    typedef T T4 __attribute__((ext_vector_type(4)));
                    T4 v;
                    v[0] = (T)acc[bi][bj][4 * g + 0];
                    v[1] = (T)acc[bi][bj][4 * g + 1];
                    v[2] = (T)acc[bi][bj][4 * g + 2];
                    v[3] = (T)acc[bi][bj][4 * g + 3];
                    *(T4*)(crow + col) = v;
                }
            }
        }
    }
}

template <typename T>
hipError_t launch_t(const Config& cfg, const LaunchArgs& a)
{
    const int tiles = cdiv_i(a.M, cfg.bm) * cdiv_i(a.N, cfg.bn);
    const dim3 grid(tiles), block(kThreads);
    const T* A = static_cast<const T*>(a.A);
    const T* B = static_cast<const T*>(a.B);
    T* C = static_cast<T*>(a.C);
    if (cfg.bm == 256 && cfg.bn == 256)
        hipLaunchKernelGGL((gemm_mfma16_kernel<T, 256, 256>), grid, block, 0, a.stream, A, B, C, a.M, a.N, a.K, cfg.group_m);
    else if (cfg.bm == 256 && cfg.bn == 128)
        hipLaunchKernelGGL((gemm_mfma16_kernel<T, 256, 128>), grid, block, 0, a.stream, A, B, C, a.M, a.N, a.K, cfg.group_m);
    else if (cfg.bm == 128 && cfg.bn == 128)
        hipLaunchKernelGGL((gemm_mfma16_kernel<T, 128, 128>), grid, block, 0, a.stream, A, B, C, a.M, a.N, a.K, cfg.group_m);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma16(const Config& cfg, const LaunchArgs& a)
{
    if (a.dtype == kF16) return launch_t<_Float16>(cfg, a);
    if (a.dtype == kBF16) return launch_t<__bf16>(cfg, a);
    return hipErrorInvalidValue;
}

}  // namespace dgr
