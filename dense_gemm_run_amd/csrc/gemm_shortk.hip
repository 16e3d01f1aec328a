// Products with a short K (at most 128) over many output tiles, such as a
// batch of attention-score-shaped products (64 x 2048 x 2048 x 128): fp16 /
// bf16, rows of whole 16-byte pieces (K and N multiples of 8, A, B, C
// 16-byte aligned).
//
// With K this short a tile's arithmetic (128 x 128 x 128: 1024 MFMA cycles
// per wavefront) is small next to moving its operands in (64 KB) and its C
// out (32 KB), and C is most of the compulsory bytes (2 bytes per output
// against 2*K*(1/128 + 1/128) bytes of A and B): the product is bound by
// writing C to HBM.  A kernel that loads, multiplies and stores one tile and
// exits leaves each tile's load latency exposed; here every workgroup stays
// resident and walks tiles t, t + G, t + 2G, ... (G = two workgroups per CU),
// and issues the next tile's loads as soon as it has read the current one out
// of LDS, so that they fly while it multiplies and stores (the tiled loop of
// kernels-book chapter "Matrix Multiplication", section "Tiles", with the
// whole K range of a tile staged at once; section "The real tiled loop" for
// the zero padding).
//
//  * 128 x 128 tiles, 4 wavefronts in 2 x 2, each 64 x 64 as 4 x 4 MFMA tiles
//    of 16 x 16 (v_mfma_f32_16x16x32_{f16,bf16}, compiler builtins, given
//    the B fragment first so that lane l accumulates row l%16, columns
//    4(l/16) .. +3).
//  * A [128][128] and B [128][128] of a tile go global -> LDS directly
//    (16-byte buffer loads with the LDS destination, 8 + 8 per lane), K
//    zero-padded to 128 through the buffer range check; each lane fetches the
//    global piece that the swizzled layout puts at its LDS slot:
//      A rows are 256 bytes; 16-byte piece p of row r sits at p ^ (r % 16), so
//      the 16 rows one 16-lane group reads (same K) hit 16 distinct pieces;
//      B rows (one K each) are 256 bytes; 32-byte group c of row k sits at
//      c ^ x(k), x(k) = (k % 4) | 4 * ((k / 8) % 2), so the 8 rows a half
//      wavefront's transpose read touches land on 8 distinct groups.
//  * Each K-step's MFMAs run while the next K-step's fragments are read;
//    after the second-last K-step's MFMAs a barrier frees LDS for the next
//    tile's loads.
//  * Epilogue: each wavefront rounds (nearest even) and stages 16 rows of its
//    block at a time in an LDS area of its own (16-byte pieces XOR-ed by
//    (row / 2) % 8) (not the operand buffers,
//    which the next tile's loads are filling), reads them back as whole
//    128-byte row segments and stores them, skipping rows >= M and columns
//    >= N.
#include "gemm_internal.h"
#include "gemm_device.h"

namespace dgr {
namespace {

constexpr int BM = 128, BN = 128, KP = 128;   // tile and the K extent staged
constexpr int KS = KP / 32;                    // MFMA K-steps of 32
constexpr int ROW = KP * 2;                    // bytes per A row in LDS
constexpr int A_BYTES = BM * ROW;              // 32 KB
constexpr int B_BYTES = KP * BN * 2;           // 32 KB
constexpr int LA = A_BYTES / 1024 / 4;         // 1 KB loads per wavefront: 8
constexpr int LB = B_BYTES / 1024 / 4;         // 8
constexpr int STG = 16 * 64 * 2;               // staging per wavefront: 16 rows x 64 columns

__device__ __forceinline__ int b_group(int k) { return (k & 3) | (((k >> 3) & 1) << 2); }

template <typename T> struct Mma;
template <> struct Mma<_Float16> {
    static __device__ __forceinline__ f32x4 run(const u32x4& b, const u32x4& a, const f32x4& c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, b), __builtin_bit_cast(f16x8, a), c,
                                                      0, 0, 0);
    }
};
template <> struct Mma<__bf16> {
    static __device__ __forceinline__ f32x4 run(const u32x4& b, const u32x4& a, const f32x4& c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, a),
                                                       c, 0, 0, 0);
    }
};

template <typename T>
__global__ __launch_bounds__(256, 2) void gemm_shortk_kernel(const T* A, const T* B, T* C, int M, int N, int K,
                                                              int group_m, Batch bt, int total)
{
    __shared__ __attribute__((aligned(1024))) unsigned char sa[A_BYTES];
    __shared__ __attribute__((aligned(1024))) unsigned char sb[B_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char sst[4 * STG];
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
    typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

    const int tiles_m = cdiv_i(M, BM), tiles_n = cdiv_i(N, BN);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int r16 = lane & 15, g = lane >> 4;

    // Loads of tile t's A and B into sa and sb (slot = 16-byte piece of LDS).
    auto issue = [&](int t) __attribute__((always_inline)) {
        int b, tm, tn;
        tile_of_block(t, tiles_m, tiles_n, bt.count, group_m, true, b, tm, tn);
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + b * bt.sa, (unsigned)M * (unsigned)K * 2u);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + b * bt.sb, (unsigned)K * (unsigned)N * 2u);
        const int m0 = tm * BM, n0 = tn * BN;
#pragma unroll
        for (int j = 0; j < LA; ++j) {
            const int slot = (wave * LA + j) * 64 + lane;
            const int r = slot >> 4, p = (slot & 15) ^ (r & 15);
            const unsigned off = (m0 + r < M && 8 * p < K) ? ((unsigned)(m0 + r) * (unsigned)K + 8u * p) * 2u : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (void __attribute__((address_space(3)))*)(sa + (wave * LA + j) * 1024), 16, off, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < LB; ++j) {
            const int slot = (wave * LB + j) * 64 + lane;
            const int k = slot >> 4, s = slot & 15;
            const int p = 2 * ((s >> 1) ^ b_group(k)) + (s & 1);
            const int col = n0 + 8 * p;
            const unsigned off = (k < K && col < N) ? ((unsigned)k * (unsigned)N + (unsigned)col) * 2u : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (void __attribute__((address_space(3)))*)(sb + (wave * LB + j) * 1024), 16, off, 0, 0, 0);
        }
        asm volatile("" ::: "memory");
    };

    // A fragment of tile row bi, K-step s: lane (i, g) -> row i, K 32s + 8g ..;
    // B fragment of tile column bj: two transpose reads (rows 32s + 8g + 4h + r
    // for lane 4r + q of group g, columns 4q .. 4q+3 of the tile's 16): lane i
    // gets column i over K 32s + 8g .. +7.
    auto read_a = [&](int s, int bi) __attribute__((always_inline)) {
        const int rr = wm * 64 + 16 * bi + r16;
        const int p = (4 * s + g) ^ (rr & 15);
        return *(const lds_u32x4*)(sa + rr * ROW + p * 16);
    };
    auto read_b = [&](int s, int bj) __attribute__((always_inline)) {
        const int r = r16 >> 2, q = r16 & 3;
        const int grp = 4 * wn + bj;
        s16x4 h[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int k = 32 * s + 8 * g + 4 * hh + r;
            h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(sb + k * (BN * 2) + (grp ^ b_group(k)) * 32 + 8 * q));
        }
        return __builtin_bit_cast(u32x4, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };

    unsigned char __attribute__((address_space(3)))* stg =
        (unsigned char __attribute__((address_space(3)))*)(sst + wave * STG);
    int t = blockIdx.x;
    issue(t);
    for (; t < total; t += gridDim.x) {
        // this wavefront's loads (and earlier stores) done, then every one's
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        u32x4 fa[KS][4], fb[KS][4];
        auto read_step = [&](int s) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[s][i] = read_a(s, i);
#pragma unroll
            for (int j = 0; j < 4; ++j) fb[s][j] = read_b(s, j);
        };
        f32x4 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        // K-step s's MFMAs run while K-step s+1's operands are read; after
        // the MFMAs of the second-last K-step (the last reads long issued)
        // every wavefront has read the tile out of LDS, and the next tile's
        // loads may overwrite it
        read_step(0);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (s + 1 < KS) read_step(s + 1);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = Mma<T>::run(fb[s][j], fa[s][i], acc[i][j]);
            if (s == KS - 2) {
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                if (t + (int)gridDim.x < total) issue(t + gridDim.x);
            }
        }

        // epilogue: 16 rows (tile row bi) at a time through the staging area;
        // logical 16-byte piece p of staging row r sits at p ^ ((r / 2) % 8):
        // rows of 128 bytes put even and odd rows on the two bank halves, and
        // the 8 rows of each parity that one pass of 8-byte writes touches
        // (same logical piece) land on 8 distinct pieces
        int b, tm, tn;
        tile_of_block(t, tiles_m, tiles_n, bt.count, group_m, true, b, tm, tn);
        T* Cb = C + b * bt.sc;
        const int row0 = tm * BM + wm * 64, col0 = tn * BN + wn * 64;
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
                u32x2 v;
                v[0] = pack2<T>(acc[bi][bj][0], acc[bi][bj][1]);
                v[1] = pack2<T>(acc[bi][bj][2], acc[bi][bj][3]);
                const int p = (2 * bj + (g >> 1)) ^ ((r16 >> 1) & 7);
                *(lds_u32x2*)(stg + r16 * 128 + p * 16 + (g & 1) * 8) = v;
            }
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            asm volatile("" ::: "memory");
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = 8 * h + (lane >> 3), pl = lane & 7;
                const u32x4 v = *(const lds_u32x4*)(stg + r * 128 + (pl ^ ((r >> 1) & 7)) * 16);
                const int row = row0 + 16 * bi + r, col = col0 + 8 * pl;
                if (row < M && col < N) __builtin_nontemporal_store(v, (u32x4*)(Cb + (size_t)row * N + col));
            }
            // the read-back is done before the next tile row overwrites it
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            asm volatile("" ::: "memory");
        }
    }
}

template <typename T> hipError_t launch_t(const Config& cfg, const LaunchArgs& a)
{
    const long long total = (long long)cdiv_i(a.M, BM) * cdiv_i(a.N, BN) * a.batch.count;
    const long long resident = 2LL * (a.cus > 0 ? a.cus : 256);
    const int grid = (int)(total < resident ? total : resident);
    hipLaunchKernelGGL((gemm_shortk_kernel<T>), dim3(grid), dim3(256), 0, a.stream, static_cast<const T*>(a.A),
                       static_cast<const T*>(a.B), static_cast<T*>(a.C), a.M, a.N, a.K, cfg.group_m, a.batch,
                       (int)total);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_shortk(const Config& cfg, const LaunchArgs& a)
{
    if (cfg.bm != BM || cfg.bn != BN || cfg.bk != KP || cfg.threads != 256 || a.K > KP) return hipErrorInvalidValue;
    if (a.dtype == kF16) return launch_t<_Float16>(cfg, a);
    if (a.dtype == kBF16) return launch_t<__bf16>(cfg, a);
    return hipErrorInvalidValue;
}

}  // namespace dgr
