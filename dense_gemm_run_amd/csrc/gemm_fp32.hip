// fp32 products on the MFMA unit: v_mfma_f32_16x16x4f32, IEEE fp32 products
// and fp32 sums (no reduced-precision input mode), for problems whose rows
// are 16-byte aligned (K and N multiples of 4, A, B, C 16-byte aligned).
//
// The tiled loop of kernels-book chapter "Matrix Multiplication", section
// "Tiles" (one workgroup per BM x BN output tile, an fp32 accumulator per
// output that lives across the whole K walk), shaped for the fp32 matrix
// instruction, which takes one 4-byte value of each operand per lane and
// does 1/16 of the fp16 instruction's work per cycle: the kernel is bound by
// the MFMA pipe, and its memory traffic (16 KB of A and 16 KB of B per
// 128 x 128 x 32 block, about 4096 MFMA cycles) is light.
//
//  * 128 x 128 tile, 4 wavefronts in 2 x 2, each owning 64 x 64 outputs as
//    4 x 4 MFMA tiles of 16 x 16 (64 accumulator registers); two workgroups
//    fit a CU, which hides one's barrier behind the other's MFMAs.  Products
//    with too few such tiles for the chip take 64 x 128 or 64 x 64 tiles
//    (the latter four workgroups per CU).
//  * K is walked in blocks of 32.  Within a block the 8 MFMAs of a tile take
//    K in an order chosen for the operand reads: MFMA j gives lane group g
//    (= lane/16) the K index 8g + j, so a lane's A values of a block are 8
//    consecutive floats of one row (two 16-byte LDS reads).  A product's sum
//    over K does not depend on which K an MFMA step carries, as long as A and
//    B use the same order.
//  * The MFMA takes the B fragment first: it computes the transposed 16 x 16
//    block, so lane l accumulates row l%16 of the tile, columns
//    4*(l/16) .. +3, and stores them as one 16-byte piece of C.
//  * Staging: global -> registers (16-byte buffer loads, one block ahead) ->
//    LDS (two stages, one barrier per block).  A rows are padded to 36 floats
//    (the two 16-byte reads of a fragment then hit 64 distinct banks across
//    16 lanes); B stays [K][N], its 16-column groups XOR-ed by 16*x(k) with
//    x(k) = ((k/8) % 4) ^ (2*(k % 2)), so that the four K rows one 4-byte
//    read gathers (k = 8g + j) land on distinct banks, and so do the four
//    rows of the 32 lanes that a paired read (rows j and j+1 at once, which
//    the compiler forms from two such reads) serves in one pass.
//  * Each block's LDS writes and global loads (for the next block and the
//    one after) are spread over its first 64 MFMAs and its fragment reads
//    over the last 64, so that a wavefront issues MFMAs throughout the block
//    and the other wavefront on its SIMD has little to cover.
//  * Out-of-range 16-byte pieces read zeros through the buffer range check
//    (the zero padding of chapter "Matrix Multiplication", section "The real
//    tiled loop"); only rows < M and columns < N of C are written.
#include "gemm_internal.h"
#include "gemm_device.h"

namespace dgr {
namespace {

constexpr int BK = 32;
constexpr int A_PITCH = BK + 4;   // floats per A row in LDS

__device__ __forceinline__ int b_col(int k, int n) { return n ^ (16 * (((k >> 3) & 3) ^ ((k & 1) << 1))); }

// BM x BN tiles (128 x 128, 64 x 128 or 64 x 64), 4 wavefronts in 2 x 2.
template <int BM, int BN> struct Tile {
    static constexpr int WM = BM / 2, WN = BN / 2;     // per-wavefront block
    static constexpr int FM = WM / 16, FN = WN / 16;   // 16 x 16 tiles per wavefront
    static constexpr int A_FLOATS = BM * A_PITCH, B_FLOATS = BK * BN;
    static constexpr int AL = BM / 32, BL = BN / 32;   // 16-byte loads per lane per block
    static constexpr int PB = BN / 4;                  // 16-byte pieces per B row
};

template <int BM, int BN>
__global__ __launch_bounds__(256, (BM * BN <= 64 * 64 ? 4 : 2)) void gemm_fp32_kernel(const float* A, const float* B,
                                                                                    float* C, int M, int N, int K,
                                                                                    int group_m, int xcd_remap,
                                                                                    Batch bt, unsigned long long* clk)
{
    clock_sample(clk, 0);
    using T = Tile<BM, BN>;
    // (the launch bound: 4 workgroups per CU at 64 x 64, whose registers allow it, else 2)
    constexpr int WM = T::WM, WN = T::WN, FM = T::FM, FN = T::FN, AL = T::AL, BL = T::BL, PB = T::PB;
    static_assert(BN >= 64 && BN % 64 == 0, "the B swizzle permutes 64-column groups");
    __shared__ __attribute__((aligned(16))) float sa[2][T::A_FLOATS];
    __shared__ __attribute__((aligned(16))) float sb[2][T::B_FLOATS];

    typedef __attribute__((address_space(3))) float lds_float;
    auto lds_a = [&](int st) __attribute__((always_inline)) { return (lds_float*)sa[st]; };
    auto lds_b = [&](int st) __attribute__((always_inline)) { return (lds_float*)sb[st]; };

    const int tiles_m = cdiv_i(M, BM), tiles_n = cdiv_i(N, BN);
    int b, tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, bt.count, group_m, xcd_remap != 0, b, tm, tn);
    A += b * bt.sa;
    B += b * bt.sb;
    C += b * bt.sc;
    const int m0 = tm * BM, n0 = tn * BN;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (unsigned)M * (unsigned)K * 4u);
    // A load i of a block: row t/8 + 32i, piece t%8 (4 floats at K 4*(t%8));
    // B load i: K row t/PB + (256/PB)*i, piece t%PB (columns 4*(t%PB) .. +3).
    unsigned a_off[AL];
    int a_k[AL];
    unsigned b_off[BL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int row = t / 8 + 32 * i;
        a_k[i] = 4 * (t % 8);
        a_off[i] = (m0 + row) < M ? ((unsigned)(m0 + row) * (unsigned)K + (unsigned)a_k[i]) * 4u : kOOB;
    }
#pragma unroll
    for (int i = 0; i < BL; ++i) {
        const int k = t / PB + (256 / PB) * i, col = n0 + 4 * (t % PB);
        b_off[i] = col < N ? ((unsigned)k * (unsigned)N + (unsigned)col) * 4u : kOOB;
    }
    u32x4 stage_a[AL], stage_b[BL];
    auto load_block = [&](int k0) __attribute__((always_inline)) {
        k0 = __builtin_amdgcn_readfirstlane(k0);
        const int krem = K - k0;
        const int rows = __builtin_amdgcn_readfirstlane(krem < 0 ? 0 : (krem > BK ? BK : krem));
        const __amdgpu_buffer_rsrc_t rb =
            make_rsrc(B + (size_t)(k0 < K ? k0 : 0) * N, (unsigned)rows * (unsigned)N * 4u);
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            const unsigned ao = a_k[i] < krem ? a_off[i] : kOOB;
            stage_a[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, ao, k0 * 4, 0));
        }
#pragma unroll
        for (int i = 0; i < BL; ++i)
            stage_b[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, b_off[i], 0, 0));
    };
    auto store_block = [&](int st) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            const int row = t / 8 + 32 * i;
            *(u32x4 __attribute__((address_space(3)))*)(lds_a(st) + row * A_PITCH + a_k[i]) = stage_a[i];
        }
#pragma unroll
        for (int i = 0; i < BL; ++i) {
            const int k = t / PB + (256 / PB) * i;
            *(u32x4 __attribute__((address_space(3)))*)(lds_b(st) + k * BN + b_col(k, 4 * (t % PB))) = stage_b[i];
        }
    };

    // fragments of one block: A tile bi, 8 floats of row wm*WM + 16*bi + l%16
    // at K 8*(l/16) ..; B tile bj, K rows 8*(l/16) + j of column
    // wn*WN + 16*bj + l%16
    typedef float f32x8 __attribute__((ext_vector_type(8)));
    f32x8 fa[2][FM], fb[2][FN];
    const int r16 = lane & 15, g = lane >> 4;
    auto read_frags = [&](int set, int st) __attribute__((always_inline)) {
#pragma unroll
        for (int bi = 0; bi < FM; ++bi) {
            const lds_float* p = lds_a(st) + (wm * WM + 16 * bi + r16) * A_PITCH + 8 * g;
            const f32x4 lo = *(const f32x4 __attribute__((address_space(3)))*)p;
            const f32x4 hi = *(const f32x4 __attribute__((address_space(3)))*)(p + 4);
            fa[set][bi] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int bj = 0; bj < FN; ++bj) {
            const int n = wn * WN + 16 * bj + r16;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int k = 8 * g + j;
                fb[set][bj][j] = lds_b(st)[k * BN + b_col(k, n)];
            }
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int bi = 0; bi < FM; ++bi)
#pragma unroll
        for (int bj = 0; bj < FN; ++bj) acc[bi][bj] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto mfma = [&](int set, int j, int bi, int bj) __attribute__((always_inline)) {
        acc[bi][bj] = __builtin_amdgcn_mfma_f32_16x16x4f32(fb[set][bj][j], fa[set][bi][j], acc[bi][bj], 0, 0, 0);
    };

    // prologue: block 0 -> stage 0, its fragments -> set 0, block 1 in flight
    const int nb = cdiv_i(K, BK);
    load_block(0);
    store_block(0);
    __syncthreads();
    read_frags(0, 0);
    load_block(BK);

    // Block it (set it%2, stage it%2): the first half of its MFMAs; the
    // staged block it+1 -> stage (it+1)%2, which every wavefront finished
    // reading (block it-1's fragments) before block it-1's barrier; the loads
    // of block it+2; the barrier; block it+1's fragments -> the other set,
    // between the second half of the MFMAs.
    // Scheduling groups (instruction classes of the compiler's interleave
    // directive): MFMA, LDS read, LDS write, global read.
    constexpr int kMfma = 0x008, kLdsRead = 0x100, kLdsWrite = 0x200, kVmemRead = 0x020;
    constexpr int HALF = 4 * FM * FN;                          // MFMAs per half block
    constexpr int PER_LOAD = (HALF + AL + BL - 1) / (AL + BL);  // MFMAs per LDS write + global load
    constexpr int RGROUPS = HALF / 4, READS = 2 * FM + 8 * FN;  // reads: at most, before pairing
    constexpr int PER_GROUP = (READS + RGROUPS - 1) / RGROUPS;  // LDS reads per 4 MFMAs
    auto block = [&](const int par, int it) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int bi = 0; bi < FM; ++bi)
#pragma unroll
                for (int bj = 0; bj < FN; ++bj) mfma(par, j, bi, bj);
        store_block(par ^ 1);
        load_block((it + 2) * BK);
        // the LDS writes and global loads spread over the MFMAs
#pragma unroll
        for (int i = 0; i < AL + BL; ++i) {
            __builtin_amdgcn_sched_group_barrier(kLdsWrite, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kVmemRead, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kMfma, PER_LOAD, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // this wavefront's LDS writes done, then the barrier (no fence: the
        // loads of block it+2 stay in flight across it); the empty asm
        // statements keep LDS accesses on their side of it
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        read_frags(par ^ 1, par ^ 1);
#pragma unroll
        for (int j = 4; j < 8; ++j)
#pragma unroll
            for (int bi = 0; bi < FM; ++bi)
#pragma unroll
                for (int bj = 0; bj < FN; ++bj) mfma(par, j, bi, bj);
        // the fragment reads of the next block spread over the MFMAs
#pragma unroll
        for (int i = 0; i < RGROUPS; ++i) {
            __builtin_amdgcn_sched_group_barrier(kLdsRead, PER_GROUP, 0);
            __builtin_amdgcn_sched_group_barrier(kMfma, 4, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // blocks rounded up to pairs: an extra block multiplies the zeros its
    // loads brought in
    for (int it = 0; it < nb; it += 2) {
        block(0, it);
        block(1, it + 1);
    }

    // epilogue: lane l of tile (bi, bj) holds row 16*bi + l%16, columns
    // 16*bj + 4*(l/16) .. +3 (N is a multiple of 4: wholly in or out)
    const int row0 = m0 + wm * WM + r16, col0 = n0 + wn * WN + 4 * g;
#pragma unroll
    for (int bi = 0; bi < FM; ++bi)
#pragma unroll
        for (int bj = 0; bj < FN; ++bj) {
            const int row = row0 + 16 * bi, col = col0 + 16 * bj;
            if (row < M && col < N) __builtin_nontemporal_store(acc[bi][bj], (f32x4*)(C + (size_t)row * N + col));
        }
    clock_sample(clk, 1);
}

template <int BM, int BN> hipError_t launch_tile(const LaunchArgs& a, const Config& cfg)
{
    const int tiles = cdiv_i(a.M, BM) * cdiv_i(a.N, BN);
    hipLaunchKernelGGL((gemm_fp32_kernel<BM, BN>), dim3(tiles * a.batch.count), dim3(256), 0, a.stream,
                       static_cast<const float*>(a.A), static_cast<const float*>(a.B), static_cast<float*>(a.C), a.M,
                       a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.clk);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fp32(const Config& cfg, const LaunchArgs& a)
{
    if (a.dtype != kF32 || cfg.bk != BK || cfg.threads != 256) return hipErrorInvalidValue;
    if (cfg.bm == 128 && cfg.bn == 128) return launch_tile<128, 128>(a, cfg);
    if (cfg.bm == 64 && cfg.bn == 128) return launch_tile<64, 128>(a, cfg);
    if (cfg.bm == 64 && cfg.bn == 64) return launch_tile<64, 64>(a, cfg);
    return hipErrorInvalidValue;
}

}  // namespace dgr
