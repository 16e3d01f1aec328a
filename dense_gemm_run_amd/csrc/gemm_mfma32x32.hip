// Pipelined MFMA kernel built on v_mfma_f32_32x32x16_{f16,bf16}, for
// fp16/bf16 problems whose rows are 16-byte aligned (K and N multiples of 8
// elements, A, B, C 16-byte aligned).
//
// Structure (the tiled loop of kernels-book chapter "Matrix Multiplication",
// section "Tiles"; one program per BM x BN output tile with an fp32
// accumulator that lives across the whole K walk):
//
//  * Tile order: 1-D grid, XCD-aware remap + grouped band order
//    (tile_of_block in gemm_internal.h).
//  * Staging: K is walked in steps of BK (32 or 64).  Global loads go to
//    registers first: the BM x BK A tile and BK x BN B tile of K-step it+L
//    (L = 128/BK register slots) are loaded while K-step it is multiplied,
//    and K-step it+1 is written from its slot into the other of two LDS
//    stages during the same step, so every load has L-1 K-steps to land.
//    Out-of-range 16-byte pieces (rows >= M, columns >= N, K positions >= K)
//    get an offset past the buffer's end, which the buffer unit returns as
//    zeros: the zero padding of the pages' tensor descriptors (chapter
//    "Matrix Multiplication", section "The real tiled loop").
//  * LDS layout: A tile [BM][BK] and B tile [BK][BN], both with their 16-byte
//    pieces XOR-swizzled by row so the MFMA operand reads hit every bank
//    once per cycle (the pages pad rows for the same purpose; chapter "Fast
//    matrix multiplication", section "Shared-memory bank conflicts").
//  * Math: 4 (or 8) wavefronts in a 2 x 2 (or 2 x 4) grid, each owning a block
//    of 32x32 MFMA tiles (v_mfma_f32_32x32x16_{f16,bf16}) whose fp32
//    accumulators stay in registers for the whole K walk.  A operands are
//    read with 16-byte LDS reads; B is stored N-contiguous (as it is in
//    memory) and read with the gfx950 LDS transpose read, which hands each
//    lane 4 consecutive K values of one column.  Operands of the next
//    16-wide K-slice are read while the current one multiplies; one barrier
//    per K-step, placed inside the step's last slice, publishes the next
//    stage.
//  * The MFMA is issued with its operands swapped (B fragment first), which
//    computes the transposed 32x32 block: each lane holds 4 consecutive
//    columns of one row.  The epilogue rounds the fp32 sums to the output
//    type (round to nearest even), stages the wavefront's block through LDS
//    and writes C with 16-byte stores covering whole row segments, skipping
//    rows >= M and columns >= N.
#include "gemm_internal.h"
#include "gemm_device.h"

namespace dgr {
namespace {

constexpr int kLeadK = 128;          // K elements of global loads kept in flight

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

// 16-byte piece swizzles (LDS: 64 banks of 4 bytes, 256 bytes per cycle).
// An A row of a BK-deep tile is 2*BK bytes = BK/8 pieces, so 128/BK rows
// share one 256-byte bank window; a 16-byte read by 16 lanes covers 16
// consecutive rows at one logical piece, and XOR-ing the piece with
// (row / (128/BK)) % (BK/8) puts each of those rows on its own 4 banks.  B
// rows hold BN/8 pieces; the B swizzle moves whole 64-byte groups so a
// transpose read (64 contiguous bytes of 4 rows per 32 lanes) hits 4
// different bank groups.
template <int BK> __device__ __forceinline__ int swz_a(int row) { return (row / (128 / BK)) % (BK / 8); }
template <int BN> __device__ __forceinline__ int swz_b(int k) { return ((k & 7) << 2) & (BN / 8 - 1); }

template <typename T, int BM, int BN, int BK, int WAVES_N>
__global__ __launch_bounds__(128 * WAVES_N, 1) void gemm_mfma32x32_kernel(
    const T* __restrict__ A, const T* __restrict__ B, T* __restrict__ C,
    int M, int N, int K, int group_m, Batch bt)
{
    typedef typename Op<T>::V8 V8;
    constexpr int NW = 2 * WAVES_N;           // wavefronts: 2 along M, WAVES_N along N
    constexpr int WM = BM / 2, WN = BN / WAVES_N;   // per-wavefront block
    constexpr int FM = WM / 32, FN = WN / 32; // 32x32 MFMA tiles per wavefront
    constexpr int NS = BK / 16;               // 16-deep K-slices per K-step
    constexpr int ROW_A = BK * 2;             // bytes in one A tile row
    constexpr int PA = BK / 8;                // 16-byte pieces per A row
    constexpr int A_BYTES = BM * ROW_A;
    constexpr int ROW_B = BN * 2;             // bytes in one B tile row
    constexpr int B_BYTES = BK * ROW_B;
    constexpr int STAGE = A_BYTES + B_BYTES;  // one LDS stage; two of them
    constexpr int A_LOADS = A_BYTES / 1024 / NW;  // 16-byte-per-lane loads per wavefront
    constexpr int B_LOADS = B_BYTES / 1024 / NW;
    constexpr int LOADS = A_LOADS + B_LOADS;      // per wavefront per K-step
    constexpr int LEAD = kLeadK / BK;             // K-steps of loads in flight = register slots
    constexpr int C_BYTES = WM * WN * 2;          // one wavefront's C block in LDS
    constexpr int SMEM = 2 * STAGE > NW * C_BYTES ? 2 * STAGE : NW * C_BYTES;
    static_assert(A_LOADS >= 1 && B_LOADS >= 1, "tile too small");
    static_assert(LEAD % 2 == 0, "the unroll assumes the slot period is a multiple of 2");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];

    const int tiles_m = cdiv_i(M, BM), tiles_n = cdiv_i(N, BN);
    int b, tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, bt.count, group_m, true, b, tm, tn);
    A += b * bt.sa;
    B += b * bt.sb;
    C += b * bt.sc;
    const int m0 = tm * BM, n0 = tn * BN;

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform per wavefront
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (unsigned)M * (unsigned)K * 2u);

    // ---- per-lane load geometry (fixed across K-steps)
    // A: load j of this wavefront fills 1 KB = 1024/ROW_A consecutive tile
    //    rows; lane -> row +lane/PA, physical piece lane%PA, logical piece
    //    p ^ swz.  voffset = (row*K + piece*8)*2 (kOOB for rows >= M); the
    //    K-step's k0*2 goes in the scalar offset.  A piece whose K range
    //    starts at or past K is switched to kOOB per K-step.
    constexpr int A_ROWS_PER_LOAD = 1024 / ROW_A;
    unsigned a_voff[A_LOADS];
    int a_kp[A_LOADS];
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
        const int row = A_ROWS_PER_LOAD * (wave * A_LOADS + j) + lane / PA;
        const int piece = (lane % PA) ^ swz_a<BK>(row);
        a_voff[j] = (m0 + row) < M ? ((unsigned)(m0 + row) * (unsigned)K + (unsigned)piece * 8u) * 2u : kOOB;
        a_kp[j] = piece * 8;
    }
    // B: 1 KB covers 1024/ROW_B rows of the B tile.  voffset = (krow*N +
    //    col)*2 (kOOB for columns >= N) relative to a buffer that starts at
    //    row k0 and ends at row min(K, k0 + BK), so rows >= K read zero.
    constexpr int B_ROWS_PER_LOAD = 1024 / ROW_B;
    unsigned b_voff[B_LOADS];
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
        const int byte = lane * 16;
        const int krow = B_ROWS_PER_LOAD * (wave * B_LOADS + j) + byte / ROW_B;
        const int piece = ((byte % ROW_B) / 16) ^ swz_b<BN>(krow);
        const int col = n0 + piece * 8;
        b_voff[j] = col < N ? ((unsigned)krow * (unsigned)N + (unsigned)col) * 2u : kOOB;
    }

    // Global loads [j0, j1) of the K-step starting at k0 into register slot
    // `slot` (16 bytes per lane per load; loads 0..A_LOADS-1 are A's, the
    // rest B's).  Loads past the end of K read zeros, so the last K-step may
    // be ragged or entirely empty.
    u32x4 stg[LEAD][LOADS];
    auto load_regs = [&](int slot, int k0_in, int j0, int j1) {
        const int k0 = __builtin_amdgcn_readfirstlane(k0_in);   // uniform: keep it scalar
        const int krem = K - k0;
#pragma unroll
        for (int j = 0; j < A_LOADS; ++j) {
            if (j < j0 || j >= j1) continue;
            const unsigned off = a_kp[j] < krem ? a_voff[j] : kOOB;
            stg[slot][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, off, k0 * 2, 0));
        }
        if (j1 <= A_LOADS) return;
        const int rows = __builtin_amdgcn_readfirstlane(krem < 0 ? 0 : (krem > BK ? BK : krem));
        const __amdgpu_buffer_rsrc_t rbk =
            make_rsrc(B + (size_t)(k0 < K ? k0 : 0) * N, (unsigned)rows * (unsigned)N * 2u);
#pragma unroll
        for (int j = 0; j < B_LOADS; ++j) {
            if (A_LOADS + j < j0 || A_LOADS + j >= j1) continue;
            // (copied to a local: clang's host pass drops the kernel stub when a
            // captured array element is passed straight to this builtin)
            const unsigned off = b_voff[j];
            stg[slot][A_LOADS + j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rbk, off, 0, 0));
        }
    };
    // Write loads [j0, j1) of register slot `slot` into LDS stage `stage`:
    // load j of this wavefront covers 1 KB of the stage, lane l its bytes
    // 16l..16l+15, so every 16-byte write of a wavefront is one contiguous,
    // conflict-free KB.
    auto store_stage = [&](int stage, int slot, int j0, int j1) {
        lds_byte* base = (lds_byte*)smem + stage * STAGE + lane * 16;
#pragma unroll
        for (int j = 0; j < A_LOADS; ++j)
            if (j >= j0 && j < j1)
                *(u32x4 __attribute__((address_space(3)))*)(base + (wave * A_LOADS + j) * 1024) = stg[slot][j];
#pragma unroll
        for (int j = 0; j < B_LOADS; ++j)
            if (A_LOADS + j >= j0 && A_LOADS + j < j1)
                *(u32x4 __attribute__((address_space(3)))*)(base + A_BYTES + (wave * B_LOADS + j) * 1024) =
                    stg[slot][A_LOADS + j];
    };

    // ---- per-lane LDS read addresses, one base register per stage; the
    // tile index and the K-slice are compile-time constants in the
    // instruction's 16-bit offset.
    // A fragment (tile bi, K-slice s): row wm*WM + 32*bi + lane%32, logical
    // piece 2s + lane/32; the row swizzle only depends on lane%32.
    const int a_sw = swz_a<BK>(lane & 31);
    int a_addr[2][NS];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int sl = 0; sl < NS; ++sl)
            a_addr[st][sl] = st * STAGE + (wm * WM + (lane & 31)) * ROW_A + (((2 * sl + (lane >> 5)) ^ a_sw) * 16);
    // B fragment via transpose reads: within each 16-lane group, lane 4r+q
    // points at row r, columns 4q..4q+3 of a 4 x 16 block; the read returns
    // to lane i the 4 rows of column i.  Lanes 0-31 cover K rows 0..7 of the
    // slice, lanes 32-63 rows 8..15; lanes 16-31 / 48-63 the upper 16 columns.
    // The B swizzle depends on k%8, which does not change with the slice.
    const int g16 = lane & 15;
    const int b_kr = 8 * (lane >> 5) + (g16 >> 2);
    const int b_cn = 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
    int b_addr[2][FN][2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int bj = 0; bj < FN; ++bj)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int k = 4 * hh + b_kr;
                const int n = wn * WN + 32 * bj + b_cn;
                const int piece = (n >> 3) ^ swz_b<BN>(k);
                b_addr[st][bj][hh] = st * STAGE + A_BYTES + k * ROW_B + piece * 16 + (n & 7) * 2;
            }

    const lds_byte* lds0 = (const lds_byte*)smem;
    // Fragments of K-slice sl of stage st.
    auto read_frags = [&](int st, int sl, V8* af, V8* bf) {
#pragma unroll
        for (int bi = 0; bi < FM; ++bi)
            af[bi] = *(const V8*)(lds0 + a_addr[st][sl] + bi * 32 * ROW_A);
#pragma unroll
        for (int bj = 0; bj < FN; ++bj) {
            s16x4 h[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 __attribute__((address_space(3)))*)(lds0 + b_addr[st][bj][hh] + 16 * sl * ROW_B));
            const s16x8 v = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
            bf[bj] = __builtin_bit_cast(V8, v);
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // MFMAs [lo, hi) of one K-slice, tile index = bi*FN + bj.
    auto mfmas = [&](const V8* af, const V8* bf, int lo, int hi) {
#pragma unroll
        for (int x = lo; x < hi; ++x)
            acc[x / FN][x % FN] = Op<T>::mfma(bf[x % FN], af[x / FN], acc[x / FN][x % FN]);
    };

    constexpr int NT = FM * FN;                  // MFMAs per wavefront per K-slice
    constexpr int NR = FM + 2 * FN;              // LDS reads per wavefront per K-slice
    // Loads and LDS writes of a K-step are spread over its first NS-1
    // slices (all of them go in slice 0 when NS == 2).
    constexpr int SPREAD = NS > 2 ? NS - 1 : 1;
    constexpr int PER = (LOADS + SPREAD - 1) / SPREAD;
    // K-steps, rounded up to the LEAD-step unroll (register slots cycle with
    // period LEAD and LDS stages with period 2): the extra steps multiply the
    // zeros their loads brought in.
    const int nk = (cdiv_i(K, BK) + LEAD - 1) / LEAD * LEAD;

    // Software pipeline.  K-step j's data travels global -> register slot
    // j%LEAD (loaded during K-step j-LEAD) -> LDS stage j%2 (written during
    // K-step j-1) -> operand registers.
    //  slices 0..NS-2 of K-step it: read the next slice's operands of stage
    //    it%2; write K-step it+1 (loaded LEAD-1 steps ago) from its slot
    //    into stage (it+1)%2, which every wavefront finished reading before
    //    the barrier of K-step it-1; load K-step it+LEAD into slot it%LEAD
    //    (its previous content, K-step it, went to LDS one step ago);
    //    multiply the slice.
    //  last slice: multiply half of it; pass the barrier (everyone's K-step
    //    it+1 now in LDS); read slice-0 operands of stage (it+1)%2; multiply
    //    the other half.
    V8 fa[2][FM], fb[2][FN];
#pragma unroll
    for (int q = 0; q < LEAD; ++q) load_regs(q, q * BK, 0, LOADS);
    store_stage(0, 0, 0, LOADS);
    __syncthreads();
    read_frags(0, 0, fa[0], fb[0]);

    // q = it % LEAD is always passed as a literal, so after inlining every
    // register slot and LDS address is fixed at compile time.
    auto kstep = [&](const int q, int it) {
        const int ST = q & 1;
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
            const int cur = sl & 1, nxt = cur ^ 1;
            if (sl < NS - 1) {
                read_frags(ST, sl + 1, fa[nxt], fb[nxt]);
                const int j0 = sl * PER, j1 = (sl + 1) * PER < LOADS ? (sl + 1) * PER : LOADS;
                if (j0 < j1) {
                    store_stage(ST ^ 1, (q + 1) % LEAD, j0, j1);
                    load_regs(q, (it + LEAD) * BK, j0, j1);
                }
                mfmas(fa[cur], fb[cur], 0, NT);
                // one MFMA, then an LDS read, an LDS write or a global load,
                // until they run out
                constexpr int NJ = PER;
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    if (i % 2 == 0 && i / 2 < NJ) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                    if (i % 2 == 1 && i / 2 < NJ) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            } else {
                mfmas(fa[cur], fb[cur], 0, NT / 2);
                __builtin_amdgcn_sched_barrier(0);
                __syncthreads();               // everyone's K-step it+1 in LDS
                __builtin_amdgcn_sched_barrier(0);
                read_frags(ST ^ 1, 0, fa[0], fb[0]);
                mfmas(fa[cur], fb[cur], NT / 2, NT);
#pragma unroll
                for (int i = 0; i < NT / 2; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, (NR + NT / 2 - 1) / (NT / 2), 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    for (int it = 0; it < nk; it += LEAD) {
#pragma unroll
        for (int q = 0; q < LEAD; ++q) kstep(q, it + q);
    }

    // ---- epilogue
    // All loads (including the zero-fills past K) have landed and every
    // wavefront is done with the stages before they are reused for C.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    store_c_block_32x32<T, WM, WN>(acc, (lds_byte*)smem + wave * C_BYTES, lane, m0 + wm * WM, n0 + wn * WN, M, N, C);
}

template <typename T>
hipError_t launch_t(const Config& cfg, const LaunchArgs& a)
{
    const int tiles = cdiv_i(a.M, cfg.bm) * cdiv_i(a.N, cfg.bn);
    const dim3 grid(tiles * a.batch.count), block(cfg.threads);
    const T* A = static_cast<const T*>(a.A);
    const T* B = static_cast<const T*>(a.B);
    T* C = static_cast<T*>(a.C);
#define DGR_LAUNCH(BM_, BN_, BK_, WN_)                                                               \
    if (cfg.bm == BM_ && cfg.bn == BN_ && cfg.bk == BK_ && cfg.threads == 128 * WN_) {               \
        hipLaunchKernelGGL((gemm_mfma32x32_kernel<T, BM_, BN_, BK_, WN_>), grid, block, 0, a.stream, A, B, C, \
                           a.M, a.N, a.K, cfg.group_m, a.batch);                                            \
        return hipGetLastError();                                                                  \
    }
    DGR_LAUNCH(256, 256, 32, 2)
    DGR_LAUNCH(256, 256, 64, 2)
    DGR_LAUNCH(256, 256, 32, 4)
    DGR_LAUNCH(256, 128, 32, 2)
    DGR_LAUNCH(128, 128, 32, 2)
#undef DGR_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_mfma32x32(const Config& cfg, const LaunchArgs& a)
{
    if (a.dtype == kF16) return launch_t<_Float16>(cfg, a);
    if (a.dtype == kBF16) return launch_t<__bf16>(cfg, a);
    return hipErrorInvalidValue;
}

}  // namespace dgr
