// MFMA kernel built on v_mfma_f32_16x16x32_{f16,bf16}, for fp16/bf16
// problems whose rows are 16-byte aligned (K and N multiples of 8 elements,
// A, B, C 16-byte aligned).
//
// Same tiled loop as the 32x32 kernel (kernels-book chapter "Matrix
// Multiplication", section "Tiles": one program per BM x BN output tile, an
// fp32 accumulator per output element that lives across the whole K walk),
// with these differences:
//
//  * Math: 4 wavefronts in a 2 x 2 grid, each owning (BM/2) x (BN/2) outputs
//    as 16x16 MFMA tiles (BM x BN = 256 x 256, 192 x 256, 256 x 128,
//    128 x 128 or 64 x 128).  Per unit of work the 16x16x32 instruction moves
//    half the accumulator data of the 32x32x16 one; under MI355X's power
//    limit this runs at a higher clock for the same issue rate.
//  * The MFMAs are written as inline assembly with the accumulator operand
//    tied to the destination ("+a"): the compiler's own selection for this
//    instruction rotates accumulators through copies every K-step.  Being
//    volatile, the statements also fix the order of every MFMA against the
//    LDS and global-memory instructions around them, so the interleave below
//    is exactly the issue order.  The compiler does not see the MFMA
//    latency through inline assembly; the kernel covers the two places where
//    it matters: the first K-step writes the accumulators without reading
//    them (source C = 0, no zero-fill before it) and the epilogue waits out
//    the last MFMAs before it reads accumulators.
//  * Staging: K is walked in steps of 32 (one MFMA K-slice).  A goes through
//    registers (LEAD register slots; K-step it+LEAD is loaded during K-step
//    it and written to LDS during K-step it+LEAD-1, into one of two A
//    stages).  B goes global -> LDS directly (buffer loads with the LDS
//    destination) into a ring of SB stages, K-step it+SB-1 during K-step
//    it.  Out-of-range 16-byte pieces read zeros, as in the 32x32 kernel (the
//    zero padding of chapter "Matrix Multiplication", section "The real
//    tiled loop").
//  * ADMA variant: A also goes global -> LDS directly, each lane fetching the
//    piece the swizzled layout puts at its slot, into the ring stage of B's
//    K-step (one LDS object per stage holds A and B); A and B of K-step
//    it+SB are issued after K-step it's barrier.  No register staging and no
//    A writes; it is the faster choice wherever the operands stay in the
//    Infinity Cache.
//  * LDS layout: A [BM][32] with 16-byte pieces XOR-swizzled by (row/2)%4
//    (the layout that measured free of bank conflicts for this read); B
//    [32][BN] with 16-byte pieces XOR-swizzled by an even
//    value taken from bits 0, 1 and 3 of the row, so the 8 rows that one
//    half-wavefront's transpose read touches (k = r, r+8 for r in a group of
//    4) cover all 64 banks (chapter "Fast matrix multiplication", section
//    "Shared-memory bank conflicts", pads rows for the same purpose).
//  * One barrier per K-step, half way through its MFMAs: it
//    publishes K-step it+1 (A written by every wavefront, B landed), after
//    which the operands of K-step it+1 are read into the second register set
//    while the rest of K-step it multiplies.
//  * The MFMA takes the B fragment first, which computes the transposed
//    16x16 block: lane l holds row l%16 of the tile, columns 4*(l/16)..+3.
//    The epilogue rounds to the output type (round to nearest even), stages
//    the wavefront's block through LDS and writes whole row segments with
//    16-byte stores, skipping rows >= M and columns >= N.
//  * Split K (SPLIT): for products with too few tiles to fill the CUs, the
//    grid holds `splits` workgroups per tile; split s walks K-steps
//    s*Q .. (s+1)*Q-1 (Q = ceil(K-steps / splits)) and writes its fp32 sums,
//    unrounded, to its own M x N slice of a workspace; a second kernel adds
//    the slices in split order and rounds once (the blocked K-loop of lesson
//    "Matrix multiplication", section "Tiles are small rectangles of work":
//    the per-block contributions are summed, here by different workgroups).
#include "gemm_internal.h"
#include "gemm_device.h"

namespace dgr {
namespace {

// The MFMAs below are inline assembly, so the compiler's hazard handling does
// not see them.  The schedule relies on these wait-state rules of the CDNA
// ISA for matrix (XDL) instructions, which the generated-code tests check:
//  (1) a VALU or memory instruction may read an accumulator only P + 3 wait
//      states after the last MFMA writing it (P passes, at most 16 here):
//      the epilogue's s_nop waits and the order of the last K-step give 27
//      or more;
//  (2) sources A and B are written by LDS reads, whose data the compiler's
//      own s_waitcnt before each MFMA covers (it sees the asm's register
//      operands), into the register set the MFMAs in flight do not read; no
//      VALU result reaches an MFMA operand within 5 wait states;
//  (3) source C is either 0 (the first K-slice) or exactly the destination,
//      of the same opcode, which the hardware orders by itself.
template <typename T> struct Mfma16x16;
template <> struct Mfma16x16<_Float16> {
    // c += b-fragment x a-fragment (16x16x32)
    static __device__ __forceinline__ void acc(f32x4& c, const u32x4& b, const u32x4& a)
    {
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
    }
    // c = b-fragment x a-fragment (source C is the constant 0)
    static __device__ __forceinline__ void first(f32x4& c, const u32x4& b, const u32x4& a)
    {
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=a"(c) : "v"(b), "v"(a));
    }
};
template <> struct Mfma16x16<__bf16> {
    static __device__ __forceinline__ void acc(f32x4& c, const u32x4& b, const u32x4& a)
    {
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
    }
    static __device__ __forceinline__ void first(f32x4& c, const u32x4& b, const u32x4& a)
    {
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(c) : "v"(b), "v"(a));
    }
};

// A rows are BK*2 bytes (4 or 8 pieces of 16 bytes).  The operand read has
// 16-lane group g read logical piece 4*sl + g of 16 consecutive rows.
// XOR-ing the piece with (row/2) % (BK/8) makes that read run without LDS
// bank conflicts on gfx950 (measured with the bank-conflict counter over
// candidate layouts); with 64-byte rows, the (row/4)%4 swizzle, which spreads
// each group's 16 reads over all 64 banks, still conflicts there about 4
// cycles per instruction.
template <int BK> __device__ __forceinline__ int swz_a(int row) { return (row >> 1) & (BK / 8 - 1); }
// B rows are BN*2 bytes (a multiple of 256): every row starts at bank 0.
template <int BN> __device__ __forceinline__ int swz_b(int k)
{
    return (2 * ((k & 3) | ((k >> 1) & 4))) & (BN / 8 - 1);
}

template <typename T, int BM, int BN, int BK, bool SPLIT, bool ADMA = false>
__global__ __launch_bounds__(256, 1) void gemm_mfma16x16_kernel(
    const T* A, const T* B, T* C,
    int M, int N, int K, int group_m, int xcd_remap, Batch bt, float* ws, int splits, unsigned long long* clk)
{
    clock_sample(clk, 0);
    constexpr int NW = 4;                        // wavefronts, 2 x 2
    constexpr int WM = BM / 2, WN = BN / 2;      // per-wavefront block
    constexpr int FM = WM / 16, FN = WN / 16;    // 16x16 tiles per wavefront
    constexpr int NT = FM * FN;                  // MFMAs per wavefront per 32-deep K-slice
    constexpr int NS = BK / 32;                  // K-slices per K-step
    constexpr int XS = NS * NT;                  // MFMAs per wavefront per K-step
    constexpr int LEAD = 128 / BK;               // A register slots (K-steps loaded ahead)
    constexpr int SB = BK == 32 ? 4 : 2;         // B stages (K-steps loaded ahead)
    constexpr int ROW_A = BK * 2;
    constexpr int PA = BK / 8;                   // 16-byte pieces per A row
    constexpr int A_BYTES = BM * ROW_A;
    constexpr int ROW_B = BN * 2;
    constexpr int B_BYTES = BK * ROW_B;
    constexpr int A_LOADS = A_BYTES / 1024 / NW; // 16-byte-per-lane loads per wavefront
    constexpr int B_LOADS = B_BYTES / 1024 / NW;
    constexpr int LOADS = A_LOADS + B_LOADS;     // vector-memory instructions per K-step
    constexpr int NR = FM + FN;                  // operand fragments per K-slice
    constexpr int BAR = XS - NT / 2;             // MFMAs of a K-step before its barrier
    static_assert(BK == 32 || BK == 64, "K-step");
    static_assert(A_LOADS >= 1 && B_LOADS >= 1, "tile too small");
    static_assert(ROW_B % 256 == 0, "B rows must be whole bank windows");
    static_assert(LEAD % 2 == 0 && LEAD % SB == 0, "slot and stage periods must divide the unroll");
    // Every stage is an LDS object of its own: the compiler tracks the
    // direct-to-LDS loads per object, so reading one B stage does not wait
    // for the loads still landing in the others.
    // ADMA: A also goes global -> LDS directly, into the same ring as B; each
    // ring stage is one LDS object holding A (first) and B of one K-step.
    static_assert(!ADMA || (SB == 4 && LEAD == 4), "direct A loads: 32-deep K-steps");
    constexpr int SA_BYTES = ADMA ? 1 : A_BYTES;
    constexpr int SB_BYTES = ADMA ? A_BYTES + B_BYTES : B_BYTES;
    __shared__ __attribute__((aligned(1024))) unsigned char sa0[SA_BYTES], sa1[SA_BYTES];
    __shared__ __attribute__((aligned(1024))) unsigned char sb0[SB_BYTES], sb1[SB_BYTES];
    __shared__ __attribute__((aligned(1024))) unsigned char sb2[SB > 2 ? SB_BYTES : 1], sb3[SB > 2 ? SB_BYTES : 1];
    auto b_obj = [&](int st) __attribute__((always_inline)) { return (lds_byte*)(st == 0 ? sb0 : st == 1 ? sb1 : st == 2 ? sb2 : sb3); };
    auto a_stage = [&](int st) __attribute__((always_inline)) {
        if constexpr (ADMA) return b_obj(st);
        else return (lds_byte*)(st == 0 ? sa0 : sa1);
    };
    auto b_stage = [&](int st) __attribute__((always_inline)) { return b_obj(st) + (ADMA ? A_BYTES : 0); };

    const int tiles_m = cdiv_i(M, BM), tiles_n = cdiv_i(N, BN);
    int b, tm, tn;
    // with split K the batch axis of the tile order is the split (one product)
    tile_of_block(blockIdx.x, tiles_m, tiles_n, SPLIT ? splits : bt.count, group_m, xcd_remap != 0, b, tm, tn);
    if constexpr (!SPLIT) {
        A += b * bt.sa;
        B += b * bt.sb;
        C += b * bt.sc;
    }
    const int m0 = tm * BM, n0 = tn * BN;
    // K range of this workgroup: [kb, ke)
    int kb = 0, ke = K;
    if constexpr (SPLIT) {
        const int q = cdiv_i(cdiv_i(K, BK), splits) * BK;
        kb = b * q;
        ke = kb + q < K ? kb + q : K;
    }

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (unsigned)M * (unsigned)K * 2u);

    // ---- global load geometry
    // A: load j of this wavefront fills 1 KB = 1024/ROW_A tile rows; lane ->
    //    row +lane/PA, physical piece lane%PA holding logical piece
    //    p ^ swz_a(row).  voffset = (row*K + piece*8)*2 (kOOB for rows >= M);
    //    the K-step's k0*2 goes in the scalar offset.  Pieces starting at or
    //    past K read zeros (checked per K-step).
    unsigned a_voff[A_LOADS];
    int a_kp[A_LOADS];
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
        const int row = (1024 / ROW_A) * (wave * A_LOADS + j) + lane / PA;
        const int piece = (lane % PA) ^ swz_a<BK>(row);
        a_voff[j] = (m0 + row) < M ? ((unsigned)(m0 + row) * (unsigned)K + (unsigned)piece * 8u) * 2u : kOOB;
        a_kp[j] = piece * 8;
    }
    // B: load j fills 1 KB = 1024/ROW_B tile rows; lane -> byte 16*lane of
    //    it, physical piece (16*lane % ROW_B)/16 holding logical piece
    //    p ^ swz_b(k).  voffset = (k*N + col)*2 (kOOB for columns >= N)
    //    relative to a buffer that starts at row k0 and ends at row
    //    min(K, k0 + BK), so rows >= K read zero.
    unsigned b_voff[B_LOADS];
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
        const int byte = 1024 * (wave * B_LOADS + j) + lane * 16;
        const int k = byte / ROW_B;
        const int piece = ((byte % ROW_B) / 16) ^ swz_b<BN>(k);
        const int col = n0 + piece * 8;
        b_voff[j] = col < N ? ((unsigned)k * (unsigned)N + (unsigned)col) * 2u : kOOB;
    }

    u32x4 stg[LEAD][A_LOADS];
    // A rows of the K-step at k0 -> register slot `slot`, load j.
    auto load_a = [&](int slot, int k0_in, int j) __attribute__((always_inline)) {
        const int k0 = __builtin_amdgcn_readfirstlane(kb + k0_in);
        const unsigned off = a_kp[j] < ke - k0 ? a_voff[j] : kOOB;
        stg[slot][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, off, k0 * 2, 0));
    };
    // ADMA: A rows of the K-step at k0, load j -> A part of ring stage `st`
    // (direct to LDS, at the place store_a gives the same piece).
    auto load_a_lds = [&](int st, int k0_in, int j) __attribute__((always_inline)) {
        const int k0 = __builtin_amdgcn_readfirstlane(kb + k0_in);
        const unsigned off = a_kp[j] < ke - k0 ? a_voff[j] : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (void __attribute__((address_space(3)))*)(a_stage(st) + (wave * A_LOADS + j) * 1024), 16,
            off, k0 * 2, 0, 0);
    };
    // Register slot `slot`, load j -> A stage `st`.
    auto store_a = [&](int st, int slot, int j) __attribute__((always_inline)) {
        lds_byte* p = a_stage(st) + (wave * A_LOADS + j) * 1024 + lane * 16;
        *(u32x4 __attribute__((address_space(3)))*)p = stg[slot][j];
    };
    // B rows of the K-step at k0, load j -> B stage `st` (direct to LDS).
    auto load_b = [&](int st, int k0_in, int j) __attribute__((always_inline)) {
        const int k0 = __builtin_amdgcn_readfirstlane(kb + k0_in);
        const int krem = ke - k0;
        const int rows = __builtin_amdgcn_readfirstlane(krem < 0 ? 0 : (krem > BK ? BK : krem));
        const __amdgpu_buffer_rsrc_t rbk =
            make_rsrc(B + (size_t)(k0 < ke ? k0 : 0) * N, (unsigned)rows * (unsigned)N * 2u);
        // (copied to a local: clang's host pass drops the kernel stub when a
        // captured array element is passed straight to a buffer builtin)
        const unsigned off = b_voff[j];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rbk, (void __attribute__((address_space(3)))*)(b_stage(st) + (wave * B_LOADS + j) * 1024), 16,
            off, 0, 0, 0);
    };

    // ---- operand read addresses (within a stage); the stage, the tile, the
    // K-slice's B rows and the half of a transpose read are constants.
    // A fragment (K-slice sl, tile bi): row wm*WM + 16*bi + lane%16, logical
    // piece 4*sl + lane/16 (K 32*sl + 8*(lane/16) .. +7); the swizzle depends
    // only on lane%16.
    int a_rd[NS];
#pragma unroll
    for (int sl = 0; sl < NS; ++sl)
        a_rd[sl] = (wm * WM + (lane & 15)) * ROW_A + (((4 * sl + (lane >> 4)) ^ swz_a<BK>(lane & 15)) * 16);
    // B fragment (tile bj) via two transpose reads: within each 16-lane group
    // g = lane/16, lane 4r+q points at K row 8g + r (+4 for the second read,
    // +32 per K-slice), columns 4q..4q+3 of the tile; lane i of the group
    // receives column i.  The swizzle is the same for rows k, k+4 and k+32.
    int b_rd[FN];
#pragma unroll
    for (int bj = 0; bj < FN; ++bj) {
        const int g16 = lane & 15;
        const int k = 8 * (lane >> 4) + (g16 >> 2);
        const int n = wn * WN + 16 * bj + 4 * (g16 & 3);
        const int piece = (n >> 3) ^ swz_b<BN>(k);
        b_rd[bj] = k * ROW_B + piece * 16 + (n & 7) * 2;
    }
    auto read_a = [&](int st, int sl, int bi) __attribute__((always_inline)) -> u32x4 {
        return *(const u32x4 __attribute__((address_space(3)))*)(a_stage(st) + a_rd[sl] + bi * 16 * ROW_A);
    };
    auto read_b = [&](int st, int sl, int bj) __attribute__((always_inline)) -> u32x4 {
        const lds_byte* p = b_stage(st) + b_rd[bj] + sl * 32 * ROW_B;
        const s16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)p);
        const s16x4 h1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p + 4 * ROW_B));
        return __builtin_bit_cast(u32x4, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    f32x4 acc[FM][FN];
    u32x4 fa[2][FM], fb[2][FN];   // two operand register sets, alternating by K-slice
    // Fragment o of a K-slice (B tiles first, then A tiles) -> register set.
    auto read_frag = [&](int set, int sta, int stb, int sl, int o) __attribute__((always_inline)) {
        if (o < FN)
            fb[set][o] = read_b(stb, sl, o);
        else
            fa[set][o - FN] = read_a(sta, sl, o - FN);
    };

    // ---- software pipeline.  Vector-memory instructions are issued in
    // groups, one per K-step: group it = [A loads of K-step it+LEAD (before
    // the step's barrier), B loads of K-step it+SB (after it)].  The
    // prologue issues groups -max(LEAD, SB) .. -1 (the parts that exist), in
    // the same order within a group (the empty statements with a memory
    // clobber keep the compiler from interleaving the parts).  When K-step
    // it waits for its B loads of K-step it+1 (the end of group it+1-SB),
    // groups it+2-SB .. it-1 and the A loads of group it were issued after
    // them: at most (SB-2)*LOADS + A_LOADS of this wavefront's loads may
    // still be in flight.
#pragma unroll
    for (int g = -LEAD; g < 0; ++g) {
        if (g + LEAD >= 0) {
#pragma unroll
            for (int j = 0; j < A_LOADS; ++j) {
                if constexpr (ADMA) load_a_lds(g + LEAD, (g + LEAD) * BK, j);
                else load_a(g + LEAD, (g + LEAD) * BK, j);
            }
        }
        asm volatile("" ::: "memory");
        if (g + SB >= 0)
#pragma unroll
            for (int j = 0; j < B_LOADS; ++j) load_b(g + SB, (g + SB) * BK, j);
        asm volatile("" ::: "memory");
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((SB - 1) * LOADS));   // group -SB (B of K-step 0) landed
    if constexpr (!ADMA) {
#pragma unroll
        for (int j = 0; j < A_LOADS; ++j) store_a(0, 0, j);
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int o = 0; o < NR; ++o) read_frag(0, 0, 0, 0, o);

    // One K-step; q = it % LEAD is a literal, so every slot, stage and
    // register set below is fixed at compile time.  K-slice sl of K-step it
    // uses register set (q*NS + sl) % 2.
    //   MFMAs 0 .. BAR-1, interleaved with: the operand reads of K-slices
    //     1 .. NS-1 of this K-step (each during the slice before it); A
    //     writes of K-step it+1 (slot (q+1)%LEAD -> A stage (q+1)%2); A loads
    //     of K-step it+LEAD (-> slot q, which K-step it left one step ago).
    //   wait for this wavefront's B loads of K-step it+1; barrier.
    //   MFMAs BAR .. XS-1, interleaved with: B loads of K-step it+SB (-> B
    //     stage q%SB: every wavefront finished reading K-step it from it
    //     before this barrier), then the operand reads of K-slice 0 of K-step
    //     it+1.
    // Issuing all of a step's loads in one burst stalls the in-order MFMA
    // stream (measured); they are spread over the step.
    // n operations spread evenly over `span` MFMAs: the ones issued after
    // MFMA number pos are op_lo(pos) .. op_lo(pos+1)-1.
    auto op_lo = [](int pos, int n, int span) __attribute__((always_inline)) { return (pos * n + span - 1) / span; };

    // K-slice sl of K-step it (q = it % LEAD): its MFMAs before the barrier
    // (x < BAR, counting over the whole K-step), then those after it.  (Two
    // loops rather than one with a branch: the compiler only unrolls loops
    // below a size limit, and everything here must unroll.)
    // ADMA: group it (A and B of K-step it+SB, into stage it % SB, which
    // every wavefront finished reading before K-step it's barrier) is issued
    // in two parts: loads 0 .. P-1 after K-step it's barrier, between the
    // operand reads, and loads P .. LOADS-1 before K-step it+1's barrier,
    // spread over its first MFMAs.  All the wavefronts issuing a whole group
    // right after one barrier queue 4 * LOADS KB at once on the CU's load
    // path, which stalls their in-order MFMA streams (measured); spread over
    // the K-step they keep one load per few MFMAs in flight instead.
    constexpr int P_ADMA = LOADS / 2;
    auto load_group = [&](int st, int k0_in, int idx) __attribute__((always_inline)) {
        if (idx < A_LOADS)
            load_a_lds(st, k0_in, idx);
        else
            load_b(st, k0_in, idx - A_LOADS);
    };
    auto kslice = [&](const int q, int it, const int sl, const bool first) __attribute__((always_inline)) {
        // ADMA: A shares B's ring (stage it % SB)
        const int sta = ADMA ? q % SB : q & 1, stb = q % SB, set = (q * NS + sl) & 1;
        const int sta_next = ADMA ? (q + 1) % SB : sta ^ 1;
        // ops before the barrier: A writes and A loads (A through
        // registers), or the second part of group it-1 (ADMA)
        constexpr int NOPS1 = ADMA ? LOADS - P_ADMA : 2 * A_LOADS;
        constexpr int LD2 = ADMA ? P_ADMA : B_LOADS;   // loads after the barrier
        constexpr int NOPS2 = LD2 + NR;
        auto mfma = [&](int xx) __attribute__((always_inline)) {
            if (first && sl == 0)
                Mfma16x16<T>::first(acc[xx / FN][xx % FN], fb[set][xx % FN], fa[set][xx / FN]);
            else
                Mfma16x16<T>::acc(acc[xx / FN][xx % FN], fb[set][xx % FN], fa[set][xx / FN]);
        };
        const int lo = sl * NT, hi = lo + NT;
#pragma unroll
        for (int x = lo; x < (hi < BAR ? hi : BAR); ++x) {
            const int xx = x - lo;
            mfma(xx);
            if (sl + 1 < NS) {
#pragma unroll
                for (int o = op_lo(xx, NR, NT); o < op_lo(xx + 1, NR, NT); ++o)
                    read_frag(set ^ 1, sta, stb, sl + 1, o);
            }
            if constexpr (ADMA) {
                // the second part of group it-1 (none in the first K-step: the
                // prologue issued group -1 whole)
                if (!first) {
#pragma unroll
                    for (int o = op_lo(x, NOPS1, BAR); o < op_lo(x + 1, NOPS1, BAR); ++o)
                        load_group((q + SB - 1) % SB, (it - 1 + SB) * BK, P_ADMA + o);
                }
            } else {
#pragma unroll
                for (int o = op_lo(x, NOPS1, BAR); o < op_lo(x + 1, NOPS1, BAR); ++o) {
                    if (o < A_LOADS)
                        store_a(sta ^ 1, (q + 1) % LEAD, o);
                    else
                        load_a(q, (it + LEAD) * BK, o - A_LOADS);
                }
            }
        }
        if (lo < BAR && BAR <= hi) {
            // The count below assumes every load of this K-step before the
            // barrier was issued above it: keep the compiler from sinking
            // any (it may otherwise move loads whose results are needed only
            // steps later).
            asm volatile("" ::: "memory");
            // ADMA: groups it-2 and it-1 were issued after K-step it+1's
            __builtin_amdgcn_s_waitcnt(waitcnt_vm((SB - 2) * LOADS + (ADMA ? 0 : A_LOADS)));
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // this wavefront's A writes (and reads) done
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
#pragma unroll
        for (int x = (lo > BAR ? lo : BAR); x < hi; ++x) {
            mfma(x - lo);
#pragma unroll
            for (int o = op_lo(x - BAR, NOPS2, XS - BAR); o < op_lo(x + 1 - BAR, NOPS2, XS - BAR); ++o) {
                if constexpr (ADMA) {
                    // loads 0 .. P-1 of group it at evenly spaced ops
                    // (o = 0, NOPS2/P, ...), the operand reads in between
                    const int nld = (o * P_ADMA) / NOPS2 + 1;   // loads at ops 0 .. o
                    if (o == 0 || (o * P_ADMA) / NOPS2 != ((o - 1) * P_ADMA) / NOPS2)
                        load_group(stb, (it + SB) * BK, nld - 1);
                    else
                        read_frag(((q + 1) * NS) & 1, sta_next, (q + 1) % SB, 0, o - nld);
                } else if (o < LD2)
                    load_b(stb, (it + SB) * BK, o);
                else
                    read_frag(((q + 1) * NS) & 1, sta_next, (q + 1) % SB, 0, o - LD2);
            }
        }
    };
    auto kstep = [&](const int q, int it, const bool first) __attribute__((always_inline)) {
        kslice(q, it, 0, first);
        if constexpr (NS > 1) kslice(q, it, 1, false);
    };

    // K-steps, rounded up to the LEAD-step unroll and at least one round:
    // the extra steps multiply the zeros their loads brought in.
    const int nk = cdiv_i(cdiv_i(ke - kb, BK), LEAD) * LEAD;
    kstep(0, 0, true);
#pragma unroll
    for (int q = 1; q < LEAD; ++q) kstep(q, q, false);
    for (int it = LEAD; it < nk; it += LEAD) {
#pragma unroll
        for (int q = 0; q < LEAD; ++q) kstep(q, it + q, false);
    }

    // ---- epilogue
    // The last row of tiles was written by the most recent MFMAs: give them
    // time to finish before any accumulator is read (the tiles of earlier
    // rows are at least FN MFMAs old): 24 wait states, rule (1) at the MFMA
    // definitions.
    static_assert(FN == 4 || FN == 8, "the wait below lists the last row's tiles");
    if constexpr (FN == 8)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(acc[FM - 1][0]), "+a"(acc[FM - 1][1]), "+a"(acc[FM - 1][2]), "+a"(acc[FM - 1][3]),
                       "+a"(acc[FM - 1][4]), "+a"(acc[FM - 1][5]), "+a"(acc[FM - 1][6]), "+a"(acc[FM - 1][7]));
    else
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(acc[FM - 1][0]), "+a"(acc[FM - 1][1]), "+a"(acc[FM - 1][2]), "+a"(acc[FM - 1][3]));
    // All loads (the B stages' direct LDS writes included) have landed and
    // every wavefront is done with the stages before they are reused for C:
    // each wavefront stages its block through one stage of its own.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    const int row0 = m0 + wm * WM, col0 = n0 + wn * WN;
    if constexpr (SPLIT) {
        // fp32 sums of this split, unrounded: lane l of tile (bi, bj) holds 4
        // consecutive columns of one row, one 16-byte store (N is a multiple
        // of 8, so the 4 columns are wholly inside or outside)
        float* P = ws + (size_t)b * M * N;
        const int r = row0 + (lane & 15), c = col0 + 4 * (lane >> 4);
#pragma unroll
        for (int bi = 0; bi < FM; ++bi)
#pragma unroll
            for (int bj = 0; bj < FN; ++bj)
                if (r + 16 * bi < M && c + 16 * bj < N)
                    *(f32x4*)(P + (size_t)(r + 16 * bi) * N + c + 16 * bj) = acc[bi][bj];
        clock_sample(clk, 1);
        return;
    }
    __syncthreads();
    if constexpr (SB == 4) {
        // as many whole 16-row tile rows per pass as a B stage holds and WM
        // divides into (64 of 128, 48 of 96)
        constexpr int RP_MAX = B_BYTES / (WN * 2);
        constexpr int RP = WM % RP_MAX == 0 ? RP_MAX : WM % 48 == 0 && RP_MAX >= 48 ? 48 : 16;
        store_c_block<T, WM, WN, RP * WN * 2>(acc, b_stage(wave), lane, row0, col0, M, N, C);
    } else {
        constexpr int CW = A_BYTES < B_BYTES ? A_BYTES : B_BYTES;
        lds_byte* cw = wave < 2 ? a_stage(wave) : b_stage(wave - 2);
        store_c_block<T, WM, WN, CW>(acc, cw, lane, row0, col0, M, N, C);
    }
    clock_sample(clk, 1);
}

// A staged two K-steps at a time (256 x 256 tiles, fp16/bf16, one product per
// workgroup, no split): otherwise the schedule of the A-direct kernel above.
//
// A 32-deep K-step of A is 64 bytes of each of the tile's rows, so a 1 KB
// load of it covers 16 rows and touches 16 cache lines for half their bytes;
// staging A for two K-steps at once makes each row 128 bytes and each load
// 8 whole lines, as B's loads already are (a copy of the A-direct kernel
// whose A loads read whole aligned lines in this pattern ran 94.7-94.9
// against 97.3-97.5 us at 4096^3 on MI355X, same box, alternating).
//
//  * LDS: two A slots of [BM][64] (128-byte rows, 16-byte pieces XOR-ed by
//    (row/2)%8, the layout of the 64-deep K-step kernels), slot p%2 for the
//    K-steps 2p, 2p+1; four B stages of [32][BN] (B's layout above), stage
//    s%4 for K-step s.  128 KB at 256 x 256, as the A-direct ring.
//  * Loads: every half K-step issues the same number of loads per
//    wavefront, spread over its MFMAs.  K-step it (odd): before its barrier,
//    B of K-step it+3; after it, the first half of the A pair of K-steps
//    it+3, it+4.  K-step it (even): before its barrier, the second half of
//    the A pair of K-steps it+2, it+3; after it, B of K-step it+3.  A stage
//    or slot is refilled only after the barrier that follows the last read of
//    its previous contents.
//  * Counted waits: before barrier it the wavefront's loads for K-step it+1
//    (whose fragments are read after the barrier) must have landed, which
//    leaves 2*B_LOADS of its loads in flight for odd it and B_LOADS + A_LOADS
//    for even it (A_LOADS per half pair).  Measured on MI355X, requiring the
//    loads half a K-step earlier than the A-direct ring does cost nothing.
template <typename T, int BM, int BN>
__global__ __launch_bounds__(256, 1) void gemm_mfma16x16_pair_kernel(
    const T* A, const T* B, T* C, int M, int N, int K, int group_m, int xcd_remap, Batch bt, unsigned long long* clk)
{
    clock_sample(clk, 0);
    constexpr int NW = 4, BK = 32;
    constexpr int WM = BM / 2, WN = BN / 2;      // per-wavefront block (2 x 2 wavefronts)
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int NT = FM * FN;                  // MFMAs per wavefront per K-step
    constexpr int BAR = NT / 2;                  // MFMAs of a K-step before its barrier
    constexpr int ROW_P = 2 * BK * 2;            // bytes of an A row of a K-step pair
    constexpr int PAIR_BYTES = BM * ROW_P;
    constexpr int ROW_B = BN * 2;
    constexpr int B_BYTES = BK * ROW_B;
    constexpr int A_LOADS2 = PAIR_BYTES / 1024 / NW;   // A loads per wavefront per pair
    constexpr int AH = A_LOADS2 / 2;                    // ... per half pair
    constexpr int B_LOADS = B_BYTES / 1024 / NW;        // B loads per wavefront per K-step
    constexpr int NR = FM + FN;                         // operand fragments per K-step
    static_assert(AH >= 1 && A_LOADS2 % 2 == 0 && B_LOADS >= 1, "tile too small");
    static_assert(ROW_B % 256 == 0, "B rows must be whole bank windows");
    static_assert(2 * PAIR_BYTES + 4 * B_BYTES <= 160 * 1024, "LDS");
    // Every slot and stage is an LDS object of its own (the compiler tracks
    // direct-to-LDS loads per object).
    __shared__ __attribute__((aligned(1024))) unsigned char pa0[PAIR_BYTES], pa1[PAIR_BYTES];
    __shared__ __attribute__((aligned(1024))) unsigned char pb0[B_BYTES], pb1[B_BYTES], pb2[B_BYTES], pb3[B_BYTES];
    auto a_slot = [&](int p) __attribute__((always_inline)) { return (lds_byte*)(p == 0 ? pa0 : pa1); };
    auto b_stage = [&](int st) __attribute__((always_inline)) {
        return (lds_byte*)(st == 0 ? pb0 : st == 1 ? pb1 : st == 2 ? pb2 : pb3);
    };

    const int tiles_m = cdiv_i(M, BM), tiles_n = cdiv_i(N, BN);
    int b, tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, bt.count, group_m, xcd_remap != 0, b, tm, tn);
    A += b * bt.sa;
    B += b * bt.sb;
    C += b * bt.sc;
    const int m0 = tm * BM, n0 = tn * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (unsigned)M * (unsigned)K * 2u);

    // A load j of a pair (j < A_LOADS2): 1 KB = 8 rows of 128 bytes; lane ->
    // row 8*(wave*A_LOADS2 + j) + lane/8, physical piece lane%8 holding
    // logical piece (lane%8) ^ swz_a<64>(row): global (m0+row)*K + k0 + 8*piece
    // (kOOB for rows >= M and, per pair, pieces at or past K).
    unsigned a_voff[A_LOADS2];
    int a_kp[A_LOADS2];
#pragma unroll
    for (int j = 0; j < A_LOADS2; ++j) {
        const int row = 8 * (wave * A_LOADS2 + j) + lane / 8;
        const int piece = (lane % 8) ^ swz_a<2 * BK>(row);
        a_voff[j] = (m0 + row) < M ? ((unsigned)(m0 + row) * (unsigned)K + (unsigned)piece * 8u) * 2u : kOOB;
        a_kp[j] = piece * 8;
    }
    // B load j of a K-step: as in the kernel above.
    unsigned b_voff[B_LOADS];
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
        const int byte = 1024 * (wave * B_LOADS + j) + lane * 16;
        const int k = byte / ROW_B;
        const int piece = ((byte % ROW_B) / 16) ^ swz_b<BN>(k);
        const int col = n0 + piece * 8;
        b_voff[j] = col < N ? ((unsigned)k * (unsigned)N + (unsigned)col) * 2u : kOOB;
    }
    // A pair starting at K k0_in, load j -> slot p.
    auto load_a = [&](int p, int k0_in, int j) __attribute__((always_inline)) {
        const int k0 = __builtin_amdgcn_readfirstlane(k0_in);
        const unsigned off = a_kp[j] < K - k0 ? a_voff[j] : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (void __attribute__((address_space(3)))*)(a_slot(p) + (wave * A_LOADS2 + j) * 1024), 16, off,
            (k0 < K ? k0 : 0) * 2, 0, 0);
    };
    // B rows of the K-step at k0_in, load j -> stage st.
    auto load_b = [&](int st, int k0_in, int j) __attribute__((always_inline)) {
        const int k0 = __builtin_amdgcn_readfirstlane(k0_in);
        const int krem = K - k0;
        const int rows = __builtin_amdgcn_readfirstlane(krem < 0 ? 0 : (krem > BK ? BK : krem));
        const __amdgpu_buffer_rsrc_t rbk =
            make_rsrc(B + (size_t)(k0 < K ? k0 : 0) * N, (unsigned)rows * (unsigned)N * 2u);
        const unsigned off = b_voff[j];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rbk, (void __attribute__((address_space(3)))*)(b_stage(st) + (wave * B_LOADS + j) * 1024), 16, off, 0,
            0, 0);
    };

    // Operand reads: A fragment of K-step h of a pair (h = 0, 1), tile bi:
    // row wm*WM + 16*bi + lane%16, logical piece 4*h + lane/16; B as above.
    int a_rd[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        a_rd[h] = (wm * WM + (lane & 15)) * ROW_P + (((4 * h + (lane >> 4)) ^ swz_a<2 * BK>(lane & 15)) * 16);
    int b_rd[FN];
#pragma unroll
    for (int bj = 0; bj < FN; ++bj) {
        const int g16 = lane & 15;
        const int k = 8 * (lane >> 4) + (g16 >> 2);
        const int n = wn * WN + 16 * bj + 4 * (g16 & 3);
        const int piece = (n >> 3) ^ swz_b<BN>(k);
        b_rd[bj] = k * ROW_B + piece * 16 + (n & 7) * 2;
    }
    f32x4 acc[FM][FN];
    u32x4 fa[2][FM], fb[2][FN];
    // Fragment o of K-step s's operands (B tiles first, then A tiles) ->
    // register set `set`; s's pair slot is (s/2)%2, its half s%2, its B
    // stage s%4 (all literals below).
    auto read_frag = [&](int set, int slot, int h, int stb, int o) __attribute__((always_inline)) {
        if (o < FN) {
            const lds_byte* p = b_stage(stb) + b_rd[o];
            const s16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)p);
            const s16x4 h1 =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p + 4 * ROW_B));
            fb[set][o] = __builtin_bit_cast(u32x4, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            fa[set][o - FN] = *(const u32x4 __attribute__((address_space(3)))*)(a_slot(slot) + a_rd[h] +
                                                                                (o - FN) * 16 * ROW_P);
        }
    };

    // ---- prologue: what K-steps -3 .. -1 would have issued: the A pair of
    // K-steps 0, 1 (slot 0), B of K-steps 0, 1, 2, the first half of the A
    // pair of K-steps 2, 3 (slot 1).  Then K-step 0's operands: the A pair
    // (0, 1) and B of K-step 0 must have landed.
#pragma unroll
    for (int j = 0; j < A_LOADS2; ++j) load_a(0, 0, j);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int s = 0; s < 3; ++s) {
#pragma unroll
        for (int j = 0; j < B_LOADS; ++j) load_b(s, s * BK, j);
        asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int j = 0; j < AH; ++j) load_a(1, 2 * BK, j);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * B_LOADS + AH));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int o = 0; o < NR; ++o) read_frag(0, 0, 0, 0, o);

    auto op_lo = [](int pos, int n, int span) __attribute__((always_inline)) { return (pos * n + span - 1) / span; };
    // K-step it (q = it % 4): MFMAs 0 .. BAR-1 with this half's loads, the
    // counted wait and the barrier, then MFMAs BAR .. NT-1 with the second
    // half's loads and the operand reads of K-step it+1 (loads at evenly
    // spaced operations, reads in between).
    auto kstep = [&](auto q_c, int it, const bool first) __attribute__((always_inline)) {
        constexpr int q = decltype(q_c)::value;
        constexpr int set = q & 1;
        constexpr int n1 = (q & 1) ? B_LOADS : AH;   // odd: B of it+3; even: A pair (it+2, it+3), 2nd half
        constexpr int n2 = (q & 1) ? AH : B_LOADS;   // odd: A pair (it+3, it+4), 1st half; even: B of it+3
        constexpr unsigned kWaitBar = waitcnt_vm((q & 1) ? 2 * B_LOADS : B_LOADS + 2 * AH);
        auto load1 = [&](int o) __attribute__((always_inline)) {
            if (q & 1)
                load_b((q + 3) % 4, (it + 3) * BK, o);
            else
                load_a((q / 2 + 1) % 2, (it + 2) * BK, AH + o);
        };
        auto load2 = [&](int o) __attribute__((always_inline)) {
            if (q & 1)
                load_a(((q + 3) / 2) % 2, (it + 3) * BK, o);
            else
                load_b((q + 3) % 4, (it + 3) * BK, o);
        };
        auto mfma = [&](int x) __attribute__((always_inline)) {
            if (first)
                Mfma16x16<T>::first(acc[x / FN][x % FN], fb[set][x % FN], fa[set][x / FN]);
            else
                Mfma16x16<T>::acc(acc[x / FN][x % FN], fb[set][x % FN], fa[set][x / FN]);
        };
#pragma unroll
        for (int x = 0; x < BAR; ++x) {
            mfma(x);
#pragma unroll
            for (int o = op_lo(x, n1, BAR); o < op_lo(x + 1, n1, BAR); ++o) load1(o);
        }
        // every load of this half was issued above (keep the compiler from
        // sinking any past the count)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kWaitBar);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // this wavefront's reads of the stages done
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        constexpr int nops2 = n2 + NR;
#pragma unroll
        for (int x = BAR; x < NT; ++x) {
            mfma(x);
#pragma unroll
            for (int o = op_lo(x - BAR, nops2, NT - BAR); o < op_lo(x + 1 - BAR, nops2, NT - BAR); ++o) {
                const int nld = (o * n2) / nops2 + 1;   // loads at operations 0 .. o
                if (o == 0 || (o * n2) / nops2 != ((o - 1) * n2) / nops2)
                    load2(nld - 1);
                else
                    read_frag(set ^ 1, ((q + 1) / 2) % 2, (q + 1) & 1, (q + 1) % 4, o - nld);
            }
        }
    };
    // K-steps, rounded up to the 4-step unroll (the extra steps multiply the
    // zeros their loads brought in).
    const int nk = cdiv_i(cdiv_i(K, BK), 4) * 4;
    using Q0 = std::integral_constant<int, 0>;
    using Q1 = std::integral_constant<int, 1>;
    using Q2 = std::integral_constant<int, 2>;
    using Q3 = std::integral_constant<int, 3>;
    kstep(Q0{}, 0, true);
    kstep(Q1{}, 1, false);
    kstep(Q2{}, 2, false);
    kstep(Q3{}, 3, false);
    for (int it = 4; it < nk; it += 4) {
        kstep(Q0{}, it, false);
        kstep(Q1{}, it + 1, false);
        kstep(Q2{}, it + 2, false);
        kstep(Q3{}, it + 3, false);
    }

    // ---- epilogue: as in the kernel above (the last row of tiles was
    // written by the most recent MFMAs; each wavefront stages its block
    // through one B stage of its own)
    static_assert(FN == 8 || FN == 4, "the wait below lists the last row's tiles");
    if constexpr (FN == 8)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(acc[FM - 1][0]), "+a"(acc[FM - 1][1]), "+a"(acc[FM - 1][2]), "+a"(acc[FM - 1][3]),
                       "+a"(acc[FM - 1][4]), "+a"(acc[FM - 1][5]), "+a"(acc[FM - 1][6]), "+a"(acc[FM - 1][7]));
    else
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(acc[FM - 1][0]), "+a"(acc[FM - 1][1]), "+a"(acc[FM - 1][2]), "+a"(acc[FM - 1][3]));
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    constexpr int RP_MAX = B_BYTES / (WN * 2);
    constexpr int RP = WM % RP_MAX == 0 ? RP_MAX : WM % 48 == 0 && RP_MAX >= 48 ? 48 : 16;
    store_c_block<T, WM, WN, RP * WN * 2>(acc, b_stage(wave), lane, m0 + wm * WM, n0 + wn * WN, M, N, C);
    clock_sample(clk, 1);
}

template <typename T>
hipError_t launch_t(const Config& cfg, const LaunchArgs& a)
{
    const int tiles = cdiv_i(a.M, cfg.bm) * cdiv_i(a.N, cfg.bn);
    const dim3 grid(tiles * a.batch.count), block(256);
    const T* A = static_cast<const T*>(a.A);
    const T* B = static_cast<const T*>(a.B);
    T* C = static_cast<T*>(a.C);
    if (cfg.threads != 256) return hipErrorInvalidValue;
    if (cfg.sched == 2) {   // A staged two K-steps at a time: 256 x 256, 192 x 256 or 128 x 128, one pass only
        if (a.splits > 1 || cfg.bk != 32) return hipErrorInvalidValue;
        if (cfg.bm == 128 && cfg.bn == 128)
            hipLaunchKernelGGL((gemm_mfma16x16_pair_kernel<T, 128, 128>), grid, block, 0, a.stream, A, B, C, a.M,
                               a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.clk);
        else if (cfg.bn != 256)
            return hipErrorInvalidValue;
        else if (cfg.bm == 256)
            hipLaunchKernelGGL((gemm_mfma16x16_pair_kernel<T, 256, 256>), grid, block, 0, a.stream, A, B, C, a.M,
                               a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.clk);
        else if (cfg.bm == 192)
            hipLaunchKernelGGL((gemm_mfma16x16_pair_kernel<T, 192, 256>), grid, block, 0, a.stream, A, B, C, a.M,
                               a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.clk);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
    if (cfg.sched == 1) {   // A direct to LDS as well; split K at 128 x 128 only
        if (a.splits > 1) {
            if (cfg.bm == 128 && cfg.bn == 128 && cfg.bk == 32)
                hipLaunchKernelGGL((gemm_mfma16x16_kernel<T, 128, 128, 32, true, true>), dim3(tiles * a.splits),
                                   block, 0, a.stream, A, B, C, a.M, a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.ws, a.splits, a.clk);
            else if (cfg.bm == 64 && cfg.bn == 128 && cfg.bk == 32)
                hipLaunchKernelGGL((gemm_mfma16x16_kernel<T, 64, 128, 32, true, true>), dim3(tiles * a.splits),
                                   block, 0, a.stream, A, B, C, a.M, a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.ws, a.splits, a.clk);
            else
                return hipErrorInvalidValue;
            return hipGetLastError();
        }
        if (cfg.bm == 256 && cfg.bn == 256 && cfg.bk == 32)
            hipLaunchKernelGGL((gemm_mfma16x16_kernel<T, 256, 256, 32, false, true>), grid, block, 0, a.stream, A, B,
                               C, a.M, a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.ws, 1, a.clk);
        else if (cfg.bm == 128 && cfg.bn == 128 && cfg.bk == 32)
            hipLaunchKernelGGL((gemm_mfma16x16_kernel<T, 128, 128, 32, false, true>), grid, block, 0, a.stream, A, B,
                               C, a.M, a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.ws, 1, a.clk);
        else if (cfg.bm == 192 && cfg.bn == 256 && cfg.bk == 32)
            hipLaunchKernelGGL((gemm_mfma16x16_kernel<T, 192, 256, 32, false, true>), grid, block, 0, a.stream, A, B,
                               C, a.M, a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.ws, 1, a.clk);
        else if (cfg.bm == 64 && cfg.bn == 128 && cfg.bk == 32)
            hipLaunchKernelGGL((gemm_mfma16x16_kernel<T, 64, 128, 32, false, true>), grid, block, 0, a.stream, A, B,
                               C, a.M, a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.ws, 1, a.clk);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
#define DGR_LAUNCH(BM_, BN_, BK_)                                                                          \
    if (cfg.bm == BM_ && cfg.bn == BN_ && cfg.bk == BK_) {                                                \
        if (a.splits > 1)                                                                                 \
            hipLaunchKernelGGL((gemm_mfma16x16_kernel<T, BM_, BN_, BK_, true>), dim3(tiles * a.splits), block, \
                               0, a.stream, A, B, C, a.M, a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.ws, a.splits, a.clk); \
        else                                                                                              \
            hipLaunchKernelGGL((gemm_mfma16x16_kernel<T, BM_, BN_, BK_, false>), grid, block, 0, a.stream, A, B, \
                               C, a.M, a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.ws, 1, a.clk);                          \
        return hipGetLastError();                                                                         \
    }
    DGR_LAUNCH(256, 256, 32)
    DGR_LAUNCH(256, 128, 32)
    DGR_LAUNCH(256, 256, 64)
    DGR_LAUNCH(256, 128, 64)
    DGR_LAUNCH(128, 128, 32)
    DGR_LAUNCH(192, 256, 32)
    DGR_LAUNCH(64, 128, 32)
#undef DGR_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_mfma16x16(const Config& cfg, const LaunchArgs& a)
{
    if (a.dtype == kF16) return launch_t<_Float16>(cfg, a);
    if (a.dtype == kBF16) return launch_t<__bf16>(cfg, a);
    return hipErrorInvalidValue;
}

}  // namespace dgr
