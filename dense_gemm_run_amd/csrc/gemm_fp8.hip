// MFMA kernel for 8-bit floating-point inputs (OCP FP8: E4M3 or E5M2, both
// operands of one format) with fp32 accumulation and a bf16 result: the FP8
// input path of notebook "Triton tiled matmul" (the exercises: FP8 inputs,
// the accumulator stays FP32, compared against FP16).  It is built on
// v_mfma_f32_32x32x64_f8f6f4, which takes 32 one-byte values of each operand
// per lane and forms every product exactly (two 4-bit significands) before
// the fp32 sums.  Rows must be 16-byte aligned: K and N multiples of 16, A,
// B and C 16-byte aligned.
//
// The structure is that of the 16x16x32 kernel (the tiled loop of
// kernels-book chapter "Matrix Multiplication", section "Tiles": one
// workgroup per BM x BN output tile, 256 x 256 or 128 x 128, fp32
// accumulators that live across the whole K walk), with one-byte elements:
//
//  * Math: 4 wavefronts in a 2 x 2 grid, each owning BM/2 x BN/2 outputs as
//    tiles of 32 x 32 (4 x 4 of them, the 256 accumulator registers of a
//    lane, at 256 x 256; 2 x 2 at 128 x 128, where two workgroups share a
//    CU).  A
//    64-deep K-slice is one MFMA per tile; a K-step of BK = 64 or 128 is one
//    or two K-slices.  The MFMAs are inline assembly with the accumulator
//    tied to the destination (and source C = 0 on the first K-slice), which
//    also fixes their order against the memory instructions around them.
//  * Operands: lane l of a tile's A fragment holds row l%32 and the 32
//    bytes k = 32*(l/32) .. +31 of the K-slice; lane l of the B fragment
//    holds column l%32 and the same 32 k.  The MFMA is given the B fragment
//    first, so it computes the transposed tile and each lane ends with 4
//    consecutive columns of one row (the layout the 32x32 epilogue takes).
//  * Staging: A goes through registers (LEAD slots, K-step it+LEAD loaded
//    during K-step it and written to one of two A stages during K-step
//    it+LEAD-1); B goes global -> LDS directly into a ring of SB stages.
//    16-byte pieces at or past K, rows past M and columns past N read zeros
//    (the zero padding of chapter "Matrix Multiplication", section "The real
//    tiled loop").
//  * LDS layout: A [BM][BK] with 16-byte pieces XOR-swizzled: a fragment
//    read has its four 16-lane groups take one piece each of rows 0-15,
//    16-31, 0-15 and 16-31 of a tile.  Measured with the bank-conflict
//    counter on that exact read, XOR (row/4) % 4 is conflict-free for 64-byte
//    rows (BK = 64) where (row/2) % 4 costs a 2-way conflict, and XOR
//    (row/2) % 8 is conflict-free for 128-byte rows.  B [BK][BN]: the 8-bit
//    transpose read of a half-wavefront covers 8 consecutive rows and one
//    32-byte column pair of each, and the swizzle puts those 8 pairs in the
//    8 different 32-byte bank groups of the 256 bytes the banks span.  With
//    256-byte rows piece p of row k is stored at p ^ 2*(k%8); with 128-byte
//    rows, two to a bank span, at p ^ 2*((k/2)%4), which separates the pairs
//    of the 4 even (and the 4 odd) rows.
//  * One barrier per K-step, half a K-slice before its end; the loads and
//    LDS traffic of a K-step are spread over its MFMAs.
//  * Epilogue: fp32 -> bf16 (round to nearest even), staged through LDS and
//    written as whole row segments, skipping rows >= M and columns >= N.
//  * A direct to LDS (ADMA, K-step 64): as in the 16x16x32 kernel, A's
//    16-byte pieces go global -> LDS at the places the register path writes
//    them, into the stage of B's ring for the same K-step (one LDS object per
//    stage); a K-step's group of A and B loads is spread over the whole
//    K-step, half after its barrier and half before the next one.
//  * Split K (SPLIT): as in the 16x16x32 kernel, `splits` workgroups per
//    tile walk disjoint ranges of K-steps and write their fp32 sums,
//    unrounded, to their own M x N slice of a workspace; a second kernel adds
//    the slices in split order and rounds once to bf16.
#include "gemm_internal.h"
#include "gemm_device.h"

namespace dgr {
namespace {

typedef unsigned u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// c (+)= b-fragment x a-fragment over one 64-deep K-slice.  FMT 0: both
// operands E4M3 (the instruction's default); FMT 1: both E5M2.
// Inline-assembly MFMAs: the wait-state rules the schedule relies on are
// those listed at the 16x16 kernel's MFMA definitions (gemm_mfma16x16.hip):
// accumulator reads 19+ wait states after the last write (the epilogue's
// s_nop waits), operands written only by LDS reads covered by the
// compiler's s_waitcnt, source C either 0 or exactly the destination.
template <int FMT> struct MfmaFp8;
template <> struct MfmaFp8<0> {
    static __device__ __forceinline__ void acc(f32x16& c, const u32x8& b, const u32x8& a)
    {
        asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
    }
    static __device__ __forceinline__ void first(f32x16& c, const u32x8& b, const u32x8& a)
    {
        asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=a"(c) : "v"(b), "v"(a));
    }
};
template <> struct MfmaFp8<1> {
    static __device__ __forceinline__ void acc(f32x16& c, const u32x8& b, const u32x8& a)
    {
        asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0 cbsz:1 blgp:1" : "+a"(c) : "v"(b), "v"(a));
    }
    static __device__ __forceinline__ void first(f32x16& c, const u32x8& b, const u32x8& a)
    {
        asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0 cbsz:1 blgp:1" : "=a"(c) : "v"(b), "v"(a));
    }
};

// c += b-fragment x a-fragment, 16 x 16 x 128 (each lane: 32 consecutive K
// of one row of A and of one column of B; C as in the 16-bit 16x16 kernels:
// lane l holds row l%16, columns 4*(l/16) .. +3).  Wait states as for the
// 32 x 32 form above.
template <int FMT> struct MfmaFp8x16;
template <> struct MfmaFp8x16<0> {
    static __device__ __forceinline__ void acc(f32x4& c, const u32x8& b, const u32x8& a)
    {
        asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
    }
    static __device__ __forceinline__ void first(f32x4& c, const u32x8& b, const u32x8& a)
    {
        asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, 0" : "=a"(c) : "v"(b), "v"(a));
    }
};
template <> struct MfmaFp8x16<1> {
    static __device__ __forceinline__ void acc(f32x4& c, const u32x8& b, const u32x8& a)
    {
        asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0 cbsz:1 blgp:1" : "+a"(c) : "v"(b), "v"(a));
    }
    static __device__ __forceinline__ void first(f32x4& c, const u32x8& b, const u32x8& a)
    {
        asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, 0 cbsz:1 blgp:1" : "=a"(c) : "v"(b), "v"(a));
    }
};

template <int BK> __device__ __forceinline__ int swz_a(int row)
{
    return BK == 64 ? (row >> 2) & 3 : (row >> 1) & 7;
}
template <int BN> __device__ __forceinline__ int swz_b(int k)
{
    return BN == 256 ? 2 * (k & 7) : 2 * ((k >> 1) & 3);
}

template <int FMT, int BM, int BN, int BK, bool SPLIT, bool ADMA = false>
__global__ __launch_bounds__(256, BM * BN >= 192 * 256 ? 1 : 2) void gemm_fp8_kernel(
    const unsigned char* A, const unsigned char* B, __bf16* C,
    int M, int N, int K, int group_m, int xcd_remap, Batch bt, float* ws, int splits, unsigned long long* clk)
{
    clock_sample(clk, 0);
    constexpr int NW = 4;                        // wavefronts, 2 x 2
    constexpr int WM = BM / 2, WN = BN / 2;      // per-wavefront block
    constexpr int FM = WM / 32, FN = WN / 32;    // 32x32 tiles per wavefront
    constexpr int NT = FM * FN;                  // MFMAs per wavefront per 64-deep K-slice
    constexpr int NS = BK / 64;                  // K-slices per K-step
    constexpr int XS = NS * NT;                  // MFMAs per wavefront per K-step
    constexpr int LEAD = 256 / BK;               // A register slots (K-steps loaded ahead)
    constexpr int SB = BK == 64 ? 4 : 2;         // B stages (K-steps loaded ahead)
    constexpr int ROW_A = BK;                    // bytes per A tile row
    constexpr int PA = BK / 16;                  // 16-byte pieces per A row
    constexpr int A_BYTES = BM * ROW_A;
    constexpr int ROW_B = BN;
    constexpr int B_BYTES = BK * ROW_B;
    constexpr int A_LOADS = A_BYTES / 1024 / NW; // 16-byte-per-lane loads per wavefront
    constexpr int B_LOADS = B_BYTES / 1024 / NW;
    constexpr int LOADS = A_LOADS + B_LOADS;     // vector-memory instructions per K-step
    constexpr int NR = FM + FN;                  // operand fragments per K-slice
    constexpr int BAR = XS - NT / 2;             // MFMAs of a K-step before its barrier
    static_assert(BK == 64 || BK == 128, "K-step");
    static_assert((BM == 256 && BN == 256) || (BM == 128 && BN == 128) || (BM == 64 && BN == 128 && ADMA) ||
                      (BM == 192 && BN == 256 && ADMA),
                  "tile");
    static_assert(LEAD % 2 == 0 && LEAD % SB == 0, "slot and stage periods must divide the unroll");
    static_assert((SB - 1) * B_BYTES < 65536, "LDS immediate offsets");
    static_assert(!ADMA || (SB == 4 && LEAD == 4), "direct A loads: 64-deep K-steps");
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

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (unsigned)M * (unsigned)K);

    // ---- global load geometry (byte offsets; one element is one byte)
    // A: load j fills 1 KB = 1024/ROW_A tile rows; lane -> row +lane/PA,
    //    physical piece lane%PA holding logical piece p ^ swz_a(row).
    unsigned a_voff[A_LOADS];
    int a_kp[A_LOADS];
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
        const int row = (1024 / ROW_A) * (wave * A_LOADS + j) + lane / PA;
        const int piece = (lane % PA) ^ swz_a<BK>(row);
        a_voff[j] = (m0 + row) < M ? (unsigned)(m0 + row) * (unsigned)K + (unsigned)piece * 16u : kOOB;
        a_kp[j] = piece * 16;
    }
    // B: load j fills 4 tile rows; lane -> row k = (1024*(wave*B_LOADS+j) +
    //    16*lane) / 256, physical piece lane%16 holding logical piece
    //    p ^ swz_b(k), i.e. columns n0 + 16*p .. +15 (kOOB past N), relative
    //    to a buffer that starts at row k0 and ends at row min(K, k0 + BK).
    unsigned b_voff[B_LOADS];
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
        const int byte = 1024 * (wave * B_LOADS + j) + lane * 16;
        const int k = byte / ROW_B;
        const int piece = ((byte % ROW_B) / 16) ^ swz_b<BN>(k);
        const int col = n0 + piece * 16;
        b_voff[j] = col < N ? (unsigned)k * (unsigned)N + (unsigned)col : kOOB;
    }

    u32x4 stg[LEAD][A_LOADS];
    auto load_a = [&](int slot, int k0_in, int j) __attribute__((always_inline)) {
        const int k0 = __builtin_amdgcn_readfirstlane(kb + k0_in);
        const unsigned off = a_kp[j] < ke - k0 ? a_voff[j] : kOOB;
        stg[slot][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, off, k0, 0));
    };
    auto load_a_lds = [&](int st, int k0_in, int j) __attribute__((always_inline)) {
        const int k0 = __builtin_amdgcn_readfirstlane(kb + k0_in);
        const unsigned off = a_kp[j] < ke - k0 ? a_voff[j] : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (void __attribute__((address_space(3)))*)(a_stage(st) + (wave * A_LOADS + j) * 1024), 16,
            off, k0, 0, 0);
    };
    auto store_a = [&](int st, int slot, int j) __attribute__((always_inline)) {
        lds_byte* p = a_stage(st) + (wave * A_LOADS + j) * 1024 + lane * 16;
        *(u32x4 __attribute__((address_space(3)))*)p = stg[slot][j];
    };
    auto load_b = [&](int st, int k0_in, int j) __attribute__((always_inline)) {
        const int k0 = __builtin_amdgcn_readfirstlane(kb + k0_in);
        const int krem = ke - k0;
        const int rows = __builtin_amdgcn_readfirstlane(krem < 0 ? 0 : (krem > BK ? BK : krem));
        const __amdgpu_buffer_rsrc_t rbk =
            make_rsrc(B + (size_t)(k0 < ke ? k0 : 0) * N, (unsigned)rows * (unsigned)N);
        const unsigned off = b_voff[j];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rbk, (void __attribute__((address_space(3)))*)(b_stage(st) + (wave * B_LOADS + j) * 1024), 16,
            off, 0, 0, 0);
    };

    // ---- operand read addresses within a stage
    // A fragment (K-slice sl, tile bi): row wm*WM + 32*bi + lane%32, logical
    // pieces 4*sl + 2*(lane/32) and the next (32 bytes); the swizzle uses bits
    // 1-3 of the row only, so it depends on lane%32 alone.
    int a_rd[NS][2];
#pragma unroll
    for (int sl = 0; sl < NS; ++sl)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            a_rd[sl][h] = (wm * WM + (lane & 31)) * ROW_A +
                          (((4 * sl + 2 * (lane >> 5) + h) ^ swz_a<BK>(lane & 31)) * 16);
    // B fragment (tile bj) via four 8-bit transpose reads h = 0..3: in 16-lane
    // group G = lane/16, lane 2r+q points at K row 32*(G/2) + 8h + r (+64 per
    // K-slice), bytes 8q .. 8q+7 of the 16 columns wn*WN + 32*bj + 16*(G%2)
    // .. +15; lane i of the group receives column i over those 8 rows, which
    // are bytes 8h .. 8h+7 of its 32-byte operand.  The swizzle depends on
    // k%8 = r alone, the same for every h and K-slice.
    int b_rd[FN];
#pragma unroll
    for (int bj = 0; bj < FN; ++bj) {
        const int G = lane >> 4, r = (lane & 15) >> 1, q = lane & 1;
        const int piece = (wn * WN + 32 * bj + 16 * (G & 1)) / 16;
        b_rd[bj] = (32 * (G >> 1) + r) * ROW_B + ((piece ^ swz_b<BN>(r)) * 16) + 8 * q;
    }
    auto read_a = [&](int st, int sl, int bi) __attribute__((always_inline)) -> u32x8 {
        const lds_byte* base = a_stage(st) + bi * 32 * ROW_A;
        const u32x4 lo = *(const u32x4 __attribute__((address_space(3)))*)(base + a_rd[sl][0]);
        const u32x4 hi = *(const u32x4 __attribute__((address_space(3)))*)(base + a_rd[sl][1]);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto read_b = [&](int st, int sl, int bj) __attribute__((always_inline)) -> u32x8 {
        const lds_byte* p = b_stage(st) + b_rd[bj] + sl * 64 * ROW_B;
        i32x2 h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            h[i] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 __attribute__((address_space(3)))*)(p + 8 * i * ROW_B));
        const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3));
        const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_shufflevector(h[2], h[3], 0, 1, 2, 3));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    f32x16 acc[FM][FN];
    u32x8 fa[2][FM], fb[2][FN];   // two operand register sets, alternating by K-slice
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

    // One K-step (q = it % LEAD, a literal): MFMAs 0 .. BAR-1 interleaved
    // with the operand reads of the next K-slice of this step, the A writes of
    // K-step it+1 and the A loads of K-step it+LEAD; the counted wait for
    // this wavefront's B loads of K-step it+1 and the barrier; MFMAs BAR ..
    // XS-1 interleaved with the B loads of K-step it+SB (into the stage every
    // wavefront finished reading before the barrier) and the operand reads of
    // K-slice 0 of K-step it+1.  n operations spread over `span` MFMAs: the
    // ones issued after MFMA number pos are op_lo(pos) .. op_lo(pos+1)-1.
    auto op_lo = [](int pos, int n, int span) __attribute__((always_inline)) { return (pos * n + span - 1) / span; };

    // ADMA: group it (A and B of K-step it+SB, into stage it % SB, which
    // every wavefront finished reading before K-step it's barrier) is issued
    // in two parts, as in the 16x16x32 kernel: loads 0 .. P-1 after K-step
    // it's barrier, between the operand reads, and loads P .. LOADS-1 before
    // K-step it+1's barrier, spread over its first MFMAs, so that the
    // wavefronts do not queue a whole group each on the CU's load path at
    // once.  The counted wait is unchanged: at barrier it, groups it-2 and
    // it-1 are whole and group it has not started.
    constexpr int P_ADMA = LOADS / 2;
    auto load_group = [&](int st, int k0_in, int idx) __attribute__((always_inline)) {
        if (idx < A_LOADS)
            load_a_lds(st, k0_in, idx);
        else
            load_b(st, k0_in, idx - A_LOADS);
    };
    auto kslice = [&](const int q, int it, const int sl, const bool first) __attribute__((always_inline)) {
        const int sta = ADMA ? q % SB : q & 1, stb = q % SB, set = (q * NS + sl) & 1;
        const int sta_next = ADMA ? (q + 1) % SB : sta ^ 1;
        // ops before the barrier: A writes and A loads (A through
        // registers), or the second part of group it-1 (ADMA)
        constexpr int NOPS1 = ADMA ? LOADS - P_ADMA : 2 * A_LOADS;
        constexpr int LD2 = ADMA ? P_ADMA : B_LOADS;   // loads after the barrier
        constexpr int NOPS2 = LD2 + NR;
        auto mfma = [&](int xx) __attribute__((always_inline)) {
            if (first && sl == 0)
                MfmaFp8<FMT>::first(acc[xx / FN][xx % FN], fb[set][xx % FN], fa[set][xx / FN]);
            else
                MfmaFp8<FMT>::acc(acc[xx / FN][xx % FN], fb[set][xx % FN], fa[set][xx / FN]);
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
            asm volatile("" ::: "memory");
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

    // K-steps, rounded up to the LEAD-step unroll: the extra steps multiply
    // the zeros their loads brought in.
    const int nk = cdiv_i(cdiv_i(ke - kb, BK), LEAD) * LEAD;
    kstep(0, 0, true);
#pragma unroll
    for (int q = 1; q < LEAD; ++q) kstep(q, q, false);
    for (int it = LEAD; it < nk; it += LEAD) {
#pragma unroll
        for (int q = 0; q < LEAD; ++q) kstep(q, it + q, false);
    }

    // ---- epilogue.  The last row of tiles was written by the most recent
    // MFMAs (16 passes each): wait them out before any accumulator is read;
    // the other rows are at least FN >= 2 MFMAs old.
    static_assert(FN == 4 || FN == 2, "the wait below lists the last row's tiles");
    if constexpr (FN == 4)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(acc[FM - 1][0]), "+a"(acc[FM - 1][1]), "+a"(acc[FM - 1][2]), "+a"(acc[FM - 1][3]));
    else
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[FM - 1][0]), "+a"(acc[FM - 1][1]));
    // All loads (the B stages' direct LDS writes included) have landed and
    // every wavefront is done with the stages before they are reused for C.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    if constexpr (SPLIT) {
        // fp32 sums of this split, unrounded: lane l of tile (bi, bj) holds
        // row 32*bi + l%32, columns 32*bj + 8g + 4*(l/32) .. +3 in registers
        // 4g .. 4g+3: one 16-byte store per g (N is a multiple of 16)
        float* P = ws + (size_t)b * M * N;
        const int r = m0 + wm * WM + (lane & 31), c = n0 + wn * WN + 4 * (lane >> 5);
#pragma unroll
        for (int bi = 0; bi < FM; ++bi)
#pragma unroll
            for (int bj = 0; bj < FN; ++bj)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    if (r + 32 * bi < M && c + 32 * bj + 8 * g < N) {
                        f32x4 v;
                        v[0] = acc[bi][bj][4 * g];
                        v[1] = acc[bi][bj][4 * g + 1];
                        v[2] = acc[bi][bj][4 * g + 2];
                        v[3] = acc[bi][bj][4 * g + 3];
                        *(f32x4*)(P + (size_t)(r + 32 * bi) * N + c + 32 * bj + 8 * g) = v;
                    }
        clock_sample(clk, 1);
        return;
    }
    __syncthreads();
    // Each wavefront stages its block through a stage of its own, at most one
    // whole block (one pass) at a time.
    const int row0 = m0 + wm * WM, col0 = n0 + wn * WN;
    constexpr int BLOCK = WM * WN * 2;
    if constexpr (SB == 4) {
        // passes of as many whole 32-row tile rows as a B stage holds and WM
        // divides into (32 of 96)
        constexpr int CWB = B_BYTES < BLOCK ? B_BYTES : BLOCK;
        constexpr int CW = WM % (CWB / (WN * 2)) == 0 ? CWB : 32 * WN * 2;
        store_c_block_32x32<__bf16, WM, WN, CW>(acc, b_stage(wave), lane, row0, col0, M, N, C);
    } else {
        static_assert(A_BYTES == B_BYTES, "one C region per wavefront");
        lds_byte* cw = wave < 2 ? a_stage(wave) : b_stage(wave - 2);
        store_c_block_32x32<__bf16, WM, WN, (A_BYTES < BLOCK ? A_BYTES : BLOCK)>(acc, cw, lane, row0, col0,
                                                                              M, N, C);
    }
    clock_sample(clk, 1);
}

// A staged two K-steps at a time (256 x 256 and 192 x 256 tiles, one product
// per workgroup, no split): the scheme of the 16-bit A-pair kernel
// (gemm_mfma16x16.hip) with this kernel's 64-deep K-steps, fragments and
// epilogue.  A 64-deep K-step of one-byte A is 64 bytes of each row, so a
// 1 KB load of it touches 16 cache lines for half their bytes; two K-steps
// at once make each row 128 bytes and each A load 8 whole lines (a copy of
// the A-direct kernel reading A in this pattern ran E4M3 4096^3 in 48.3
// against 50.2-50.3 us on MI355X, same box, alternating).
//  * LDS: two A slots of [BM][128 B] (the 128-byte-row layout above, pieces
//    XOR-ed by (row/2)%8), K-steps 2p, 2p+1 in slot p%2; four B stages of
//    [64][BN], K-step s in stage s%4.
//  * Loads and counted waits as in the 16-bit A-pair kernel: an odd K-step
//    issues B of K-step it+3 before its barrier and the first half of the A
//    pair (it+3, it+4) after it; an even K-step the second half of the pair
//    (it+2, it+3) before and B of it+3 after; before barrier it the loads
//    for K-step it+1 have landed, leaving 2*B_LOADS loads in flight (odd it)
//    or B_LOADS + A_LOADS per half pair (even it).
template <int FMT, int BM, int BN>
__global__ __launch_bounds__(256, 1) void gemm_fp8_pair_kernel(const unsigned char* A, const unsigned char* B,
                                                               __bf16* C, int M, int N, int K, int group_m,
                                                               int xcd_remap, Batch bt, unsigned long long* clk)
{
    clock_sample(clk, 0);
    constexpr int NW = 4, BK = 64;
    constexpr int WM = BM / 2, WN = BN / 2;      // per-wavefront block (2 x 2 wavefronts)
    constexpr int FM = WM / 32, FN = WN / 32;    // 32x32 tiles per wavefront
    constexpr int NT = FM * FN;                  // MFMAs per wavefront per K-step
    constexpr int BAR = NT / 2;                  // MFMAs of a K-step before its barrier
    constexpr int ROW_P = 2 * BK;                // bytes of an A row of a K-step pair
    constexpr int PAIR_BYTES = BM * ROW_P;
    constexpr int ROW_B = BN;
    constexpr int B_BYTES = BK * ROW_B;
    constexpr int A_LOADS2 = PAIR_BYTES / 1024 / NW;   // A loads per wavefront per pair
    constexpr int AH = A_LOADS2 / 2;                    // ... per half pair
    constexpr int B_LOADS = B_BYTES / 1024 / NW;        // B loads per wavefront per K-step
    constexpr int NR = FM + FN;                         // operand fragments per K-step
    static_assert((BM == 256 || BM == 192) && BN == 256, "tile");
    static_assert(AH >= 1 && A_LOADS2 % 2 == 0 && B_LOADS >= 1, "tile too small");
    static_assert(2 * PAIR_BYTES + 4 * B_BYTES <= 160 * 1024, "LDS");
    // Every slot and stage is an LDS object of its own.
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
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (unsigned)M * (unsigned)K);

    // A load j of a pair: 8 rows of 128 bytes; lane -> row
    // 8*(wave*A_LOADS2 + j) + lane/8, physical piece lane%8 holding logical
    // piece (lane%8) ^ swz_a<128>(row) (kOOB for rows >= M and, per pair,
    // pieces at or past K).
    unsigned a_voff[A_LOADS2];
    int a_kp[A_LOADS2];
#pragma unroll
    for (int j = 0; j < A_LOADS2; ++j) {
        const int row = 8 * (wave * A_LOADS2 + j) + lane / 8;
        const int piece = (lane % 8) ^ swz_a<2 * BK>(row);
        a_voff[j] = (m0 + row) < M ? (unsigned)(m0 + row) * (unsigned)K + (unsigned)piece * 16u : kOOB;
        a_kp[j] = piece * 16;
    }
    // B load j of a K-step: as in the kernel above.
    unsigned b_voff[B_LOADS];
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
        const int byte = 1024 * (wave * B_LOADS + j) + lane * 16;
        const int k = byte / ROW_B;
        const int piece = ((byte % ROW_B) / 16) ^ swz_b<BN>(k);
        const int col = n0 + piece * 16;
        b_voff[j] = col < N ? (unsigned)k * (unsigned)N + (unsigned)col : kOOB;
    }
    auto load_a = [&](int p, int k0_in, int j) __attribute__((always_inline)) {
        const int k0 = __builtin_amdgcn_readfirstlane(k0_in);
        const unsigned off = a_kp[j] < K - k0 ? a_voff[j] : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (void __attribute__((address_space(3)))*)(a_slot(p) + (wave * A_LOADS2 + j) * 1024), 16, off,
            k0 < K ? k0 : 0, 0, 0);
    };
    auto load_b = [&](int st, int k0_in, int j) __attribute__((always_inline)) {
        const int k0 = __builtin_amdgcn_readfirstlane(k0_in);
        const int krem = K - k0;
        const int rows = __builtin_amdgcn_readfirstlane(krem < 0 ? 0 : (krem > BK ? BK : krem));
        const __amdgpu_buffer_rsrc_t rbk = make_rsrc(B + (size_t)(k0 < K ? k0 : 0) * N, (unsigned)rows * (unsigned)N);
        const unsigned off = b_voff[j];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rbk, (void __attribute__((address_space(3)))*)(b_stage(st) + (wave * B_LOADS + j) * 1024), 16, off, 0,
            0, 0);
    };

    // Operand reads: A fragment of K-step h of a pair, tile bi: row wm*WM +
    // 32*bi + lane%32, logical pieces 4*h + 2*(lane/32) and the next; B as
    // in the kernel above.
    int a_rd[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 2; ++i)
            a_rd[h][i] = (wm * WM + (lane & 31)) * ROW_P + (((4 * h + 2 * (lane >> 5) + i) ^ swz_a<2 * BK>(lane & 31)) * 16);
    int b_rd[FN];
#pragma unroll
    for (int bj = 0; bj < FN; ++bj) {
        const int G = lane >> 4, r = (lane & 15) >> 1, q = lane & 1;
        const int piece = (wn * WN + 32 * bj + 16 * (G & 1)) / 16;
        b_rd[bj] = (32 * (G >> 1) + r) * ROW_B + ((piece ^ swz_b<BN>(r)) * 16) + 8 * q;
    }
    f32x16 acc[FM][FN];
    u32x8 fa[2][FM], fb[2][FN];
    auto read_frag = [&](int set, int slot, int h, int stb, int o) __attribute__((always_inline)) {
        if (o < FN) {
            const lds_byte* p = b_stage(stb) + b_rd[o];
            i32x2 hh[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                hh[i] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (i32x2 __attribute__((address_space(3)))*)(p + 8 * i * ROW_B));
            const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_shufflevector(hh[0], hh[1], 0, 1, 2, 3));
            const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_shufflevector(hh[2], hh[3], 0, 1, 2, 3));
            fb[set][o] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
            const lds_byte* base = a_slot(slot) + (o - FN) * 32 * ROW_P;
            const u32x4 lo = *(const u32x4 __attribute__((address_space(3)))*)(base + a_rd[h][0]);
            const u32x4 hi = *(const u32x4 __attribute__((address_space(3)))*)(base + a_rd[h][1]);
            fa[set][o - FN] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };

    // ---- prologue: what K-steps -3 .. -1 would have issued (the A pair of
    // K-steps 0, 1; B of K-steps 0, 1, 2; the first half of the A pair of
    // K-steps 2, 3), then K-step 0's operands.
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
    // half's loads and the operand reads of K-step it+1.
    auto kstep = [&](auto q_c, int it, const bool first) __attribute__((always_inline)) {
        constexpr int q = decltype(q_c)::value;
        constexpr int set = q & 1;
        constexpr int n1 = (q & 1) ? B_LOADS : AH;
        constexpr int n2 = (q & 1) ? AH : B_LOADS;
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
                MfmaFp8<FMT>::first(acc[x / FN][x % FN], fb[set][x % FN], fa[set][x / FN]);
            else
                MfmaFp8<FMT>::acc(acc[x / FN][x % FN], fb[set][x % FN], fa[set][x / FN]);
        };
#pragma unroll
        for (int x = 0; x < BAR; ++x) {
            mfma(x);
#pragma unroll
            for (int o = op_lo(x, n1, BAR); o < op_lo(x + 1, n1, BAR); ++o) load1(o);
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kWaitBar);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        constexpr int nops2 = n2 + NR;
#pragma unroll
        for (int x = BAR; x < NT; ++x) {
            mfma(x);
#pragma unroll
            for (int o = op_lo(x - BAR, nops2, NT - BAR); o < op_lo(x + 1 - BAR, nops2, NT - BAR); ++o) {
                const int nld = (o * n2) / nops2 + 1;
                if (o == 0 || (o * n2) / nops2 != ((o - 1) * n2) / nops2)
                    load2(nld - 1);
                else
                    read_frag(set ^ 1, ((q + 1) / 2) % 2, (q + 1) & 1, (q + 1) % 4, o - nld);
            }
        }
    };
    using Q0 = std::integral_constant<int, 0>;
    using Q1 = std::integral_constant<int, 1>;
    using Q2 = std::integral_constant<int, 2>;
    using Q3 = std::integral_constant<int, 3>;
    const int nk = cdiv_i(cdiv_i(K, BK), 4) * 4;
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

    // ---- epilogue: as in the kernel above
    static_assert(FN == 4, "the wait below lists the last row's tiles");
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[FM - 1][0]), "+a"(acc[FM - 1][1]), "+a"(acc[FM - 1][2]), "+a"(acc[FM - 1][3]));
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    constexpr int BLOCK = WM * WN * 2;
    constexpr int CWB = B_BYTES < BLOCK ? B_BYTES : BLOCK;
    constexpr int CW = WM % (CWB / (WN * 2)) == 0 ? CWB : 32 * WN * 2;
    store_c_block_32x32<__bf16, WM, WN, CW>(acc, b_stage(wave), lane, m0 + wm * WM, n0 + wn * WN, M, N, C);
    clock_sample(clk, 1);
}

// 128-deep K-steps on 16 x 16 x 128 MFMAs (256 x 256 and 192 x 256 tiles,
// one product per workgroup, no split).  Each wavefront owns WM x 128 of the
// tile as (WM/16) x 8 tiles of 16 x 16; one K-step is (WM/16) x 8 MFMAs,
// issued row of tiles by row of tiles.  Half the accumulator data per FLOP
// of the 32 x 32 x 64 form lets the board hold a higher clock under its
// power limit (E4M3 4096^3 on MI355X: 2.0-2.1 against 1.85 GHz), which
// outweighs the lower share of cycles it keeps the MFMA pipe busy: 2-5 %
// less time than the A-pair kernel above on 3072^3 .. 8192^3.
//  * LDS: two A slots of [BM][128 B] (128-byte rows, pieces XOR-ed by
//    (row/2)%8) and two B stages of [128][BN] (256-byte rows, piece p of row
//    k at p ^ (2*(k%8) + (k/32)%2)); K-step t in slot and stage t%2.
//  * Registers: the B fragments of a K-step stay in one of two register
//    sets for the whole K-step; A fragments are read two rows of tiles
//    ahead of their MFMAs; the transpose reads of the next K-step's B
//    fragments are spread one or two per MFMA.
//  * K-step t: rows 0 .. MB-1 issue the A loads of K-step t+1 (into the
//    other slot, free since barrier E(t-1)); barrier M(t) once the B
//    loads of K-step t+1 have landed; rows MB .. FM-1 issue the B loads of
//    K-step t+2 (into this K-step's stage, whose fragments were read before
//    M(t)) and read the B fragments of K-step t+1; barrier E(t) after row
//    FM-2, once the A loads of K-step t+1 have landed and this K-step's A
//    reads are done; row FM-1 reads A fragments 0 and 1 of K-step t+1.
template <int FMT, int BM, int BN>
__global__ __launch_bounds__(256, 1) void gemm_fp8_k128_kernel(const unsigned char* A, const unsigned char* B,
                                                               __bf16* C, int M, int N, int K, int group_m,
                                                               int xcd_remap, Batch bt, unsigned long long* clk)
{
    clock_sample(clk, 0);
    constexpr int NW = 4, BK = 128;
    constexpr int WM = BM / 2, WN = BN / 2;      // per-wavefront block (2 x 2 wavefronts)
    constexpr int FM = WM / 16, FN = WN / 16;    // 16x16 tiles per wavefront
    constexpr int MB = FM / 2 - 1;               // rows of tiles before barrier M
    constexpr int ROW_A = BK;
    constexpr int A_BYTES = BM * ROW_A;
    constexpr int ROW_B = BN;
    constexpr int B_BYTES = BK * ROW_B;
    constexpr int A_LOADS = A_BYTES / 1024 / NW;   // A loads per wavefront per K-step
    constexpr int B_LOADS = B_BYTES / 1024 / NW;   // B loads per wavefront per K-step
    constexpr int NX = MB * FN;                    // MFMAs before barrier M
    constexpr int NY = (FM - MB) * FN;             // MFMAs after it
    constexpr int NYE = (FM - 1 - MB) * FN;        // ... of them before barrier E
    static_assert((BM == 256 || BM == 192) && BN == 256, "tile");
    static_assert(2 * A_BYTES + 2 * B_BYTES <= 160 * 1024, "LDS");
    static_assert(FM - 1 > MB + 1, "A reads of the last rows must precede barrier E");
    __shared__ __attribute__((aligned(1024))) unsigned char sa0[A_BYTES], sa1[A_BYTES];
    __shared__ __attribute__((aligned(1024))) unsigned char sb0[B_BYTES], sb1[B_BYTES];
    auto a_slot = [&](int p) __attribute__((always_inline)) { return (lds_byte*)(p == 0 ? sa0 : sa1); };
    auto b_stage = [&](int p) __attribute__((always_inline)) { return (lds_byte*)(p == 0 ? sb0 : sb1); };
    auto swz_b16 = [](int k) __attribute__((always_inline)) { return 2 * (k & 7) + ((k >> 5) & 1); };

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
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (unsigned)M * (unsigned)K);

    // A load j: 8 rows of 128 bytes; lane -> row 8*(wave*A_LOADS + j) +
    // lane/8, physical piece lane%8 holding logical piece (lane%8) ^
    // swz_a<128>(row) (kOOB for rows >= M and pieces at or past K).
    unsigned a_voff[A_LOADS];
    int a_kp[A_LOADS];
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
        const int row = 8 * (wave * A_LOADS + j) + lane / 8;
        const int piece = (lane % 8) ^ swz_a<BK>(row);
        a_voff[j] = (m0 + row) < M ? (unsigned)(m0 + row) * (unsigned)K + (unsigned)piece * 16u : kOOB;
        a_kp[j] = piece * 16;
    }
    // B load j: 4 rows of 256 bytes; lane -> row k = byte/256 of the K-step,
    // physical piece (byte%256)/16 holding columns n0 + 16*(piece ^
    // swz_b16(k)) .. +15 (kOOB past N; rows past K lie outside the range of
    // the K-step's buffer resource).
    unsigned b_voff[B_LOADS];
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
        const int byte = 1024 * (wave * B_LOADS + j) + lane * 16;
        const int k = byte / ROW_B;
        const int piece = ((byte % ROW_B) / 16) ^ swz_b16(k);
        const int col = n0 + piece * 16;
        b_voff[j] = col < N ? (unsigned)k * (unsigned)N + (unsigned)col : kOOB;
    }
    auto load_a = [&](int p, int k0_in, int j) __attribute__((always_inline)) {
        const int k0 = __builtin_amdgcn_readfirstlane(k0_in);
        const unsigned off = a_kp[j] < K - k0 ? a_voff[j] : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (void __attribute__((address_space(3)))*)(a_slot(p) + (wave * A_LOADS + j) * 1024), 16, off,
            k0 < K ? k0 : 0, 0, 0);
    };
    auto load_b = [&](int p, int k0_in, int j) __attribute__((always_inline)) {
        const int k0 = __builtin_amdgcn_readfirstlane(k0_in);
        const int krem = K - k0;
        const int rows = __builtin_amdgcn_readfirstlane(krem < 0 ? 0 : (krem > BK ? BK : krem));
        const __amdgpu_buffer_rsrc_t rbk = make_rsrc(B + (size_t)(k0 < K ? k0 : 0) * N, (unsigned)rows * (unsigned)N);
        const unsigned off = b_voff[j];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rbk, (void __attribute__((address_space(3)))*)(b_stage(p) + (wave * B_LOADS + j) * 1024), 16, off, 0, 0,
            0);
    };

    // A fragment of tile row i: row wm*WM + 16*i + lane%16, logical pieces
    // 2*(lane/16) and the next (K 32*(lane/16) .. +31); the swizzle depends
    // on lane%16 only, so row i is 16*i rows further.
    int a_rd[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        a_rd[h] = (wm * WM + (lane & 15)) * ROW_A + (((2 * (lane >> 4) + h) ^ swz_a<BK>(lane & 15)) * 16);
    // B fragment of tile column j: four transpose reads of 8 rows x 16
    // columns; lane -> column wn*WN + 16*j + lane%16, K 32*(lane/16) .. +31
    // (read i covers K 32*(lane/16) + 8*i .. +7, one row further by 8).
    int b_rd[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int k = 32 * (lane >> 4) + ((lane & 15) >> 1);
        const int piece = (wn * WN + 16 * j) / 16;
        b_rd[j] = k * ROW_B + ((piece ^ swz_b16(k)) * 16) + 8 * (lane & 1);
    }
    f32x4 acc[FM][FN];
    u32x8 fa[FM], fb[2][FN];
    auto read_a = [&](int slot, int i) __attribute__((always_inline)) {
        const lds_byte* base = a_slot(slot) + i * 16 * ROW_A;
        const u32x4 lo = *(const u32x4 __attribute__((address_space(3)))*)(base + a_rd[0]);
        const u32x4 hi = *(const u32x4 __attribute__((address_space(3)))*)(base + a_rd[1]);
        fa[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // part i (K 32*(lane/16) + 8*i .. +7) of the B fragment of tile column j
    auto read_b = [&](int set, int stage, int j, int i) __attribute__((always_inline)) {
        const lds_byte* p = b_stage(stage) + b_rd[j] + 8 * i * ROW_B;
        const u32x2 h = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 __attribute__((address_space(3)))*)p));
        fb[set][j][2 * i] = h.x;
        fb[set][j][2 * i + 1] = h.y;
    };

    // ---- prologue: the A and B loads of K-step 0, the B loads of K-step 1;
    // once K-step 0's have landed, its B fragments and A fragments 0 and 1.
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) load_a(0, 0, j);
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) load_b(0, 0, j);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) load_b(1, BK, j);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(B_LOADS));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int r = 0; r < 4 * FN; ++r) read_b(0, 0, r / 4, r % 4);
    read_a(0, 0);
    read_a(0, 1);

    auto op_lo = [](int pos, int n, int span) __attribute__((always_inline)) { return (pos * n + span - 1) / span; };
    // K-step t, s = t % 2 (slot, stage and B register set of K-step t).
    auto kstep = [&](auto s_c, int t, auto first_c) __attribute__((always_inline)) {
        constexpr int s = decltype(s_c)::value;
        constexpr bool first = decltype(first_c)::value;
        // B loads of K-step t+2 issued before barrier E
        constexpr int NBE = op_lo(NYE, B_LOADS, NY);
        // The 4*FN transpose reads of K-step t+1's B fragments, spread over
        // the NY MFMAs after barrier M (read r: fragment r/4, part r%4).
        constexpr int NBR = 4 * FN;
        // LDS reads each barrier must see completed: at M, every read of
        // this K-step's B stage (issued before the MB A-fragment reads of
        // rows 0 .. MB-1, two operations each); at E, every read of this
        // K-step's A slot (the last, fragment FM-1, at MFMA YA after M; after
        // it only B reads, those of MFMAs YA+1 .. NYE-1).  LDS operations
        // complete in order.
        constexpr int YA = (FM - 3 - MB) * FN + FN / 2;
        constexpr int NRE = op_lo(NYE, NBR, NY) - op_lo(YA + 1, NBR, NY);
        constexpr unsigned kLgkmM = waitcnt_lgkm(2 * MB);
        constexpr unsigned kLgkmE = waitcnt_lgkm(NRE);
        auto mfma = [&](int i, int j) __attribute__((always_inline)) {
            if constexpr (first)
                MfmaFp8x16<FMT>::first(acc[i][j], fb[s][j], fa[i]);
            else
                MfmaFp8x16<FMT>::acc(acc[i][j], fb[s][j], fa[i]);
        };
        // rows 0 .. MB-1: the A loads of K-step t+1; A fragments 2 .. MB+1
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int x = i * FN + j;
                mfma(i, j);
#pragma unroll
                for (int o = op_lo(x, A_LOADS, NX); o < op_lo(x + 1, A_LOADS, NX); ++o)
                    load_a(s ^ 1, (t + 1) * BK, o);
                if (j == FN / 2) read_a(s, i + 2);
            }
        // barrier M: the B loads of K-step t+1 have landed (only the A loads
        // above are still in flight)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(A_LOADS));
        __builtin_amdgcn_s_waitcnt(kLgkmM);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        // rows MB .. FM-1: the B loads of K-step t+2, the B fragments of
        // K-step t+1, A fragments MB+2 .. FM-1; barrier E before row FM-1,
        // whose reads are A fragments 0, 1 of K-step t+1
#pragma unroll
        for (int i = MB; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int y = (i - MB) * FN + j;
                if (y == NYE) {
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm(NBE));
                    __builtin_amdgcn_s_waitcnt(kLgkmE);
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                }
                mfma(i, j);
#pragma unroll
                for (int o = op_lo(y, B_LOADS, NY); o < op_lo(y + 1, B_LOADS, NY); ++o)
                    load_b(s, (t + 2) * BK, o);
                // the B fragments of K-step t+1, a transpose read or two
                // per MFMA
#pragma unroll
                for (int r = op_lo(y, NBR, NY); r < op_lo(y + 1, NBR, NY); ++r) read_b(s ^ 1, s ^ 1, r / 4, r % 4);
                if (j == FN / 2 && i + 2 < FM) read_a(s, i + 2);
                if (i == FM - 1 && j == 0) read_a(s ^ 1, 0);
                if (i == FM - 1 && j == FN / 2) read_a(s ^ 1, 1);
            }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    const int nk = cdiv_i(cdiv_i(K, BK), 2) * 2;
    kstep(S0{}, 0, std::true_type{});
    kstep(S1{}, 1, std::false_type{});
    for (int t = 2; t < nk; t += 2) {
        kstep(S0{}, t, std::false_type{});
        kstep(S1{}, t + 1, std::false_type{});
    }

    // ---- epilogue: the last row of tiles was written by the most recent
    // MFMAs; each wavefront stages its block through a slot or stage of its
    // own
    static_assert(FN == 8, "the wait below lists the last row's tiles");
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[FM - 1][0]), "+a"(acc[FM - 1][1]), "+a"(acc[FM - 1][2]), "+a"(acc[FM - 1][3]),
                   "+a"(acc[FM - 1][4]), "+a"(acc[FM - 1][5]), "+a"(acc[FM - 1][6]), "+a"(acc[FM - 1][7]));
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    constexpr int CW = A_BYTES < WM * WN * 2 ? A_BYTES : WM * WN * 2;
    lds_byte* cw = wave < 2 ? a_slot(wave) : b_stage(wave - 2);
    store_c_block<__bf16, WM, WN, CW>(acc, cw, lane, m0 + wm * WM, n0 + wn * WN, M, N, C);
    clock_sample(clk, 1);
}

template <int FMT>
hipError_t launch_fmt(const Config& cfg, const LaunchArgs& a)
{
    const int tiles = cdiv_i(a.M, cfg.bm) * cdiv_i(a.N, cfg.bn);
    const dim3 grid(tiles * a.batch.count), block(256);
    const unsigned char* A = static_cast<const unsigned char*>(a.A);
    const unsigned char* B = static_cast<const unsigned char*>(a.B);
    __bf16* C = static_cast<__bf16*>(a.C);
    if (cfg.threads != 256) return hipErrorInvalidValue;
    if (cfg.sched == 3) {   // 128-deep K-steps on 16 x 16 x 128 MFMAs: 256 x 256 or 192 x 256, one pass only
        if (a.splits > 1 || cfg.bn != 256 || cfg.bk != 128) return hipErrorInvalidValue;
        if (cfg.bm == 256)
            hipLaunchKernelGGL((gemm_fp8_k128_kernel<FMT, 256, 256>), grid, block, 0, a.stream, A, B, C, a.M, a.N,
                               a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.clk);
        else if (cfg.bm == 192)
            hipLaunchKernelGGL((gemm_fp8_k128_kernel<FMT, 192, 256>), grid, block, 0, a.stream, A, B, C, a.M, a.N,
                               a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.clk);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
    if (cfg.sched == 2) {   // A staged two K-steps at a time: 256 x 256 or 192 x 256, one pass only
        if (a.splits > 1 || cfg.bn != 256 || cfg.bk != 64) return hipErrorInvalidValue;
        if (cfg.bm == 256)
            hipLaunchKernelGGL((gemm_fp8_pair_kernel<FMT, 256, 256>), grid, block, 0, a.stream, A, B, C, a.M, a.N,
                               a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.clk);
        else if (cfg.bm == 192)
            hipLaunchKernelGGL((gemm_fp8_pair_kernel<FMT, 192, 256>), grid, block, 0, a.stream, A, B, C, a.M, a.N,
                               a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.clk);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
    if (cfg.sched == 1) {   // A direct to LDS as well; split K at 128 x 128 and 64 x 128 only
        if (a.splits > 1) {
            if (cfg.bm == 128 && cfg.bn == 128 && cfg.bk == 64)
                hipLaunchKernelGGL((gemm_fp8_kernel<FMT, 128, 128, 64, true, true>), dim3(tiles * a.splits), block,
                                   0, a.stream, A, B, C, a.M, a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.ws, a.splits, a.clk);
            else if (cfg.bm == 64 && cfg.bn == 128 && cfg.bk == 64)
                hipLaunchKernelGGL((gemm_fp8_kernel<FMT, 64, 128, 64, true, true>), dim3(tiles * a.splits), block,
                                   0, a.stream, A, B, C, a.M, a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.ws, a.splits, a.clk);
            else
                return hipErrorInvalidValue;
            return hipGetLastError();
        }
        if (cfg.bm == 256 && cfg.bn == 256 && cfg.bk == 64)
            hipLaunchKernelGGL((gemm_fp8_kernel<FMT, 256, 256, 64, false, true>), grid, block, 0, a.stream, A, B, C,
                               a.M, a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.ws, 1, a.clk);
        else if (cfg.bm == 128 && cfg.bn == 128 && cfg.bk == 64)
            hipLaunchKernelGGL((gemm_fp8_kernel<FMT, 128, 128, 64, false, true>), grid, block, 0, a.stream, A, B, C,
                               a.M, a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.ws, 1, a.clk);
        else if (cfg.bm == 64 && cfg.bn == 128 && cfg.bk == 64)
            hipLaunchKernelGGL((gemm_fp8_kernel<FMT, 64, 128, 64, false, true>), grid, block, 0, a.stream, A, B, C,
                               a.M, a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.ws, 1, a.clk);
        else if (cfg.bm == 192 && cfg.bn == 256 && cfg.bk == 64)
            hipLaunchKernelGGL((gemm_fp8_kernel<FMT, 192, 256, 64, false, true>), grid, block, 0, a.stream, A, B, C,
                               a.M, a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.ws, 1, a.clk);
        else
            return hipErrorInvalidValue;
        return hipGetLastError();
    }
#define DGR_FP8(BM_, BN_, BK_)                                                                            \
    else if (cfg.bm == BM_ && cfg.bn == BN_ && cfg.bk == BK_) {                                          \
        if (a.splits > 1)                                                                                \
            hipLaunchKernelGGL((gemm_fp8_kernel<FMT, BM_, BN_, BK_, true>), dim3(tiles * a.splits), block, 0, \
                               a.stream, A, B, C, a.M, a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.ws, a.splits, a.clk);  \
        else                                                                                             \
            hipLaunchKernelGGL((gemm_fp8_kernel<FMT, BM_, BN_, BK_, false>), grid, block, 0, a.stream, A, B, C, \
                               a.M, a.N, a.K, cfg.group_m, cfg.xcd_remap, a.batch, a.ws, 1, a.clk);                            \
    }
    if (false) {}
    DGR_FP8(256, 256, 64)
    DGR_FP8(256, 256, 128)
    DGR_FP8(128, 128, 64)
    DGR_FP8(128, 128, 128)
    else
        return hipErrorInvalidValue;
#undef DGR_FP8
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8(const Config& cfg, const LaunchArgs& a)
{
    if (a.dtype == kFP8E4M3) return launch_fmt<0>(cfg, a);
    if (a.dtype == kFP8E5M2) return launch_fmt<1>(cfg, a);
    return hipErrorInvalidValue;
}

}  // namespace dgr
