// Few-row products: C = A·B with small M (a batch of tokens against a weight
// matrix B [K, N]), fp16/bf16 or 8-bit (E4M3 / E5M2, bf16 C) inputs, rows
// 16-byte aligned (K and N multiples of 16 bytes of A's and B's rows, N a
// multiple of 8, A, B and C 16-byte aligned).
//
// With few rows of A, every element of B is used M times at most, so the
// product is bound by streaming B from HBM (arithmetic intensity about M
// FLOP per byte, below the MI355X ridge for M < 300), and the tiled kernels
// leave most CUs idle: they have only ceil(N/BN) output tiles.  Like the
// matrix-vector kernel (chapter "Fast matrix multiplication", section "Decode
// is a different problem: GEMV": coalesced 16-byte loads, enough parallelism,
// partial sums combined at the end), this kernel is organised around the
// stream of B:
//
//  * one workgroup of W wavefronts owns BMS rows of A (all of M, normally)
//    and a strip of BN = 16 or 32 columns, so there are N/BN workgroups;
//  * the wavefronts split the K walk: wavefront w takes K-steps w, w+W, ...
//    (BK = 32 or 64 K each), so at any time the wavefronts of a workgroup,
//    and the workgroups of neighbouring strips, read nearby rows of B;
//  * each wavefront streams its K-steps of the B strip straight into a ring
//    of 7 LDS stages of its own (buffer loads with the LDS destination), 7
//    K-steps ahead, and never waits for another wavefront until the end; the
//    A fragments (16 rows x 32 K per 16x16 tile and K-slice) come straight
//    from global memory into registers 4 K-steps ahead (A is small and stays
//    in the L2 cache, so a shorter lead covers it, and fewer registers hold
//    it);
//  * the MFMA is v_mfma_f32_16x16x32 for 16-bit inputs and
//    v_mfma_f32_16x16x128_f8f6f4 for 8-bit ones (compiler builtins), given
//    the B fragment first (transpose reads: each lane gets 8 consecutive K
//    of one column from a 16-bit read pair, or 32 from four 8-bit reads), so
//    each lane accumulates 4 consecutive columns of one row;
//  * at the end the partial sums of the wavefronts are added through LDS,
//    rounded (nearest even) and stored, skipping rows >= M.
// Out-of-range pieces read zeros through the buffer range check, as in the
// tiled kernels; workgroups are ordered so that the strips one XCD runs are
// adjacent (they share the cache lines of B rows), and, where M takes two
// row blocks, so that both row blocks of a strip run on one XCD (band height
// 2: they read the same B strip through one L2).
#include "gemm_internal.h"
#include "gemm_device.h"

namespace dgr {
namespace {

// LDS stages per wavefront (K-steps of B in flight).  Each stage is an LDS
// object of its own, so that the compiler's tracking of direct-to-LDS loads
// can tell them apart; it keeps 7 such objects apart (with 8 it merged some
// and waited for loads issued 3 K-steps earlier).
constexpr int kStages = 7;
constexpr int kLeadA = 4;   // K-steps of A fragments in flight

template <int N> struct Steps {
    static constexpr int value = N;
};

// f(Steps<I>{}) for I = B .. E-1, in order.
template <int B, int E, typename F> __device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (B < E) {
        f(Steps<B>{});
        static_for<B + 1, E>(f);
    }
}

// Loads the prologue issues after the B loads of K-step t (t < kStages): B of
// the kStages-1-t later virtual steps, and A of those virtual steps (that of
// step t's own one included) that have an A part.
constexpr int after_prologue(int t, int b_loads, int a_loads)
{
    return (kStages - 1 - t) * b_loads + (kStages - t < kLeadA ? kStages - t : kLeadA) * a_loads;
}

// Element types of A and B.  Per lane, an MFMA operand fragment is FRAG
// bytes of one row of A (or column of B): KI consecutive K.  c += b-fragment
// x a-fragment.  The compiler's builtins, not inline assembly: the tails of
// this kernel merge into one epilogue, and the compiler copies accumulators
// there; it only waits out the MFMA latency before such copies when it knows
// the instruction is an MFMA.
typedef unsigned u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
struct E4M3 {};
struct E5M2 {};
template <typename E> struct Elem;
template <> struct Elem<_Float16> {
    using Out = _Float16;
    using Frag = u32x4;
    static constexpr int BYTES = 2, KI = 32;
    static __device__ __forceinline__ void mma(f32x4& c, const Frag& b, const Frag& a)
    {
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, b), __builtin_bit_cast(f16x8, a), c, 0,
                                                   0, 0);
    }
};
template <> struct Elem<__bf16> {
    using Out = __bf16;
    using Frag = u32x4;
    static constexpr int BYTES = 2, KI = 32;
    static __device__ __forceinline__ void mma(f32x4& c, const Frag& b, const Frag& a)
    {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, a), c,
                                                    0, 0, 0);
    }
};
// 8-bit: operand format 0 = E4M3, 1 = E5M2 for both operands; the scale
// operands are 0, which the compiler emits as the unscaled instruction.
template <int FMT> struct Elem8 {
    using Out = __bf16;
    using Frag = u32x8;
    static constexpr int BYTES = 1, KI = 128;
    static __device__ __forceinline__ void mma(f32x4& c, const Frag& b, const Frag& a)
    {
        c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(__builtin_bit_cast(i32x8, b),
                                                              __builtin_bit_cast(i32x8, a), c, FMT, FMT, 0, 0, 0, 0);
    }
};
template <> struct Elem<E4M3> : Elem8<0> {};
template <> struct Elem<E5M2> : Elem8<1> {};

template <typename E, int BMS, int BN, int BK, int W>
__global__ __launch_bounds__(64 * W, 1) void gemm_skinny_kernel(const unsigned char* A, const unsigned char* B,
                                                              typename Elem<E>::Out* C, int M, int N, int K,
                                                              int group_m, Batch bt)
{
    using Frag = typename Elem<E>::Frag;
    using Out = typename Elem<E>::Out;
    constexpr int ES = Elem<E>::BYTES;               // bytes per element of A and B
    constexpr int KI = Elem<E>::KI;                  // K per MFMA
    constexpr int FRAG = (int)sizeof(Frag);          // fragment bytes per lane (KI/4 * ES)
    constexpr int FM = BMS / 16, FN = BN / 16;       // 16x16 tiles
    constexpr int NS = BK / KI;                      // K-slices per K-step
    constexpr int ROW_B = BN * ES;                   // bytes of one B row in LDS
    constexpr int STEP_B = BK * ROW_B;               // bytes of one K-step of B
    constexpr int B_LOADS = STEP_B / 1024;           // direct-to-LDS loads per K-step
    constexpr int AP = FRAG / 16;                    // 16-byte loads per A fragment
    constexpr int A_LOADS = NS * FM * AP;            // A loads per K-step
    constexpr int L = B_LOADS + A_LOADS;             // vector-memory instructions per K-step
    // The transpose reads of a half-wavefront take rows r.. of two row
    // groups that land on the same banks (16-bit: rows k and k+8, 4 rows per
    // group; 8-bit: rows k and k+32, 8 rows per group): rows with that row
    // bit set are XOR-ed by half of the bank span a group touches.
    constexpr int SWZ_BIT = ES == 2 ? 8 : 32;
    constexpr int SWZ = BN == 16 ? 128 : (ES == 2 ? 32 : 16);
    static_assert(BN == 16 || BN == 32, "strip width");
    static_assert(BK % KI == 0 && (BK == KI || BK == 2 * KI), "K-step");
    static_assert(BMS % 16 == 0 && BMS <= 64, "rows");
    static_assert(STEP_B % 1024 == 0, "a K-step of B is whole 1 KB loads");
    static_assert(kStages * L <= 63, "loads in flight must fit the vmcnt field");
    static_assert(kStages * W * STEP_B <= 160 * 1024, "LDS");
    static_assert(BMS * BN * 4 <= kStages * STEP_B, "partial sums must fit a wavefront's slices of the stages");
    static_assert(kStages == 7, "one LDS object per stage below");
    __shared__ __attribute__((aligned(1024))) unsigned char s0[W * STEP_B], s1[W * STEP_B], s2[W * STEP_B],
        s3[W * STEP_B], s4[W * STEP_B], s5[W * STEP_B], s6[W * STEP_B];
    auto stage = [&](int st) __attribute__((always_inline)) {
        return (lds_byte*)(st == 0 ? s0 : st == 1 ? s1 : st == 2 ? s2 : st == 3 ? s3 : st == 4 ? s4 : st == 5 ? s5 : s6);
    };

    const int tiles_m = cdiv_i(M, BMS), tiles_n = cdiv_i(N, BN);
    int b, tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, bt.count, group_m, true, b, tm, tn);
    A += b * bt.sa * ES;
    B += b * bt.sb * ES;
    C += b * bt.sc;
    const int m0 = tm * BMS, n0 = tn * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (unsigned)M * (unsigned)K * ES);

    // A fragment of tile mi, K-slice s: lane -> row m0 + 16*mi + lane%16, K
    // KI*s + (KI/4)*(lane/16) .. of the step, AP pieces of 16 bytes (kOOB for
    // rows >= M; pieces at or past K per step).
    unsigned a_voff[FM];
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) {
        const int m = m0 + 16 * mi + (lane & 15);
        a_voff[mi] = m < M ? (unsigned)m * (unsigned)K * ES + (unsigned)(FRAG * (lane >> 4)) : kOOB;
    }
    // B load j of a step: lane -> LDS byte p = 1024*j + 16*lane of the stage
    // slice, holding logical byte p ^ swizzle = row k, 16-byte piece c:
    // global k*N*ES + n0*ES + 16c relative to the step's first row (kOOB past N).
    unsigned b_voff[B_LOADS];
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
        const int p = 1024 * j + 16 * lane;
        const int lg = p ^ (((p / ROW_B) & SWZ_BIT) ? SWZ : 0);
        const int k = lg / ROW_B, c = (lg % ROW_B) / 16;
        const int col = n0 + c * (16 / ES);
        b_voff[j] = col < N ? ((unsigned)k * (unsigned)N + (unsigned)col) * ES : kOOB;
    }
    // B fragment of tile ni, K-slice s by transpose reads (RD of them):
    //  16-bit: in 16-lane group g, lane 4r+q points at rows KI*s + 8g + 4h + r
    //    (h = 0, 1), columns 16*ni + 4q .. +3: lane i gets column i over 4 rows;
    //  8-bit: in 16-lane group g, lane 2r+q points at rows KI*s + 32g + 8h + r
    //    (h = 0..3), bytes 8q .. 8q+7 of the 16 columns of tile ni: lane i gets
    //    column i over 8 rows.
    constexpr int RD = ES == 2 ? 2 : 4;
    int b_rd[FN][RD];
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
#pragma unroll
        for (int h = 0; h < RD; ++h) {
            int k, byte;
            if constexpr (ES == 2) {
                k = 8 * (lane >> 4) + 4 * h + ((lane & 15) >> 2);
                byte = (16 * ni + 4 * (lane & 3)) * 2;
            } else {
                k = 32 * (lane >> 4) + 8 * h + ((lane & 15) >> 1);
                byte = 16 * ni + 8 * (lane & 1);
            }
            const int lg = k * ROW_B + byte;
            b_rd[ni][h] = lg ^ ((k & SWZ_BIT) ? SWZ : 0);
        }

    const int nsteps = cdiv_i(K, BK);
    const int per_wave = cdiv_i(nsteps, W);   // K-steps of every wavefront (those past K read zeros)

    // B of K-step j of this wavefront (global K-step wave + W*j) -> stage st.
    auto issue_b = [&](int st, int j) __attribute__((always_inline)) {
        const int k0 = __builtin_amdgcn_readfirstlane((wave + W * j) * BK);
        const int krem = K - k0;
        const int rows = __builtin_amdgcn_readfirstlane(krem < 0 ? 0 : (krem > BK ? BK : krem));
        const __amdgpu_buffer_rsrc_t rbk =
            make_rsrc(B + (size_t)(k0 < K ? k0 : 0) * N * ES, (unsigned)rows * (unsigned)N * ES);
#pragma unroll
        for (int l = 0; l < B_LOADS; ++l) {
            const unsigned off = b_voff[l];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rbk, (void __attribute__((address_space(3)))*)(stage(st) + wave * STEP_B + 1024 * l), 16, off, 0, 0,
                0);
        }
        asm volatile("" ::: "memory");
    };
    Frag areg[kStages][NS][FM];
    // A fragments of K-step j -> slot sl.  Pieces at or past K read zeros:
    // their offset is forced to kOOB with a mask (a select here became a
    // branch around the load).
    auto issue_a = [&](int sl, int j) __attribute__((always_inline)) {
        const int k0 = __builtin_amdgcn_readfirstlane((wave + W * j) * BK);
        const int krem = K - k0;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int mi = 0; mi < FM; ++mi) {
                u32x4 piece[AP];
#pragma unroll
                for (int h = 0; h < AP; ++h) {
                    const int kk = KI * s + (KI / 4) * (lane >> 4) + (16 / ES) * h;   // first K of the piece
                    const unsigned past = 0u - (unsigned)(kk >= krem);
                    const unsigned off = (a_voff[mi] + (unsigned)((KI * s + (16 / ES) * h) * ES)) | (past & kOOB);
                    piece[h] = __builtin_bit_cast(
                        u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, off, (k0 < K ? k0 : 0) * ES, 0));
                }
                if constexpr (AP == 1)
                    areg[sl][s][mi] = __builtin_bit_cast(Frag, piece[0]);
                else
                    areg[sl][s][mi] = __builtin_bit_cast(Frag, __builtin_shufflevector(piece[0], piece[1], 0, 1, 2, 3, 4, 5, 6, 7));
            }
        asm volatile("" ::: "memory");
    };
    // Fragment of tile ni, K-slice s from stage st.
    auto read_b = [&](int st, int s, int ni) __attribute__((always_inline)) -> Frag {
        const lds_byte* base = stage(st) + wave * STEP_B + KI * s * ROW_B;
        if constexpr (ES == 2) {
            const s16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (s16x4 __attribute__((address_space(3)))*)(base + b_rd[ni][0]));
            const s16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (s16x4 __attribute__((address_space(3)))*)(base + b_rd[ni][1]));
            return __builtin_bit_cast(Frag, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            i32x2 h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                h[i] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 __attribute__((address_space(3)))*)(base + b_rd[ni][i]));
            const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3));
            const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_shufflevector(h[2], h[3], 0, 1, 2, 3));
            return __builtin_bit_cast(Frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };

    f32x4 acc[FN][FM];
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) acc[ni][mi] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Per K-step j (stage and A slot j % kStages): wait until this
    // wavefront's B loads of the step have landed, read the B fragments,
    // multiply, then (refill) load the stage with K-step j+kStages and fetch
    // the A fragments of K-step j+kLeadA, in that order.  The wait counts
    // the loads this wavefront issued after the B loads of step j (each
    // wavefront reads only the stages it filled itself):
    //  * steady state: the A loads issued with them, then kStages-1 steps of
    //    L loads;
    //  * the first round (peeled, straight-line code): what the prologue
    //    issued after them (it issues no A loads for its first
    //    kStages-kLeadA virtual steps) plus t steps of L loads;
    //  * a partial last round issues no B loads; its steps wait as if no
    //    full round had run (the stricter of the two possible histories).
    auto step = [&](const int st, int j, const bool refill, const bool fetch_a, auto count_c)
                    __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(decltype(count_c)::value));
        asm volatile("" ::: "memory");
        Frag bf[NS][FN];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int ni = 0; ni < FN; ++ni) bf[s][ni] = read_b(st, s, ni);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // the stage is read: it may be refilled
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int ni = 0; ni < FN; ++ni)
#pragma unroll
                for (int mi = 0; mi < FM; ++mi) Elem<E>::mma(acc[ni][mi], bf[s][ni], areg[st][s][mi]);
        if (refill) issue_b(st, j + kStages);
        if (refill || fetch_a) issue_a((st + kLeadA) % kStages, j + kLeadA);
    };
    constexpr int kSteady = (kStages - 1) * L + A_LOADS;
    // prologue: virtual steps -kStages .. -1 issue B of step s+kStages and A of
    // step s+kLeadA (when it exists), in the order the steps use
#pragma unroll
    for (int s = -kStages; s < 0; ++s) {
        issue_b(s + kStages, s + kStages);
        if (s + kLeadA >= 0) issue_a(s + kLeadA, s + kLeadA);
    }
    const int full = per_wave / kStages, rem = per_wave - full * kStages;
    if (full > 0) {
        static_for<0, kStages>([&](auto t_c) __attribute__((always_inline)) {
            constexpr int t = decltype(t_c)::value;
            step(t, t, true, true, Steps<after_prologue(t, B_LOADS, A_LOADS) + t * L>{});
        });
        // Full rounds run in a loop with no other exit (an exit inside it
        // made the compiler copy the A slots at the loop head, waiting for
        // their loads).
        for (int r = 1; r < full; ++r)
            static_for<0, kStages>([&](auto t_c) __attribute__((always_inline)) {
                constexpr int t = decltype(t_c)::value;
                step(t, r * kStages + t, true, true, Steps<kSteady>{});
            });
    }
    // the last, partial round of n steps: one of kStages-1 straight-line
    // variants.  It loads no more B, and A only for its own later steps (its
    // steps kLeadA .. n-1 get their A from its steps 0 .. n-1-kLeadA); the
    // loads it adds come after every B load it waits for.
    auto tail = [&](auto n_c) __attribute__((always_inline)) {
        constexpr int n = decltype(n_c)::value;
        static_for<0, n>([&](auto t_c) __attribute__((always_inline)) {
            constexpr int t = decltype(t_c)::value;
            step(t, full * kStages + t, false, t + kLeadA < n, Steps<after_prologue(t, B_LOADS, A_LOADS)>{});
        });
    };
    static_assert(kStages == 7, "the partial rounds below list 1 .. kStages-1 steps");
    switch (rem) {
    case 1: tail(Steps<1>{}); break;
    case 2: tail(Steps<2>{}); break;
    case 3: tail(Steps<3>{}); break;
    case 4: tail(Steps<4>{}); break;
    case 5: tail(Steps<5>{}); break;
    case 6: tail(Steps<6>{}); break;
    default: break;
    }

    // ---- combine the partial sums of the wavefronts through LDS
    // Every load still in flight writes a stage reused below: wait for all.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    // The partial sums of wavefront w, fp32 [BMS][BN] (byte o), go to the
    // wavefront's own slices of the stage objects: chunk o / STEP_B into
    // stage o / STEP_B at w*STEP_B + o % STEP_B (16-byte pieces never
    // straddle a chunk).
    auto part = [&](int w, int o) __attribute__((always_inline)) {
        return (float __attribute__((address_space(3)))*)(stage(o / STEP_B) + w * STEP_B + o % STEP_B);
    };
    // tile (ni, mi): lane l holds row 16*mi + l%16, columns 16*ni + 4*(l/16) .. +3
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) {
            const int m = 16 * mi + (lane & 15), n = 16 * ni + 4 * (lane >> 4);
            *(f32x4 __attribute__((address_space(3)))*)part(wave, (m * BN + n) * 4) = acc[ni][mi];
        }
    __syncthreads();
    // thread t sums 4 consecutive columns of one row over the wavefronts
    for (int e = threadIdx.x; e < BMS * BN / 4; e += 64 * W) {
        const int m = e / (BN / 4), n = 4 * (e % (BN / 4));
        const int o = (m * BN + n) * 4;
        f32x4 sum = *(const f32x4 __attribute__((address_space(3)))*)part(0, o);
#pragma unroll
        for (int w = 1; w < W; ++w) sum += *(const f32x4 __attribute__((address_space(3)))*)part(w, o);
        const int row = m0 + m, col = n0 + n;
        if (row < M && col < N) {
            u32x2 v;
            v[0] = pack2<Out>(sum[0], sum[1]);
            v[1] = pack2<Out>(sum[2], sum[3]);
            *(u32x2*)(C + (size_t)row * N + col) = v;
        }
    }
}

template <typename E>
hipError_t launch_e(const Config& cfg, const LaunchArgs& a)
{
    const int tiles = cdiv_i(a.M, cfg.bm) * cdiv_i(a.N, cfg.bn);
    const unsigned char* A = static_cast<const unsigned char*>(a.A);
    const unsigned char* B = static_cast<const unsigned char*>(a.B);
    auto* C = static_cast<typename Elem<E>::Out*>(a.C);
#define DGR_LAUNCH(BMS_, BN_, BK_, W_)                                                                  \
    if (cfg.bm == BMS_ && cfg.bn == BN_ && cfg.bk == BK_ && cfg.threads == 64 * W_) {                  \
        hipLaunchKernelGGL((gemm_skinny_kernel<E, BMS_, BN_, BK_, W_>), dim3(tiles * a.batch.count),   \
                           dim3(64 * W_), 0, a.stream, A, B, C, a.M, a.N, a.K, cfg.group_m, a.batch);  \
        return hipGetLastError();                                                                      \
    }
    if constexpr (Elem<E>::BYTES == 2) {
        DGR_LAUNCH(16, 16, 64, 8)
        DGR_LAUNCH(32, 16, 64, 8)
        DGR_LAUNCH(64, 16, 32, 4)
        DGR_LAUNCH(16, 32, 64, 4)
        DGR_LAUNCH(32, 32, 64, 4)
        DGR_LAUNCH(64, 32, 32, 4)
        DGR_LAUNCH(16, 16, 32, 8)
        DGR_LAUNCH(16, 16, 32, 16)
        DGR_LAUNCH(16, 32, 32, 8)
    } else {
        DGR_LAUNCH(16, 16, 128, 8)
        DGR_LAUNCH(32, 16, 128, 8)
        DGR_LAUNCH(16, 32, 128, 4)
        DGR_LAUNCH(32, 32, 128, 4)
    }
#undef DGR_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_skinny(const Config& cfg, const LaunchArgs& a)
{
    if (a.dtype == kF16) return launch_e<_Float16>(cfg, a);
    if (a.dtype == kBF16) return launch_e<__bf16>(cfg, a);
    if (a.dtype == kFP8E4M3) return launch_e<E4M3>(cfg, a);
    if (a.dtype == kFP8E5M2) return launch_e<E5M2>(cfg, a);
    return hipErrorInvalidValue;
}

}  // namespace dgr
