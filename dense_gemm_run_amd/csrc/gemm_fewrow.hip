// Few-row products in one launch, with A streamed beside B: C = A·B for a
// few rows of A (up to 128 tokens against a weight matrix B [K, N]),
// fp16/bf16 or 8-bit (E4M3 / E5M2, bf16 C) inputs, rows 16-byte aligned (K
// and N multiples of 16 bytes of A's and B's rows, A, B and C 16-byte
// aligned).
//
// The product is bound by streaming B once from HBM (chapter "Fast matrix
// multiplication", section "Decode is a different problem: GEMV": coalesced
// 16-byte loads, enough parallelism, partial sums combined at the end).  Each
// workgroup owns a strip of BN columns and every K, so each one also needs
// all of its rows of A: 256 strips of a 4096-column B read A 256 times, as
// many bytes as B itself, from the L2 caches.  How those A reads are issued
// decides the speed (load-pattern probes on MI355X, 16 x 4096 x 4096 bf16):
// per-step A fragments loaded straight into registers, every workgroup
// walking K in the same order, took 10.4 us against 5.8 for B alone; A
// loaded by the DMA path into the same LDS stages as B, with each wavefront
// owning a contiguous K range and the workgroups of an XCD starting their
// walks at different K-steps, 7.5-8.1 us.  This kernel is the latter:
//
//  * one workgroup of W wavefronts owns BMS rows (16; 8 for products of at
//    most 8 rows, which then load half the A bytes per K-step; 32 or 64 for
//    more rows, as 2 or 4 rows of 16x16 tiles) and a strip of BN columns of
//    C;
//  * wavefront w owns the contiguous K-steps [w*S, (w+1)*S) and walks them
//    starting at a step that depends on the strip (so neighbouring
//    workgroups read different columns of A and rows of B at any moment);
//  * each K-step's B rows (BK x BN) and A columns (BMS x BK) go global -> LDS
//    by buffer loads with the LDS destination into a ring of NSTG stages of
//    the wavefront's own, NSTG-1 K-steps ahead; the wavefront never waits for
//    another until the end;
//  * the MFMA is v_mfma_f32_16x16x32 (16-bit) or v_mfma_f32_16x16x128_f8f6f4
//    (8-bit) with the B fragment first (transpose reads: each lane gets KI/4
//    consecutive K of one column), so each lane accumulates 4 consecutive
//    columns of one row;
//  * at the end the partial sums of the wavefronts are added through LDS in
//    wavefront order, rounded (nearest even) and stored, skipping rows >= M.
// Out-of-range pieces read zeros through the buffer range check (rows of A
// at or past M, K past the end, columns at or past N), as in the tiled
// kernels.
#include "gemm_internal.h"
#include "gemm_device.h"

namespace dgr {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x8 __attribute__((ext_vector_type(8)));

template <int N> struct Int {
    static constexpr int value = N;
};
// f(Int<I>{}) for I = B .. E-1, in order.
template <int B, int E, typename F> __device__ __forceinline__ void each(F&& f)
{
    if constexpr (B < E) {
        f(Int<B>{});
        each<B + 1, E>(f);
    }
}

// Element types.  KI = K per MFMA; a fragment is KI/4 consecutive K of one
// row of A or column of B per lane (16 bytes for 16-bit inputs, 32 for
// 8-bit).  c += b-fragment x a-fragment.
struct E4M3 {};
struct E5M2 {};
template <typename E> struct Mma;
template <> struct Mma<_Float16> {
    using Out = _Float16;
    using Frag = u32x4;
    static constexpr int BYTES = 2, KI = 32;
    static __device__ __forceinline__ void run(f32x4& c, const Frag& b, const Frag& a)
    {
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, b), __builtin_bit_cast(f16x8, a), c, 0,
                                                   0, 0);
    }
};
template <> struct Mma<__bf16> {
    using Out = __bf16;
    using Frag = u32x4;
    static constexpr int BYTES = 2, KI = 32;
    static __device__ __forceinline__ void run(f32x4& c, const Frag& b, const Frag& a)
    {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, a), c,
                                                    0, 0, 0);
    }
};
// operand format 0 = E4M3, 1 = E5M2 for both operands; scale operands 0
template <int FMT> struct Mma8 {
    using Out = __bf16;
    using Frag = u32x8;
    static constexpr int BYTES = 1, KI = 128;
    static __device__ __forceinline__ void run(f32x4& c, const Frag& b, const Frag& a)
    {
        c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(__builtin_bit_cast(i32x8, b),
                                                              __builtin_bit_cast(i32x8, a), c, FMT, FMT, 0, 0, 0, 0);
    }
};
template <> struct Mma<E4M3> : Mma8<0> {};
template <> struct Mma<E5M2> : Mma8<1> {};

template <typename E, int BMS, int BN, int BK, int W, int NSTG>
__global__ __launch_bounds__(64 * W, 1) void gemm_fewrow_kernel(const unsigned char* A, const unsigned char* B,
                                                              typename Mma<E>::Out* C, int M, int N, int K,
                                                              int group_m, Batch bt)
{
    using Frag = typename Mma<E>::Frag;
    using Out = typename Mma<E>::Out;
    constexpr int ES = Mma<E>::BYTES;                // bytes per element of A and B
    constexpr int KI = Mma<E>::KI;                   // K per MFMA
    constexpr int FB = (int)sizeof(Frag);            // fragment bytes per lane (KI/4 * ES)
    constexpr int FN = BN / 16;                      // 16x16 tiles per row of them
    constexpr int FM = BMS < 16 ? 1 : BMS / 16;      // rows of 16x16 tiles
    constexpr int NS = BK / KI;                      // K-slices per K-step
    constexpr int ROW_B = BN * ES;                   // bytes of one B row of the strip
    constexpr int ROW_A = BK * ES;                   // bytes of one A row of a K-step
    constexpr int STEP_B = BK * ROW_B;
    constexpr int STEP_A = BMS * ROW_A;
    constexpr int STEP = STEP_B + STEP_A;            // bytes of one stage
    constexpr int LB = STEP_B / 1024, LA = STEP_A / 1024;
    constexpr int L = LB + LA;                       // direct-to-LDS loads per K-step
    constexpr int PA = ROW_A / 16;                   // 16-byte pieces per A row of a step
    static_assert(BMS == 8 || BMS == 16 || BMS == 32 || BMS == 64, "rows");
    static_assert(BN == 16 || BN == 32, "strip width");
    static_assert(BK % KI == 0, "K-step");
    static_assert(STEP_B % 1024 == 0 && STEP_A % 1024 == 0, "whole 1 KB loads");
    static_assert(PA == 4 || PA == 8, "A swizzle");
    static_assert(NSTG == 4, "one LDS object per stage below");
    static_assert(NSTG * L <= 63, "loads in flight must fit the vmcnt field");
    static_assert(NSTG * W * STEP <= 160 * 1024, "LDS");
    static_assert(W * BMS * BN * 4 <= NSTG * W * STEP, "partial sums must fit the stages");
    // Each stage is an LDS object of its own (the compiler's tracking of
    // direct-to-LDS loads then tells them apart); wavefront w uses bytes
    // [w*STEP, (w+1)*STEP) of each: B rows first, then A.
    __shared__ __attribute__((aligned(1024))) unsigned char s0[W * STEP], s1[W * STEP], s2[W * STEP], s3[W * STEP];
    auto stage = [&](int st) __attribute__((always_inline)) {
        return (lds_byte*)(st == 0 ? s0 : st == 1 ? s1 : st == 2 ? s2 : s3);
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

    // S = K-steps of every wavefront, a multiple of NSTG (the last ones may
    // lie past K: they read zeros), and rot = the step this workgroup's walk
    // starts at.  Where the B rows that the strips of one XCD cover fit its
    // 4 MB L2, each strip starts 5 steps after its neighbour; otherwise the
    // strips that share a 128-byte line of B rows start together, so that
    // all of them read the line while it is in the L2, and the next such
    // group 5 steps later.  (Measured, 16 rows, bf16: 4096 x 4096 8.6 us
    // per strip against 9.7 per group and 9.5 unrotated; 4096 x 14336 32.5
    // per group, 33.1 unrotated, 61.8 per strip.)
    const int nsteps = cdiv_i(K, BK);
    const int rounds_ = cdiv_i(cdiv_i(nsteps, W), NSTG);
    const int S = (rounds_ > 0 ? rounds_ : 1) * NSTG;   // K = 0: one round of zeros
    const long long xcd_bytes = (long long)cdiv_i(tiles_m * tiles_n * bt.count, kNumXcd) * ROW_B * K;
    const int lead = xcd_bytes <= (4ll << 20) ? tn : tn * ROW_B / 128;
    const int rot = __builtin_amdgcn_readfirstlane(lead * 5 % S);
    const int kw0 = wave * S;

    // B load l of a step: lane -> LDS byte p = 1024*l + 16*lane of the B part,
    // holding logical byte p ^ swizzle = row k, 16-byte piece c: global
    // (k0 + k)*N*ES + n0*ES + 16c (kOOB past N).  The transpose reads of a
    // half-wavefront take rows that land on the same banks (16-bit: rows k
    // and k+8, 4 rows per group; 8-bit: rows k and k+32, 8 rows per group);
    // rows with that row bit set are XOR-ed by half of the bank span a group
    // touches.
    constexpr int SWZ_BIT = ES == 2 ? 8 : 32;
    constexpr int SWZ = BN == 16 ? 128 : (ES == 2 ? 32 : 16);
    unsigned b_voff[LB];
#pragma unroll
    for (int l = 0; l < LB; ++l) {
        const int p = 1024 * l + 16 * lane;
        const int lg = p ^ (((p / ROW_B) & SWZ_BIT) ? SWZ : 0);
        const int k = lg / ROW_B, c = (lg % ROW_B) / 16;
        const int col = n0 + c * (16 / ES);
        b_voff[l] = col < N ? ((unsigned)k * (unsigned)N + (unsigned)col) * ES : kOOB;
    }
    // A load l of a step: lane -> LDS byte p = 1024*l + 16*lane of the A part
    // = row r, physical piece q holding logical piece q ^ swz(r) (K
    // (16/ES)*(q ^ swz(r)) .. of the step): global (m0 + r)*K*ES + k0*ES +
    // 16*(q ^ swz(r)), kOOB for rows >= M and, per step, pieces at or past K.
    // swz(r) spreads the 16 rows of a fragment read over distinct 16-byte
    // bank slots: 4 pieces per row -> (r/4)%4, 8 -> (r/2)%8.
    auto swz_a = [](int r) __attribute__((always_inline)) { return PA == 4 ? (r >> 2) & 3 : (r >> 1) & 7; };
    unsigned a_voff[LA];
    int a_kp[LA];   // first K of the piece within the step
#pragma unroll
    for (int l = 0; l < LA; ++l) {
        const int p = 1024 * l + 16 * lane;
        const int r = p / ROW_A, q = (p % ROW_A) / 16;
        const int lq = q ^ swz_a(r);
        a_kp[l] = lq * (16 / ES);
        a_voff[l] = m0 + r < M ? (unsigned)(m0 + r) * (unsigned)K * ES + (unsigned)lq * 16u : kOOB;
    }
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (unsigned)M * (unsigned)K * ES);

    // The wavefront's j-th K-step (j = 0 .. S-1) -> stage st.
    auto issue = [&](int st, int j) __attribute__((always_inline)) {
        const int jj = j + rot < S ? j + rot : j + rot - S;
        const int k0 = __builtin_amdgcn_readfirstlane((kw0 + jj) * BK);
        const int krem = K - k0;
        const int rows = __builtin_amdgcn_readfirstlane(krem < 0 ? 0 : (krem > BK ? BK : krem));
        const __amdgpu_buffer_rsrc_t rbk =
            make_rsrc(B + (size_t)(k0 < K ? k0 : 0) * N * ES, (unsigned)rows * (unsigned)N * ES);
        lds_byte* base = stage(st) + wave * STEP;
#pragma unroll
        for (int l = 0; l < LB; ++l) {
            const unsigned off = b_voff[l];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rbk, (void __attribute__((address_space(3)))*)(base + 1024 * l),
                                                     16, off, 0, 0, 0);
        }
#pragma unroll
        for (int l = 0; l < LA; ++l) {
            const unsigned off = a_kp[l] < krem ? a_voff[l] : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (void __attribute__((address_space(3)))*)(base + STEP_B + 1024 * l),
                                                     16, off, (k0 < K ? k0 : 0) * ES, 0, 0);
        }
        asm volatile("" ::: "memory");
    };

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
    // A fragment of K-slice s, tile row mi: lane -> row 16*mi + lane%16
    // (lane%8 with 8 rows: the MFMA's rows 8-15 repeat rows 0-7 and are
    // never stored), K from KI*s + (KI/4)*(lane/16): logical pieces
    // (KI*s + (KI/4)*(lane/16))/(16/ES) + h, h < AH.  The swizzle of row r
    // and of row r + 16 is the same, so tile row mi is 16*mi rows further.
    constexpr int AH = FB / 16;   // 16-byte reads per A fragment
    int a_rd[NS][AH];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int h = 0; h < AH; ++h) {
            const int r = lane & (BMS < 16 ? BMS - 1 : 15);
            const int lq = (KI * s + (KI / 4) * (lane >> 4)) / (16 / ES) + h;
            a_rd[s][h] = STEP_B + r * ROW_A + 16 * (lq ^ swz_a(r));
        }

    auto read_b = [&](const lds_byte* base, int s, int ni) __attribute__((always_inline)) -> Frag {
        const lds_byte* p = base + KI * s * ROW_B;
        if constexpr (ES == 2) {
            const s16x4 h0 =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p + b_rd[ni][0]));
            const s16x4 h1 =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p + b_rd[ni][1]));
            return __builtin_bit_cast(Frag, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            i32x2 h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                h[i] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 __attribute__((address_space(3)))*)(p + b_rd[ni][i]));
            const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3));
            const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_shufflevector(h[2], h[3], 0, 1, 2, 3));
            return __builtin_bit_cast(Frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };
    auto read_a = [&](const lds_byte* base, int s, int mi) __attribute__((always_inline)) -> Frag {
        const lds_byte* p = base + mi * 16 * ROW_A;
        if constexpr (AH == 1) {
            return __builtin_bit_cast(Frag, *(const u32x4 __attribute__((address_space(3)))*)(p + a_rd[s][0]));
        } else {
            const u32x4 lo = *(const u32x4 __attribute__((address_space(3)))*)(p + a_rd[s][0]);
            const u32x4 hi = *(const u32x4 __attribute__((address_space(3)))*)(p + a_rd[s][1]);
            return __builtin_bit_cast(Frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };

    f32x4 acc[FN][FM];
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) acc[ni][mi] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Step j of the wavefront (stage j % NSTG, a literal below): wait until
    // its loads have landed (`after` = this wavefront's loads issued after
    // them), read the fragments, refill the stage with step j + NSTG when
    // there is one, multiply.
    auto step = [&](const int st, int j, const bool refill, auto after_c) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(decltype(after_c)::value));
        asm volatile("" ::: "memory");
        const lds_byte* base = stage(st) + wave * STEP;
        Frag bf[NS][FN], af[NS][FM];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int ni = 0; ni < FN; ++ni) bf[s][ni] = read_b(base, s, ni);
#pragma unroll
            for (int mi = 0; mi < FM; ++mi) af[s][mi] = read_a(base, s, mi);
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // the stage is read: it may be refilled
        if (refill) issue(st, j + NSTG);
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int ni = 0; ni < FN; ++ni)
#pragma unroll
                for (int mi = 0; mi < FM; ++mi) Mma<E>::run(acc[ni][mi], bf[s][ni], af[s][mi]);
    };
    // prologue: steps 0 .. NSTG-1 (S is a multiple of NSTG)
    each<0, NSTG>([&](auto t) __attribute__((always_inline)) { issue(decltype(t)::value, decltype(t)::value); });
    // whole rounds with refills, then the last round without
    const int rounds = S / NSTG;
    for (int r = 0; r + 1 < rounds; ++r)
        each<0, NSTG>([&](auto t) __attribute__((always_inline)) {
            constexpr int tt = decltype(t)::value;
            step(tt, r * NSTG + tt, true, Int<(NSTG - 1) * L>{});
        });
    each<0, NSTG>([&](auto t) __attribute__((always_inline)) {
        constexpr int tt = decltype(t)::value;
        step(tt, (rounds - 1) * NSTG + tt, false, Int<(NSTG - 1 - tt) * L>{});
    });

    // ---- combine the partial sums of the wavefronts through LDS (every load
    // has landed: the last step waited for all of them)
    __syncthreads();
    // wavefront w's fp32 [BMS][BN] partial sums at byte w*BMS*BN*4 of the
    // stage objects taken as one run (chunk o / (W*STEP) of stage o / (W*STEP))
    auto part = [&](int w, int o) __attribute__((always_inline)) {
        const int g = w * BMS * BN * 4 + o;
        return (float __attribute__((address_space(3)))*)(stage(g / (W * STEP)) + g % (W * STEP));
    };
    // tile (ni, mi): lane l holds row 16*mi + l%16, columns 16*ni + 4*(l/16)
    // .. +3 (rows below BMS only)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) {
            const int m = 16 * mi + (lane & 15), n = 16 * ni + 4 * (lane >> 4);
            if (m < BMS) *(f32x4 __attribute__((address_space(3)))*)part(wave, (m * BN + n) * 4) = acc[ni][mi];
        }
    __syncthreads();
    // thread t sums 4 consecutive columns of one row over the wavefronts, in order
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
    auto* C = static_cast<typename Mma<E>::Out*>(a.C);
#define DGR_LAUNCH(BMS_, BN_, BK_, W_)                                                                      \
    if (cfg.bm == BMS_ && cfg.bn == BN_ && cfg.bk == BK_ && cfg.threads == 64 * W_) {                      \
        hipLaunchKernelGGL((gemm_fewrow_kernel<E, BMS_, BN_, BK_, W_, 4>), dim3(tiles * a.batch.count),    \
                           dim3(64 * W_), 0, a.stream, A, B, C, a.M, a.N, a.K, cfg.group_m, a.batch);      \
        return hipGetLastError();                                                                          \
    }
    if constexpr (Mma<E>::BYTES == 2) {
        DGR_LAUNCH(16, 16, 32, 8)
        DGR_LAUNCH(16, 16, 64, 8)
        DGR_LAUNCH(16, 32, 32, 8)
        DGR_LAUNCH(8, 16, 64, 8)
        DGR_LAUNCH(32, 16, 32, 8)
        DGR_LAUNCH(32, 32, 32, 8)
        DGR_LAUNCH(64, 16, 32, 8)
        DGR_LAUNCH(64, 32, 32, 4)
    } else {
        DGR_LAUNCH(16, 16, 128, 8)
        DGR_LAUNCH(16, 32, 128, 4)
        DGR_LAUNCH(8, 32, 128, 4)
        DGR_LAUNCH(32, 32, 128, 4)
    }
#undef DGR_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fewrow(const Config& cfg, const LaunchArgs& a)
{
    if (a.dtype == kF16) return launch_e<_Float16>(cfg, a);
    if (a.dtype == kBF16) return launch_e<__bf16>(cfg, a);
    if (a.dtype == kFP8E4M3) return launch_e<E4M3>(cfg, a);
    if (a.dtype == kFP8E5M2) return launch_e<E5M2>(cfg, a);
    return hipErrorInvalidValue;
}

}  // namespace dgr
