// Host side of the C ABI declared in include/dense_gemm.h: argument checks,
// the handle, the configuration table, configuration choice and launch.
//
// The contract follows the pages' wrappers (notebook "Triton tiled matmul",
// section "The kernel", and chapter "Fast matrix multiplication", the
// Triton wrapper): [M,K] @ [K,N] -> [M,N], the caller provides C of the input
// type, one 1-D grid of ceil(M/BM)*ceil(N/BN) workgroups, asynchronous launch.
#include <mutex>
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../include/dense_gemm.h"
#include "gemm_internal.h"

// Scratch of gemm_run_noalloc (for callers that cannot allocate): the fp32
// partial sums of a split-K product.  Every device the library runs on holds
// its own copy until the process ends.  In host code this name is only a
// stand-in for the device array; its device address, looked up once per
// device by gemm_create, is what the kernels get.
static __device__ __align__(256) unsigned char scratch[GEMM_NOALLOC_SCRATCH_BYTES];

struct gemm_ctx {
    int device;
    int cu_count;
    char arch[64];
    void* scratch;   // device address of `scratch` on `device`
};

namespace dgr {
namespace {

enum Kind { kGeneric = 0, kMfma32x32 = 1, kMfma16x16 = 2, kGemv = 3, kFp8 = 4, kSkinny = 5, kFp32 = 6, kShortK = 7, kFewRow = 8 };

struct Entry {
    Config cfg;
    Kind kind;
};

// Configuration table.  Entry 0 accepts everything and is the fallback.
// The MFMA entries need 16-byte aligned A, B, C and K, N multiples of 16
// bytes of their matrices' rows (so every 16-byte global access lies wholly
// inside or wholly outside a row).
const Entry kTable[] = {
    {{0, 64, 64, 32, 8, 256, 0x1f, 0, 0, "generic_64x64"}, kGeneric},
    {{1, 256, 256, 32, 4, 256, 0x6, 1, 1, "mfma32x32_256x256x32"}, kMfma32x32},
    {{2, 256, 128, 32, 4, 256, 0x6, 1, 1, "mfma32x32_256x128x32"}, kMfma32x32},
    {{3, 128, 128, 32, 4, 256, 0x6, 1, 1, "mfma32x32_128x128x32"}, kMfma32x32},
    {{4, 256, 256, 32, 4, 512, 0x6, 1, 1, "mfma32x32_256x256x32_w8"}, kMfma32x32},
    {{5, 256, 256, 64, 4, 256, 0x6, 1, 1, "mfma32x32_256x256x64"}, kMfma32x32},
    {{6, 256, 256, 32, 4, 256, 0x6, 1, 1, "mfma16x16_256x256x32"}, kMfma16x16},
    {{7, 256, 128, 32, 4, 256, 0x6, 1, 1, "mfma16x16_256x128x32"}, kMfma16x16},
    {{8, 256, 256, 64, 4, 256, 0x6, 1, 1, "mfma16x16_256x256x64"}, kMfma16x16},
    {{9, 256, 128, 64, 4, 256, 0x6, 1, 1, "mfma16x16_256x128x64"}, kMfma16x16},
    // matrix-vector: bm = rows per workgroup, bn = the most columns of B, bk =
    // the K elements one wavefront instruction covers
    {{10, 8, 4, 512, 1, 256, 0x6, 1, 0, "gemv_8rows"}, kGemv},
    {{11, 16, 4, 512, 1, 256, 0x6, 1, 0, "gemv_16rows"}, kGemv},
    {{12, 128, 128, 32, 4, 256, 0x6, 1, 1, "mfma16x16_128x128x32"}, kMfma16x16},
    // 8-bit inputs (E4M3, E5M2), bf16 output; bk in elements (= bytes)
    {{13, 256, 256, 64, 4, 256, 0x18, 1, 1, "fp8_256x256x64"}, kFp8},
    {{14, 256, 256, 128, 4, 256, 0x18, 1, 1, "fp8_256x256x128"}, kFp8},
    // few rows: bm = rows of A per workgroup (all of M, normally), bn =
    // columns of the strip, bk = K per step; the wavefronts (threads / 64)
    // of a workgroup split K
    {{15, 16, 16, 64, 2, 512, 0x6, 1, 1, "skinny_16x16x64"}, kSkinny},
    {{16, 32, 16, 64, 2, 512, 0x6, 1, 1, "skinny_32x16x64"}, kSkinny},
    {{17, 64, 16, 32, 2, 256, 0x6, 1, 1, "skinny_64x16x32"}, kSkinny},
    {{18, 16, 32, 64, 2, 256, 0x6, 1, 1, "skinny_16x32x64"}, kSkinny},
    {{19, 32, 32, 64, 2, 256, 0x6, 1, 1, "skinny_32x32x64"}, kSkinny},
    {{20, 64, 32, 32, 2, 256, 0x6, 1, 1, "skinny_64x32x32"}, kSkinny},
    {{21, 16, 16, 32, 2, 512, 0x6, 1, 1, "skinny_16x16x32"}, kSkinny},
    // the same for 8-bit inputs (bk in elements = bytes)
    {{22, 16, 16, 128, 2, 512, 0x18, 1, 1, "skinny8_16x16x128"}, kSkinny},
    {{23, 32, 16, 128, 2, 512, 0x18, 1, 1, "skinny8_32x16x128"}, kSkinny},
    {{24, 16, 32, 128, 2, 256, 0x18, 1, 1, "skinny8_16x32x128"}, kSkinny},
    {{25, 32, 32, 128, 2, 256, 0x18, 1, 1, "skinny8_32x32x128"}, kSkinny},
    // 8-bit tiles of 128 x 128 (two workgroups per CU)
    {{26, 128, 128, 64, 4, 256, 0x18, 1, 1, "fp8_128x128x64"}, kFp8},
    {{27, 128, 128, 128, 4, 256, 0x18, 1, 1, "fp8_128x128x128"}, kFp8},
    // 192 x 256 tiles: whole waves of CUs where 256 x 256 leaves a partial one
    {{28, 192, 256, 32, 4, 256, 0x6, 1, 1, "mfma16x16_192x256x32"}, kMfma16x16},
    // the 16x16x32 kernel with A loaded direct to LDS too (one ring for A and B)
    {{29, 256, 256, 32, 4, 256, 0x6, 1, 1, "mfma16x16_256x256x32_adma", 1}, kMfma16x16},
    {{30, 128, 128, 32, 4, 256, 0x6, 1, 1, "mfma16x16_128x128x32_adma", 1}, kMfma16x16},
    {{31, 192, 256, 32, 4, 256, 0x6, 1, 1, "mfma16x16_192x256x32_adma", 1}, kMfma16x16},
    // the 8-bit kernel with A loaded direct to LDS
    {{32, 256, 256, 64, 4, 256, 0x18, 1, 1, "fp8_256x256x64_adma", 1}, kFp8},
    {{33, 128, 128, 64, 4, 256, 0x18, 1, 1, "fp8_128x128x64_adma", 1}, kFp8},
    // matrix-vector with the wavefronts of a workgroup splitting K (bm = R)
    {{34, 4, 4, 512, 1, 256, 0x6, 1, 0, "gemv_kslice_4rows", 1}, kGemv},
    {{35, 8, 4, 512, 1, 256, 0x6, 1, 0, "gemv_kslice_8rows", 1}, kGemv},
    // the 16x16 kernel at 64 x 128: few rows with split K
    {{36, 64, 128, 32, 4, 256, 0x6, 1, 1, "mfma16x16_64x128x32"}, kMfma16x16},
    {{37, 64, 128, 32, 4, 256, 0x6, 1, 1, "mfma16x16_64x128x32_adma", 1}, kMfma16x16},
    // the 8-bit kernel at 64 x 128 x 64, A direct to LDS: few rows with split K
    {{38, 64, 128, 64, 4, 256, 0x18, 1, 1, "fp8_64x128x64_adma", 1}, kFp8},
    // the 8-bit kernel at 192 x 256 x 64, A direct to LDS: partial last waves
    {{39, 192, 256, 64, 4, 256, 0x18, 1, 1, "fp8_192x256x64_adma", 1}, kFp8},
    // the default 256 x 256 configuration (29) with other tile orders, for
    // measuring the order's effect on cache reuse; never selected: the band
    // height GROUP_M = 1 (row-major) and 8, and no XCD remap
    {{40, 256, 256, 32, 1, 256, 0x6, 1, 1, "mfma16x16_256x256x32_g1_adma", 1}, kMfma16x16},
    {{41, 256, 256, 32, 8, 256, 0x6, 1, 1, "mfma16x16_256x256x32_g8_adma", 1}, kMfma16x16},
    {{42, 256, 256, 32, 4, 256, 0x6, 1, 0, "mfma16x16_256x256x32_noxcd_adma", 1}, kMfma16x16},
    // few rows: strips with more K-steps of B in flight per CU (16 wavefronts
    // on a 16-column strip; 32-column strips with 32-deep K-steps)
    {{43, 16, 16, 32, 2, 1024, 0x6, 1, 1, "skinny_16x16x32_w16"}, kSkinny},
    {{44, 16, 32, 32, 2, 512, 0x6, 1, 1, "skinny_16x32x32"}, kSkinny},
    // fp32 on the MFMA unit (v_mfma_f32_16x16x4f32), 128 x 128 x 32 tiles
    {{45, 128, 128, 32, 4, 256, 0x1, 1, 1, "fp32_128x128x32"}, kFp32},
    // the same at 64 x 128 and 64 x 64, for products with few 128 x 128 tiles
    {{46, 64, 128, 32, 4, 256, 0x1, 1, 1, "fp32_64x128x32"}, kFp32},
    {{47, 64, 64, 32, 4, 256, 0x1, 1, 1, "fp32_64x64x32"}, kFp32},
    // short K (at most 128, bk = the K extent staged): persistent 128 x 128
    // tiles, the next tile's loads in flight during the current one's stores
    {{48, 128, 128, 128, 4, 256, 0x6, 1, 1, "shortk_128x128x128"}, kShortK},
    // few rows in one launch with A streamed beside B (bm = rows per
    // workgroup, bn = strip columns, bk = K per step; each of the threads/64
    // wavefronts owns a contiguous K range)
    {{49, 16, 16, 32, 2, 512, 0x6, 1, 1, "fewrow_16x16x32"}, kFewRow},
    {{50, 16, 16, 64, 2, 512, 0x6, 1, 1, "fewrow_16x16x64"}, kFewRow},
    {{51, 16, 32, 32, 2, 512, 0x6, 1, 1, "fewrow_16x32x32"}, kFewRow},
    {{52, 16, 16, 128, 2, 512, 0x18, 1, 1, "fewrow8_16x16x128"}, kFewRow},
    {{53, 16, 32, 128, 2, 256, 0x18, 1, 1, "fewrow8_16x32x128"}, kFewRow},
    // the same with 8 rows per workgroup (half the A loads) for up to 8 rows
    {{54, 8, 16, 64, 2, 512, 0x6, 1, 1, "fewrow_8x16x64"}, kFewRow},
    {{55, 8, 32, 128, 2, 256, 0x18, 1, 1, "fewrow8_8x32x128"}, kFewRow},
    // the same with 32 or 64 rows per workgroup
    {{56, 32, 16, 32, 2, 512, 0x6, 1, 1, "fewrow_32x16x32"}, kFewRow},
    {{57, 32, 32, 32, 2, 512, 0x6, 1, 1, "fewrow_32x32x32"}, kFewRow},
    {{58, 64, 16, 32, 2, 512, 0x6, 1, 1, "fewrow_64x16x32"}, kFewRow},
    {{59, 64, 32, 32, 2, 256, 0x6, 1, 1, "fewrow_64x32x32"}, kFewRow},
    {{60, 32, 32, 128, 2, 256, 0x18, 1, 1, "fewrow8_32x32x128"}, kFewRow},
    // the 16x16x32 kernel at 256 x 256 with A staged two K-steps at a time
    // (whole cache lines per A load)
    {{61, 256, 256, 32, 4, 256, 0x6, 1, 1, "mfma16x16_256x256x32_apair", 2}, kMfma16x16},
    {{62, 192, 256, 32, 4, 256, 0x6, 1, 1, "mfma16x16_192x256x32_apair", 2}, kMfma16x16},
    // the 8-bit kernel with A staged two K-steps at a time
    {{63, 256, 256, 64, 4, 256, 0x18, 1, 1, "fp8_256x256x64_apair", 2}, kFp8},
    {{64, 192, 256, 64, 4, 256, 0x18, 1, 1, "fp8_192x256x64_apair", 2}, kFp8},
    {{65, 256, 256, 128, 4, 256, 0x18, 1, 1, "fp8_256x256x128_k128", 3}, kFp8},
    {{66, 192, 256, 128, 4, 256, 0x18, 1, 1, "fp8_192x256x128_k128", 3}, kFp8},
    {{67, 128, 128, 32, 4, 256, 0x6, 1, 1, "mfma16x16_128x128x32_apair", 2}, kMfma16x16},
};
constexpr int kTableSize = sizeof(kTable) / sizeof(kTable[0]);

// Bytes per element of A and B, and of C (8-bit inputs give a bf16 C).
inline int64_t in_bytes(int32_t dtype) { return dtype == kF32 ? 4 : (dtype == kF16 || dtype == kBF16) ? 2 : 1; }
inline int64_t out_bytes(int32_t dtype) { return dtype == kF32 ? 4 : 2; }
inline bool valid_dtype(int32_t d) { return d >= kF32 && d <= kFP8E5M2; }

// One call's arguments: `batch` products, matrix b of A (B, C) starting
// b*sa (b*sb, b*sc) elements after A (B, C).  A single product is batch 1.
struct Problem {
    const void* A;
    const void* B;
    void* C;
    int64_t M, N, K;
    int32_t dtype;
    int64_t batch, sa, sb, sc;
};

inline Problem single(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                      int32_t dtype)
{
    return Problem{A, B, C, M, N, K, dtype, 1, M * K, K * N, M * N};
}

inline bool overlaps(const void* p, int64_t pbytes, const void* q, int64_t qbytes)
{
    if (pbytes <= 0 || qbytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), a1 = a0 + (uintptr_t)pbytes;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(q), b1 = b0 + (uintptr_t)qbytes;
    return a0 < b1 && b0 < a1;
}

// Elements spanned by `batch` matrices of `elems` elements, `stride` apart
// (0 when empty); -1 when that does not fit in int64.
inline int64_t extent(int64_t batch, int64_t elems, int64_t stride)
{
    if (batch == 0 || elems == 0) return 0;
    if (batch > 1 && stride > (INT64_MAX - elems) / (batch - 1)) return -1;
    return (batch - 1) * stride + elems;
}

gemm_status_t check_args(const Problem& p)
{
    if (p.M < 0 || p.N < 0 || p.K < 0 || p.batch < 0 || p.sa < 0 || p.sb < 0 || p.sc < 0)
        return GEMM_ERR_INVALID_VALUE;
    if (!valid_dtype(p.dtype)) return GEMM_ERR_UNSUPPORTED_DTYPE;
    const int64_t lim = INT32_MAX;
    if (p.M > lim || p.N > lim || p.K > lim || p.batch > lim) return GEMM_ERR_TOO_LARGE;
    const int64_t si = in_bytes(p.dtype), so = out_bytes(p.dtype);
    // each matrix must stay below 2^31 bytes (32-bit byte offsets in the kernels);
    // products of two sizes <= 2^31-1 fit in int64
    const int64_t a_elems = p.M * p.K, b_elems = p.K * p.N, c_elems = p.M * p.N;
    const int64_t two31 = (int64_t)1 << 31;
    if (a_elems >= two31 / si || b_elems >= two31 / si || c_elems >= two31 / so)
        return GEMM_ERR_TOO_LARGE;
    // the whole grid (at the smallest tile, 64 x 64) must fit a 32-bit id
    if (((p.M + 63) / 64) * ((p.N + 63) / 64) * p.batch > lim) return GEMM_ERR_TOO_LARGE;
    const int64_t ea = extent(p.batch, a_elems, p.sa), eb = extent(p.batch, b_elems, p.sb),
                  ec = extent(p.batch, c_elems, p.sc);
    if (ea < 0 || eb < 0 || ec < 0 || ea > INT64_MAX / si || eb > INT64_MAX / si || ec > INT64_MAX / so)
        return GEMM_ERR_TOO_LARGE;
    if ((ea && !p.A) || (eb && !p.B) || (ec && !p.C)) return GEMM_ERR_INVALID_VALUE;
    if (overlaps(p.C, ec * so, p.A, ea * si) || overlaps(p.C, ec * so, p.B, eb * si))
        return GEMM_ERR_ALIASING;
    if (p.batch > 1 && c_elems > 0 && p.sc < c_elems) return GEMM_ERR_ALIASING;   // C matrices overlap
    return GEMM_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Whether configuration e can run these (already checked) arguments.
bool accepts(const Entry& e, const Problem& p)
{
    if (!((e.cfg.dtype_mask >> p.dtype) & 1)) return false;
    if (e.kind == kGemv) {
        // 16-byte pieces of A rows and of B's 8-row runs; C is stored element-wise
        const int64_t per16 = 16 / in_bytes(p.dtype);
        if (p.N < 1 || p.N > e.cfg.bn || p.K % per16) return false;
        if (!aligned16(p.A) || !aligned16(p.B)) return false;
        if (p.batch > 1 && (p.sa % per16 || p.sb % per16)) return false;
        return true;
    }
    if (e.kind == kShortK && p.K > e.cfg.bk) return false;   // the whole K range is staged at once
    if (e.cfg.needs_vec_align) {
        // elements per 16 bytes of A and B rows, and of C rows
        const int64_t pi = 16 / in_bytes(p.dtype), po = 16 / out_bytes(p.dtype);
        if (p.K % pi || p.N % pi || p.N % po) return false;
        if (!aligned16(p.A) || !aligned16(p.B) || !aligned16(p.C)) return false;
        if (p.batch > 1 && (p.sa % pi || p.sb % pi || p.sc % po)) return false;
    }
    return true;
}

// Shape classes (measured with bench.py --sweep over square 512^3 .. 8192^3,
// few-row products and the prefill projections):
//  * N <= 4: the matrix-vector kernel (it streams A at HBM bandwidth);
//  * M <= 128 (few rows, B streamed once): kernels of N/16 or N/32
//    workgroups per row block, one per strip of B's columns, which fill the
//    chip where the tiled kernels have a few dozen tiles (M = 16, N = K =
//    4096: 44 against 18 TFLOP/s) - the one-launch few-row kernel (A
//    streamed beside B) in the workgroup shape that fills the most CUs
//    within one wave of 256 workgroups, the 64 x 128 tiles where no shape
//    fits one wave (the rules below, from a sweep over 1-128 rows, bench.py
//    --sweep-fewrow);
//  * fp32 with 16-byte rows: the fp32 MFMA kernel (128 x 128 tiles from 1024
//    of them, else 64 x 64);
//  * K <= 128 over at least 1024 tiles of 128 x 128: the persistent short-K
//    kernel (config 48);
//  * small (M*N*K*batch < 128^3), other fp32 or unaligned: the generic kernel;
//  * at least 128 output tiles of 256 x 256 over the whole batch (half the
//    256 CUs or more): the 16x16x32 kernel at 256 x 256.  At one wave of
//    tiles it is 30-40 % faster than the 128 x 128 tile, and even at 144
//    tiles (3072^3) it matches it.  Where its last wave of tiles is partial
//    and 192 x 256 tiles fill fewer waves at lower cost (the wave model
//    below), the same kernel at 192 x 256 (3072^3: 58.9 against 69.7 us;
//    6144^3: 394 against 410);
//  * otherwise the 16x16x32 kernel at 128 x 128, which gives 4x the tiles
//    (2048^3: 842 TFLOP/s against 383 at 256 x 256);
//  * each of these tiled choices in its variant with A loaded direct to
//    LDS (configs 29-31), the 256 x 256 and 192 x 256 ones with A staged two
//    K-steps at a time (configs 61, 62).
// The 32x32x16 configurations and the 256 x 128 tiles were never the fastest
// in the sweep and stay available through gemm_run_config.
int select(const Problem& p)
{
    if (p.M == 0 || p.N == 0 || p.K == 0 || p.batch == 0) return 0;
    if (p.dtype == kF32) {
        // fp32 on the MFMA unit for aligned rows: 128 x 128 tiles from 1024
        // of them (4 per CU) over the batch, else 64 x 64 (4096^3 sustained:
        // 147.1 against 144.6 TFLOP/s on 64 x 64; 3072^3, 576 tiles: 141.8
        // against 104.6; 1024^3: 96.6 on 64 x 64 against 32.7 on 128 x 128
        // and 21.8 on the generic kernel; 64^3, graph-timed: 3.5 against
        // 6.7 us on the generic kernel)
        if (accepts(kTable[45], p))
            return ((p.M + 127) / 128) * ((p.N + 127) / 128) * p.batch >= 1024 ? 45 : 47;
        return 0;
    }
    if (p.dtype == kFP8E4M3 || p.dtype == kFP8E5M2) {
        if (!accepts(kTable[13], p) || p.M * p.N * p.K * p.batch < (int64_t)128 * 128 * 128) return 0;
        // Few rows: the one-launch few-row kernel wherever one of its
        // configurations fits one wave (at most 256 workgroups, one per CU: a
        // partial second wave costs about as much as the first); else the
        // tiled rules below (the 64 x 128 tiles).  Per row count (E4M3,
        // graph-timed):
        //  * up to 16 rows: 32-column strips, of 8 rows up to 8 rows (1-16 x
        //    4096 x 4096 5.6-6.2 us against 6.4-7.7 on the strip kernel), and
        //    16-column strips of 16 rows where K >= 8192 and they number
        //    129-256 (1-16 x 3072 x 8192 11.8-12.5 against 17.4-18.6 on 32
        //    columns; 16 x 4096 x 11008 19.9 against 21.7);
        //  * 17-32 rows: two row blocks of 16 rows where they fill at most
        //    192 CUs, or 256 from K = 8192 (24-32 x 1024 x 4096 5.3 against
        //    6.0 on 32-row workgroups, 24-32 x 3072 x 8192 15.7 against 19.7),
        //    else one of 32 rows (24-32 x 4096 x 4096 7.1 against 7.8);
        //  * 33-64 rows: row blocks of 16 where they fill at most 192 CUs and K
        //    < 8192 (40 x 2048^2 4.7 against 5.1; from K = 8192 three or more
        //    blocks of 16 rows run up to 1.9 times slower), else of 32 rows;
        //  * 65-128 rows: row blocks of 32 (96-128 x 2048 x 4096 7.3-8.1
        //    against 10.7 on the 64 x 128 tiles);
        //  * more workgroups than one wave: the 64 x 128 tiles (40-64 x 6144
        //    x 4096 13.8-15.1 against 16.8-17.6 on 384 workgroups; 1-16 x 11008
        //    x 4096 12.9-13.0 against 15.5-16.9).
        const int64_t s16 = (p.N + 15) / 16 * p.batch, s32 = (p.N + 31) / 32 * p.batch;
        if (p.M <= 16) {
            if (p.K >= 8192 && s16 > 128 && s16 <= 256) return 52;
            if (s32 <= 256) return p.M <= 8 ? 55 : 53;
        } else if (p.M <= 128) {
            const int64_t r16 = (p.M + 15) / 16 * s32, r32 = (p.M + 31) / 32 * s32;
            if (p.M <= 32 && (r16 <= 192 || (r16 <= 256 && p.K >= 8192))) return 53;
            if (p.M <= 64 && p.K < 8192 && r16 <= 192) return 53;
            if (r32 <= 256) return 60;
        }
        // at most 4 K-steps of 64: 128 x 128 tiles with A through registers,
        // for the same reason as the 16-bit short-K rule below (E4M3,
        // 64 x 2048^2, 8192^2, 8 x 4096^2: 12-22 % faster at K = 64-256)
        if (p.K <= 256) return 26;
        // 256 x 256 tiles once they cover half the CUs, else 128 x 128 (also
        // for few rows of a wide B, whose 16-byte strip rows cost one cache
        // line per lane).  A goes direct to LDS except for a partial single
        // wave of 256 x 256 tiles (sustained, E4M3: 8192^3 2881 against 2793
        // TFLOP/s, 512 x 4096 x 4096 15.6 against 17.1 us; 3072^3 34.8
        // against 33.4 us the other way round).
        // Fewer than 128 of them: 64 x 128 tiles with A direct to LDS while
        // they fit one wave (E4M3, one pass: 512^3-1024^3 11-21 % faster than
        // on 128 x 128 tiles, 256 x 4096 x 4096 28 %; 1536^3 slower).
        const int64_t t256 = ((p.M + 255) / 256) * ((p.N + 255) / 256) * p.batch;
        const int64_t t64 = ((p.M + 63) / 64) * ((p.N + 127) / 128) * p.batch;
        // a partial last wave of 256 x 256 tiles: 192 x 256 where its waves
        // cost less, by the 16-bit rule below
        const int64_t t192 = ((p.M + 191) / 192) * ((p.N + 255) / 256) * p.batch;
        // The 256 x 256 and 192 x 256 tiles run 128-deep K-steps on the
        // 16 x 16 x 128 MFMA (configs 65, 66).  Median of five 200-launch
        // blocks against the A-pair kernel with 64-deep K-steps on the
        // 32 x 32 x 64 MFMA (63, 64), same box, alternating: E4M3 4096^3
        // 49.6 against 50.7-50.8 us, E5M2 4096^3 48.4-48.6 against 49.5,
        // E4M3 8192^3 356.1-357.9 against 371.5-371.7, 8192 x 12288 x 4096
        // 287.5-288.3 against 297.1-297.2; on 192 x 256 tiles 3072^3
        // 25.7-25.9 against 26.8-26.9, 6144^3 159.3-159.9 against
        // 167.0-168.0.  The A-pair kernel itself beat the one-K-step ring (32,
        // 39) by 1.6-2.4 % on the same shapes.  Config 65 also takes 128-255
        // tiles (a partial single wave) where 192 x 256 tiles do not fit
        // better, in place of the 256 x 256 tile with A through registers
        // (13): 2048 x 6144 x 4096 40.2 against 43.9 us, 1024 x 14336 x 4096
        // 45.5 against 49.5-50.4, 1024 x 10240 x 4096 38.3 against 40.5.
        if (t256 >= 128 && ((t192 + 255) / 256) * 80 < ((t256 + 255) / 256) * 95) return 66;
        return t256 >= 128 ? 65 : t64 <= 256 ? 38 : 33;
    }
    if (p.N <= 4 && accepts(kTable[10], p)) {
        // Timed on bf16 shapes with M 2K-28K, K 2K-14K, N 1-4.  A K-slice
        // wavefront step covers 2048 (U = 4) or 1024 (U = 2) K positions, so
        // below K = 4096 some of the four wavefronts would idle: there the
        // rows are split instead.  From K = 4096 the K-slice kernels lead:
        // 4 rows per workgroup, or 8 with 3-4 columns (more outputs per
        // wavefront against fewer loads of B) once A is tall or K short.
        if (p.K < 4096) return 10;
        if (p.N >= 3 && (p.M * p.batch >= 8192 || p.K <= 4096)) return 35;
        return 34;
    }
    if (!accepts(kTable[6], p)) return 0;
    if (p.M * p.N * p.K * p.batch < (int64_t)128 * 128 * 128) return 0;
    if (p.M <= 128) {
        // Few rows: the one-launch few-row kernel (A streamed beside B)
        // wherever one of its configurations fits one wave (at most 256
        // workgroups, one per CU: a partial second wave costs about as much
        // as the first), with as many workgroups as that allows, mostly.
        // Per row count (bf16, graph-timed):
        //  * up to 16 rows: 16-column strips with 64-deep K-steps, of 8 rows
        //    up to 8 rows (1-16 x 4096 x 4096 7.8-9.2 us against 8.9-12.0 on
        //    the strip kernel; 16 x 4096 x 14336 32.6 against 37.2), 32-deep
        //    where K <= 3072 (1-16 x 3072^2 7.4-8.1 against 7.5-8.2), and
        //    32-column strips where K <= 2048 from N = 4096 or where 16
        //    columns take more than 256 workgroups (1-16 x 6144 x 4096
        //    12.6-14.1 against 16.9-18.8 on 384 workgroups); up to 8 rows
        //    also up to 384 strips of 32 (1 x 11008 x 4096 21.0 against 23.3
        //    on the 64 x 128 tiles);
        //  * 17-32 rows: two row blocks of 16 x 16 from K = 8192 (24-32 x
        //    2048 x 8192 16.2-16.7 against 17.6-18.5 on 16 x 32), else of 16 x
        //    32 (24-32 x 4096 x 4096 11.4-11.8 against 12.7-13.2 on 32 x 32),
        //    else one of 32 x 32 (24-32 x 6144 x 4096 15.7-16.5 against
        //    19.9-21.0);
        //  * 33-64 rows: row blocks of 16 x 32 where K <= 3072 (40-48 x 2048^2
        //    5.8-5.9 against 6.3-6.4 on 32 x 32), two of 32 x 16 from K = 8192
        //    (40 x 2048 x 8192 19.2 against 20.2), else of 32 x 32, else
        //    one of 64 x 32 (40-64 x 6144 x 4096 18.1-20.5 against 21.9-24.9
        //    on 384 workgroups of 32 x 32);
        //  * 65-128 rows: two row blocks of 64 x 32 (96-128 x 4096 x 4096
        //    16.9-18.6 against 22.5-23.6 on the 64 x 128 tiles);
        //  * more workgroups than one wave: the 64 x 128 tiles where they fit
        //    one (96-128 x 6144 x 4096 23.0-25.3 against 28.5-32.1 on 384
        //    workgroups of 64 x 32; 24-64 x 11008 x 4096 23.5-25.5 against
        //    25.9-35.4), through the tile rules below from 33 rows; up to 32
        //    rows below K = 1024 the strip kernel, and the few-row kernel in
        //    several waves where the tiles do not fit one either.
        const int64_t s16 = (p.N + 15) / 16 * p.batch, s32 = (p.N + 31) / 32 * p.batch;
        if (p.M <= 16) {
            if (s16 <= 256) {
                if (p.K <= 2048 && p.N >= 4096) return 51;
                if (p.K <= 3072) return 49;
                return p.M <= 8 ? 54 : 50;
            }
            if (s32 <= 256 || (p.M <= 8 && s32 <= 384)) return 51;
        } else if (p.M <= 32) {
            if (p.K >= 8192 && 2 * s16 <= 256) return 50;
            if (2 * s32 <= 256) return 51;
            if (s32 <= 256) return 57;
        } else if (p.M <= 64) {
            if (p.K <= 3072 && (p.M + 15) / 16 * s32 <= 256) return 51;
            if (p.K >= 8192 && 2 * s16 <= 256) return 56;
            if (2 * s32 <= 256) return 57;
            if (s32 <= 256) return 59;
        } else if (2 * s32 <= 256) {
            return 59;
        }
        if (p.M <= 32) {
            if ((p.N + 127) / 128 * p.batch <= 256) return p.K >= 1024 ? 37 : p.M <= 16 ? 18 : 19;
            return p.M <= 16 ? 51 : 57;
        }
    }
    // At most 128 K and at least 1024 tiles of 128 x 128: the persistent
    // short-K kernel, whose workgroups load their next tile while they store
    // the current one (bf16, graph-timed: 64 x 2048^2 x 128 122.6 against
    // 133.6 us on config 12; short bursts: 8192^2 x 128 32.2 against 35.8,
    // 8192^2 x 32 29.8 against 34.1, 16 x 2048^2 x 64 30.8 against 32.9;
    // 4096^2 x 128, 1024 tiles, even)
    if (p.K <= 128 && accepts(kTable[48], p) && ((p.M + 127) / 128) * ((p.N + 127) / 128) * p.batch >= 1024)
        return 48;
    // At most 8 K-steps of 32: a workgroup is mostly its prologue and its C
    // stores, and the 128 x 128 tile with A through registers (several
    // workgroups per CU) overlaps one's stores with another's loads (bf16,
    // 64 x 2048^2 and 8192^2 and 8 x 4096^2: 9-17 % faster than 256 x 256 at
    // K = 64-128, 0-6 % at 256, slower from 512)
    if (p.K <= 256) return 12;
    // Few tiles: 64 x 128 tiles with A direct to LDS while they fit one wave
    // of workgroups, else 128 x 128 (bf16, one pass: 40-128 rows of a wide B
    // 9-28 % faster than on 128 x 128 tiles, 512^3-1024^3 17-21 %,
    // 512 x 4096 x 4096 11 % faster than the 128 x 128 tiles split in two;
    // 1536^3 and 128 x 28672, 288 and 448 tiles of 64 x 128, slower)
    const int64_t t64 = ((p.M + 63) / 64) * ((p.N + 127) / 128) * p.batch;
    if (p.M <= 128 && t64 <= 256) return 37;
    const int64_t t256 = ((p.M + 255) / 256) * ((p.N + 255) / 256) * p.batch;
    // 128 x 128 tiles: A staged two K-steps at a time (67) beyond one wave
    // of them, the one-K-step ring (30) within it.  Median of five
    // 200-launch blocks, same box, alternating, 67 against 30: bf16
    // 2304^2 x 4096 (324 tiles) 46.9 against 60.2 us, 2560^2 x 2048 28.1
    // against 33.3, 3072 x 2048^2 27.4 against 32.3, 2816^2 x 1024 17.2-17.7
    // against 19.3-19.4; at 196-256 tiles 67 is 2-6 % slower (2048^3 19.9
    // against 19.3-19.4, 1792^3 17.3 against 16.3, 1024 x 4096^2 35.9-36.1
    // against 34.5-34.6).
    const int64_t t128 = ((p.M + 127) / 128) * ((p.N + 127) / 128) * p.batch;
    if (t256 < 128) return t64 <= 256 ? 37 : t128 > 256 ? 67 : 30;
    // A partial single wave of 256 x 256 tiles whose 128 x 128 tiles fill at
    // most the two workgroups a CU holds of them (t128 <= 512): 67 over the
    // 192 x 256 tile (62), sustained, alternating: bf16 2048 x 4096^2 59.3
    // against 61.0-61.2 us, 1024 x 8192 x 4096 58.9-59.2 against 62.6-62.8,
    // 2048 x 4096 x 14336 200.4-201.0 against 202.1-202.6, fp16 4096 x 2048 x
    // 8192 120.4-120.7 against 125.0-125.4 (3072^3, 576 tiles: 62.6 against
    // 48.2-48.7, so not beyond 512).
    if (t256 < 256 && t128 <= 512) return 67;
    // Tiles run in waves of one per CU (256 CUs).  A 192 x 256 tile holds 3/4
    // of a 256 x 256 tile's work at ~94 % of its rate, so a wave of them costs
    // ~0.8 of a wave of 256 x 256 tiles; it wins where 256 x 256 leaves a
    // partial last wave (3072^2: 144 tiles, one wave of 192 x 256 tiles).
    const int64_t t192 = ((p.M + 191) / 192) * ((p.N + 255) / 256) * p.batch;
    const int64_t w256 = (t256 + 255) / 256, w192 = (t192 + 255) / 256;
    const bool rows192 = w192 * 80 < w256 * 95;
    // A direct to LDS, staged two K-steps at a time so that every A load
    // reads whole cache lines (configs 61, 62), also where the operands
    // overflow the 256 MB Infinity Cache.  Median of five 200-step blocks
    // against the one-K-step A ring (29, 31), same box, alternating: fp16
    // 4096^3 1352-1358 against 1318-1320 TFLOP/s, bf16 8192^3 1524-1528
    // against 1507, the prefill projections QKV 1454 against 1430, out
    // 1424-1435 against 1406-1412, up 1437-1439 against 1415-1416, down
    // 1463-1465 against 1430, batched 16 x 2048^3 1361-1363 against 1344-1345,
    // 3072^3 on 192 x 256 tiles 1131-1141 against 1107-1121.  (The ring with
    // A direct to LDS led the A-through-registers configuration by 3-5 % on
    // the same products.)
    return rows192 ? 62 : 61;
}

// ---- split K (gemm_run_ws)

// Split count actually launched for `splits` requested: lowered until no
// split is left without K-steps of bk.
int effective_splits(int splits, int64_t K, int bk)
{
    const int64_t steps = (K + bk - 1) / bk;
    if (splits <= 1 || steps <= 1) return 1;
    const int64_t q = (steps + splits - 1) / splits;
    return (int)((steps + q - 1) / q);
}

constexpr int kSplitConfigFew = 37;  // the 16x16x32 kernel at 64 x 128, A direct to LDS
constexpr int kSplitConfig8 = 38;    // the 8-bit kernel at 64 x 128 x 64, A direct to LDS

// Split count for `tiles` tiles and `steps` K-steps: near 256 workgroups in
// all, at most 16 splits, at least `min_steps` K-steps per split, and none
// without K-steps.
int split_count(int64_t tiles, int64_t steps, int64_t K, int bk, int min_steps = 16)
{
    int s = (int)((256 + tiles / 2) / tiles);
    if (s > 16) s = 16;
    while (s > 1 && steps < min_steps * (int64_t)s) --s;
    return effective_splits(s, K, bk);
}

// The choice of gemm_run_ws: a configuration and a split count (1: none).
// Products of one matrix only; the numbers are from the shape sweep.
//  * fp16/bf16 with K >= 2048 (64 K-steps) and at most 160 tiles of
//    64 x 128: the 16x16x32 kernel at 64 x 128 with A direct to LDS with
//    split_count splits (a quarter of the MFMAs of a 128-row tile on rows
//    past M, and room for more workgroups per CU).  (256 x 4096 x 4096: 19.6
//    us with 4 splits against 31.9 in one pass; 16 x 4096 x 14336: 22.6
//    with 8 against 38.0 on the strip kernel; 1024^3: 14.4 with 2 against
//    10.7, hence the K floor.  64 x 128 against 128 x 128 tiles, 16-256 rows
//    x 1024-14336 x 2048-14336: 2-15 % faster, e.g. 16 x 4096 x 4096 7.9
//    against 8.9 us, 128 x 4096 x 4096 14.0 against 15.5.  Against the strip
//    kernel for 1-8 rows: 7.0-7.3 against 8.9-11.0 us at 4096 x 4096, 20.2
//    against 34.3 at 8 x 4096 x 14336.)
//  * 8-bit inputs, up to 128 rows, K >= 2048: the 8-bit kernel at
//    64 x 128 x 64 with A direct to LDS, split likewise, with at least 8
//    K-steps of 64 per split up to 16 rows, 16 up to 64 rows and 32 above
//    (the fp32 partial sums, 4 bytes per output against 1-byte inputs, weigh
//    more with more rows; 1-16 rows x 4096 x 4096: 5.4-6.3 us with 8 splits
//    against 6.1-6.6 with 4 and 6.4-7.7 on the strip kernel; 64 rows: 8.9
//    with 4, 11.3 with 8).  Beyond 128 rows they cost more than the split gains.  (E4M3,
//    against the 128 x 128 split: 16-128 rows x 4096 x 4096 6.6-9.7 us
//    against 7.6-13.4, 1-5 % faster with N or K = 14336; 64 x 4096 x 14336:
//    17.0 us with 8 splits on 128 x 128 tiles against 38.4 on the strip
//    kernel; 256 x 4096 x 4096: 16.5 in one pass, 17.6 with 2 splits.)
int select_ws(const Problem& p, int64_t ws_bytes, int& splits)
{
    splits = 1;
    const int c = select(p);
    if (p.batch != 1 || p.M == 0 || p.N == 0) return c;
    int cfg = -1, s = 1;
    if (p.dtype == kF16 || p.dtype == kBF16) {
        if (!accepts(kTable[kSplitConfigFew], p) || kTable[c].kind == kGemv) return c;
        // the one-launch few-row kernel beats a split where K or B is small
        // (bf16: 16 x 2048 x 2048 4.5 against 6.6 us with 4 splits, 16 x 4096
        // x 2048 5.0 against 7.1, 16 x 2048 x 4096 6.3 against 7.0; 16 x 3072
        // x 3072 7.9 against 7.1 and 16 x 4096 x 4096 8.8 against 8.2 the
        // other way round)
        if (kTable[c].kind == kFewRow && (p.K <= 2048 || (p.K <= 4096 && p.N <= 2048))) return c;
        const int64_t steps = (p.K + 31) / 32;
        const int64_t t = ((p.M + 63) / 64) * ((p.N + 127) / 128);
        if (steps < 64 || t > 160) return c;
        cfg = kSplitConfigFew;
        s = split_count(t, steps, p.K, 32);
    } else if (p.dtype == kFP8E4M3 || p.dtype == kFP8E5M2) {
        if (!accepts(kTable[kSplitConfig8], p) || p.M > 128) return c;
        // up to 64 rows with K and N at most 4096: the one-launch few-row
        // kernel (E4M3: 16 x 4096 x 4096 6.0 against 6.5 us with 8 splits,
        // 24-64 rows 6.8-8.5 against 7.1-9.1, 16 x 2048-3072 x 2048-4096
        // 3.9-5.0 against 5.6-6.1; 1-8 rows x 4096 x 4096 5.6-6.0 against
        // 5.6-5.9)
        if (kTable[c].kind == kFewRow && p.M <= 64 && p.K <= 4096 && p.N <= 4096) return c;
        const int64_t steps = (p.K + 63) / 64;
        if (steps < 32) return c;
        cfg = kSplitConfig8;
        s = split_count(((p.M + 63) / 64) * ((p.N + 127) / 128), steps, p.K, 64,
                        p.M <= 16 ? 8 : p.M <= 64 ? 16 : 32);
    } else {
        return c;
    }
    if (s < 2 || (int64_t)s * p.M * p.N * 4 > ws_bytes) return c;
    splits = s;
    return cfg;
}

// Workspace argument checks (after check_args).
gemm_status_t check_ws(const Problem& p, const void* ws, int64_t ws_bytes)
{
    if (ws_bytes < 0 || (!ws && ws_bytes > 0)) return GEMM_ERR_INVALID_VALUE;
    if (ws && (reinterpret_cast<uintptr_t>(ws) & 15u)) return GEMM_ERR_INVALID_VALUE;
    const int64_t si = in_bytes(p.dtype), so = out_bytes(p.dtype);
    if (overlaps(ws, ws_bytes, p.A, p.M * p.K * si) || overlaps(ws, ws_bytes, p.B, p.K * p.N * si) ||
        overlaps(ws, ws_bytes, p.C, p.M * p.N * so))
        return GEMM_ERR_ALIASING;
    return GEMM_OK;
}

// Whether configuration e's grid for these arguments fits the launch: its
// kernels number their workgroups with 32-bit ints (at most 2^31-1 of them),
// and HIP takes at most 2^32-1 lanes in one grid.  Every launcher makes
// ceil(M/bm) * ceil(N/bn) workgroups per product (ceil(M/bm) for the
// matrix-vector kernel, whose workgroups cover all N <= 4 columns), times the
// batch, or times the split count for a split product.
bool grid_fits(const Entry& e, const Problem& p, int splits)
{
    const int64_t tm = (p.M + e.cfg.bm - 1) / e.cfg.bm;
    const int64_t tn = e.kind == kGemv ? 1 : (p.N + e.cfg.bn - 1) / e.cfg.bn;
    const int64_t per = tm * tn;   // < 2^62: M, N < 2^31
    if (per > INT32_MAX) return false;
    const int64_t groups = per * (splits > 1 ? splits : p.batch);   // < 2^62
    return groups <= INT32_MAX && groups * e.cfg.threads <= (int64_t)UINT32_MAX;
}

// The checks of gemm_run before anything is enqueued: the arguments, then
// the grid of the configuration it selects.
gemm_status_t check_run(const Problem& p)
{
    const gemm_status_t st = check_args(p);
    if (st != GEMM_OK) return st;
    return grid_fits(kTable[select(p)], p, 1) ? GEMM_OK : GEMM_ERR_TOO_LARGE;
}

gemm_status_t launch(const Entry& e, gemm_handle_t h, const Problem& p, void* stream, int splits = 1,
                     void* ws = nullptr, unsigned long long* clk = nullptr)
{
    if (!grid_fits(e, p, splits)) return GEMM_ERR_TOO_LARGE;
    if (!h) return GEMM_ERR_INVALID_VALUE;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return GEMM_ERR_HIP;
    if (cur != h->device) return GEMM_ERR_INVALID_VALUE;
    if (p.M == 0 || p.N == 0 || p.batch == 0) return GEMM_OK;
    LaunchArgs la{p.A, p.B, p.C, (int)p.M, (int)p.N, (int)p.K, p.dtype, static_cast<hipStream_t>(stream),
                  Batch{(int)p.batch, p.sa, p.sb, p.sc}};
    la.splits = splits;
    la.ws = static_cast<float*>(ws);
    la.cus = h->cu_count;
    la.clk = clk;
    hipError_t err = hipSuccess;
    switch (e.kind) {
    case kGeneric: err = launch_generic(e.cfg, la); break;
    case kMfma32x32: err = launch_mfma32x32(e.cfg, la); break;
    case kMfma16x16:
        err = launch_mfma16x16(e.cfg, la);
        if (err == hipSuccess && splits > 1) err = launch_reduce_splits(la);
        break;
    case kGemv: err = launch_gemv(e.cfg, la); break;
    case kFp8:
        err = launch_fp8(e.cfg, la);
        if (err == hipSuccess && splits > 1) err = launch_reduce_splits(la);
        break;
    case kSkinny: err = launch_skinny(e.cfg, la); break;
    case kFp32: err = launch_fp32(e.cfg, la); break;
    case kShortK: err = launch_shortk(e.cfg, la); break;
    case kFewRow: err = launch_fewrow(e.cfg, la); break;
    }
    return err == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

gemm_status_t run(gemm_handle_t h, const Problem& p, void* stream)
{
    const gemm_status_t st = check_args(p);
    if (st != GEMM_OK) return st;
    return launch(kTable[select(p)], h, p, stream);
}

gemm_status_t run_clocked(gemm_handle_t h, const Problem& p, void* clk, void* stream)
{
    const gemm_status_t st = check_args(p);
    if (st != GEMM_OK) return st;
    if (!clk || (reinterpret_cast<uintptr_t>(clk) & 7u)) return GEMM_ERR_INVALID_VALUE;
    return launch(kTable[select(p)], h, p, stream, 1, nullptr, static_cast<unsigned long long*>(clk));
}

gemm_status_t run_ws(gemm_handle_t h, const Problem& p, void* ws, int64_t ws_bytes, void* stream)
{
    gemm_status_t st = check_args(p);
    if (st != GEMM_OK) return st;
    if ((st = check_ws(p, ws, ws_bytes)) != GEMM_OK) return st;
    int splits = 1;
    const int c = select_ws(p, ws ? ws_bytes : 0, splits);
    return launch(kTable[c], h, p, stream, splits, ws);
}

gemm_status_t run_ws_config(gemm_handle_t h, const Problem& p, int32_t config_id, int32_t splits, void* ws,
                            int64_t ws_bytes, void* stream)
{
    gemm_status_t st = check_args(p);
    if (st != GEMM_OK) return st;
    if ((st = check_ws(p, ws, ws_bytes)) != GEMM_OK) return st;
    if (config_id < 0 || config_id >= kTableSize || splits < 1 || splits > 64) return GEMM_ERR_INVALID_VALUE;
    const Entry& e = kTable[config_id];
    if (!accepts(e, p)) return GEMM_ERR_CONFIG_MISMATCH;
    int s = 1;
    if (splits > 1) {
        // split forms: every tile configuration with A through registers, and
        // the 128 x 128 ones with A direct to LDS
        const bool adma128 = e.cfg.sched == 1 && e.cfg.bm <= 128 && e.cfg.bn == 128;
        if ((e.kind != kMfma16x16 && e.kind != kFp8) || (e.cfg.sched != 0 && !adma128) || p.batch != 1)
            return GEMM_ERR_CONFIG_MISMATCH;
        s = effective_splits(splits, p.K, e.cfg.bk);
        if (s > 1 && (int64_t)s * p.M * p.N * 4 > ws_bytes) return GEMM_ERR_INVALID_VALUE;
    }
    return launch(e, h, p, stream, s, ws);
}

gemm_status_t run_config(gemm_handle_t h, const Problem& p, int32_t config_id, void* stream)
{
    const gemm_status_t st = check_args(p);
    if (st != GEMM_OK) return st;
    if (config_id < 0 || config_id >= kTableSize) return GEMM_ERR_INVALID_VALUE;
    const Entry& e = kTable[config_id];
    if (!accepts(e, p)) return GEMM_ERR_CONFIG_MISMATCH;
    return launch(e, h, p, stream);
}

// Device address of `scratch` per device, looked up once per device (with
// that device current) and kept for the life of the process.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

gemm_status_t scratch_address(int dev, void** out)
{
    if (dev < 0 || dev >= kMaxDevices) return GEMM_ERR_UNSUPPORTED_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return GEMM_ERR_HIP;
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return GEMM_OK;
}

// gemm_run_ws's choice with the library's scratch as the workspace.
gemm_status_t run_noalloc(gemm_handle_t h, const Problem& p, void* stream)
{
    const gemm_status_t st = check_args(p);
    if (st != GEMM_OK) return st;
    if (!h || !h->scratch) return GEMM_ERR_INVALID_VALUE;
    int splits = 1;
    const int c = select_ws(p, INT64_MAX, splits);
    if (splits > 1 && (int64_t)splits * p.M * p.N * 4 > (int64_t)GEMM_NOALLOC_SCRATCH_BYTES)
        return GEMM_ERR_TOO_LARGE;
    return launch(kTable[c], h, p, stream, splits, splits > 1 ? h->scratch : nullptr);
}

}  // namespace
}  // namespace dgr

using namespace dgr;

extern "C" {

gemm_status_t gemm_create(gemm_handle_t* out)
{
    if (!out) return GEMM_ERR_INVALID_VALUE;
    *out = nullptr;
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return GEMM_ERR_UNSUPPORTED_DEVICE;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_ERR_HIP;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GEMM_ERR_UNSUPPORTED_DEVICE;
    void* sp = nullptr;
    const gemm_status_t st = scratch_address(dev, &sp);
    if (st != GEMM_OK) return st;
    gemm_ctx* h = new (std::nothrow) gemm_ctx;
    if (!h) return GEMM_ERR_HIP;
    h->scratch = sp;
    h->device = dev;
    h->cu_count = prop.multiProcessorCount;
    strncpy(h->arch, prop.gcnArchName, sizeof(h->arch) - 1);
    h->arch[sizeof(h->arch) - 1] = 0;
    *out = h;
    return GEMM_OK;
}

gemm_status_t gemm_destroy(gemm_handle_t h)
{
    delete h;
    return GEMM_OK;
}

const char* gemm_status_string(int32_t s)
{
    switch (s) {
    case GEMM_OK: return "ok";
    case GEMM_ERR_INVALID_VALUE: return "invalid value";
    case GEMM_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case GEMM_ERR_UNSUPPORTED_DEVICE: return "unsupported device (needs a gfx950 GPU)";
    case GEMM_ERR_TOO_LARGE: return "problem too large";
    case GEMM_ERR_ALIASING: return "C overlaps A, B or another C matrix";
    case GEMM_ERR_HIP: return "HIP runtime error";
    case GEMM_ERR_CONFIG_MISMATCH: return "configuration does not accept these arguments";
    default: return "unknown status";
    }
}

gemm_status_t gemm_check_args(const void* A, const void* B, const void* C,
                              int64_t M, int64_t N, int64_t K, int32_t dtype)
{
    return check_run(single(A, B, const_cast<void*>(C), M, N, K, dtype));
}

gemm_status_t gemm_check_args_batched(const void* A, const void* B, const void* C, int64_t batch,
                                      int64_t M, int64_t N, int64_t K, int64_t stride_a,
                                      int64_t stride_b, int64_t stride_c, int32_t dtype)
{
    return check_run(Problem{A, B, const_cast<void*>(C), M, N, K, dtype, batch, stride_a, stride_b, stride_c});
}

int32_t gemm_config_count(void) { return kTableSize; }

gemm_status_t gemm_config_info(int32_t id, gemm_config_info_t* out)
{
    if (!out || id < 0 || id >= kTableSize) return GEMM_ERR_INVALID_VALUE;
    const Config& c = kTable[id].cfg;
    memset(out, 0, sizeof(*out));
    out->id = c.id;
    out->bm = c.bm;
    out->bn = c.bn;
    out->bk = c.bk;
    out->group_m = c.group_m;
    out->threads = c.threads;
    out->dtype_mask = c.dtype_mask;
    out->needs_vec_align = c.needs_vec_align;
    out->xcd_remap = c.xcd_remap;
    strncpy(out->name, c.name, sizeof(out->name) - 1);
    return GEMM_OK;
}

int32_t gemm_select_config(const void* A, const void* B, const void* C,
                           int64_t M, int64_t N, int64_t K, int32_t dtype)
{
    const Problem p = single(A, B, const_cast<void*>(C), M, N, K, dtype);
    if (check_args(p) != GEMM_OK) return -1;
    return select(p);
}

int32_t gemm_select_config_batched(const void* A, const void* B, const void* C, int64_t batch,
                                   int64_t M, int64_t N, int64_t K, int64_t stride_a,
                                   int64_t stride_b, int64_t stride_c, int32_t dtype)
{
    const Problem p{A, B, const_cast<void*>(C), M, N, K, dtype, batch, stride_a, stride_b, stride_c};
    if (check_args(p) != GEMM_OK) return -1;
    return select(p);
}

gemm_status_t gemm_tile_of_block_batched(int32_t id, int64_t M, int64_t N, int64_t batch, int64_t block,
                                         int64_t* batch_index, int64_t* tile_m, int64_t* tile_n)
{
    if (id < 0 || id >= kTableSize || !batch_index || !tile_m || !tile_n || M <= 0 || N <= 0 ||
        batch <= 0 || M > INT32_MAX || N > INT32_MAX || batch > INT32_MAX)
        return GEMM_ERR_INVALID_VALUE;
    const Config& c = kTable[id].cfg;
    const int tiles_m = cdiv_i((int)M, c.bm), tiles_n = cdiv_i((int)N, c.bn);
    if ((int64_t)tiles_m * tiles_n * batch > INT32_MAX) return GEMM_ERR_TOO_LARGE;
    if (block < 0 || block >= (int64_t)tiles_m * tiles_n * batch) return GEMM_ERR_INVALID_VALUE;
    int b, tm, tn;
    tile_of_block((int)block, tiles_m, tiles_n, (int)batch, c.group_m, c.xcd_remap != 0, b, tm, tn);
    *batch_index = b;
    *tile_m = tm;
    *tile_n = tn;
    return GEMM_OK;
}

gemm_status_t gemm_tile_of_block(int32_t id, int64_t M, int64_t N, int64_t block,
                                 int64_t* tile_m, int64_t* tile_n)
{
    int64_t b = 0;
    return gemm_tile_of_block_batched(id, M, N, 1, block, &b, tile_m, tile_n);
}

gemm_status_t gemm_run(gemm_handle_t h, const void* A, const void* B, void* C,
                       int64_t M, int64_t N, int64_t K, int32_t dtype, void* stream)
{
    return run(h, single(A, B, C, M, N, K, dtype), stream);
}

int64_t gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t dtype)
{
    // any distinct, far apart, 16-byte aligned addresses: the choice looks
    // only at alignment
    const uintptr_t base = (uintptr_t)1 << 44;
    const Problem p = single(reinterpret_cast<const void*>(base), reinterpret_cast<const void*>(2 * base),
                             reinterpret_cast<void*>(3 * base), M, N, K, dtype);
    if (check_args(p) != GEMM_OK) return -1;
    int splits = 1;
    select_ws(p, INT64_MAX, splits);
    return splits > 1 ? (int64_t)splits * M * N * 4 : 0;
}

gemm_status_t gemm_run_ws(gemm_handle_t h, const void* A, const void* B, void* C, int64_t M, int64_t N,
                          int64_t K, int32_t dtype, void* workspace, int64_t workspace_bytes, void* stream)
{
    return run_ws(h, single(A, B, C, M, N, K, dtype), workspace, workspace_bytes, stream);
}

gemm_status_t gemm_run_noalloc(gemm_handle_t h, const void* A, const void* B, void* C, int64_t M, int64_t N,
                               int64_t K, int32_t dtype, void* stream)
{
    return run_noalloc(h, single(A, B, C, M, N, K, dtype), stream);
}

gemm_status_t gemm_run_clocked(gemm_handle_t h, const void* A, const void* B, void* C, int64_t M, int64_t N,
                               int64_t K, int32_t dtype, void* clk, void* stream)
{
    return run_clocked(h, single(A, B, C, M, N, K, dtype), clk, stream);
}

gemm_status_t gemm_run_ws_config(gemm_handle_t h, const void* A, const void* B, void* C, int64_t M,
                                 int64_t N, int64_t K, int32_t dtype, int32_t config_id, int32_t splits,
                                 void* workspace, int64_t workspace_bytes, void* stream)
{
    return run_ws_config(h, single(A, B, C, M, N, K, dtype), config_id, splits, workspace, workspace_bytes,
                         stream);
}

int32_t gemm_select_config_ws(const void* A, const void* B, const void* C, int64_t M, int64_t N, int64_t K,
                              int32_t dtype, int64_t workspace_bytes, int32_t* splits)
{
    const Problem p = single(A, B, const_cast<void*>(C), M, N, K, dtype);
    if (check_args(p) != GEMM_OK || workspace_bytes < 0) return -1;
    int s = 1;
    const int c = select_ws(p, workspace_bytes, s);
    if (splits) *splits = s;
    return c;
}

gemm_status_t gemm_run_batched(gemm_handle_t h, const void* A, const void* B, void* C, int64_t batch,
                               int64_t M, int64_t N, int64_t K, int64_t stride_a, int64_t stride_b,
                               int64_t stride_c, int32_t dtype, void* stream)
{
    return run(h, Problem{A, B, C, M, N, K, dtype, batch, stride_a, stride_b, stride_c}, stream);
}

gemm_status_t gemm_run_config(gemm_handle_t h, const void* A, const void* B, void* C,
                              int64_t M, int64_t N, int64_t K, int32_t dtype,
                              int32_t config_id, void* stream)
{
    return run_config(h, single(A, B, C, M, N, K, dtype), config_id, stream);
}

gemm_status_t gemm_run_batched_config(gemm_handle_t h, const void* A, const void* B, void* C,
                                      int64_t batch, int64_t M, int64_t N, int64_t K,
                                      int64_t stride_a, int64_t stride_b, int64_t stride_c,
                                      int32_t dtype, int32_t config_id, void* stream)
{
    return run_config(h, Problem{A, B, C, M, N, K, dtype, batch, stride_a, stride_b, stride_c},
                      config_id, stream);
}

}  // extern "C"
