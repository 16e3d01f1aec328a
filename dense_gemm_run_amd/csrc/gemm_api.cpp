// Host side of the C ABI declared in include/dense_gemm.h: argument checks,
// the handle, the configuration table, configuration choice and launch.
//
// The contract follows the pages' wrappers (notebook "Triton tiled matmul",
// section "The kernel", and chapter "Fast matrix multiplication", the
// Triton wrapper): [M,K] @ [K,N] -> [M,N], the caller provides C of the input
// type, one 1-D grid of ceil(M/BM)*ceil(N/BN) workgroups, asynchronous launch.
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../include/dense_gemm.h"
#include "gemm_internal.h"

struct gemm_ctx {
    int device;
    int cu_count;
    char arch[64];
};

namespace dgr {
namespace {

enum Kind { kGeneric = 0, kMfma32x32 = 1, kMfma16x16 = 2 };

struct Entry {
    Config cfg;
    Kind kind;
};

// Configuration table.  Entry 0 accepts everything and is the fallback.
// The MFMA entries need 16-byte aligned A, B, C and K, N multiples of 8
// elements (so every 16-byte global access lies wholly inside or wholly
// outside a row).
const Entry kTable[] = {
    {{0, 64, 64, 32, 8, 256, 0x7, 0, 0, "generic_64x64"}, kGeneric},
    {{1, 256, 256, 32, 4, 256, 0x6, 1, 1, "mfma32x32_256x256x32"}, kMfma32x32},
    {{2, 256, 128, 32, 4, 256, 0x6, 1, 1, "mfma32x32_256x128x32"}, kMfma32x32},
    {{3, 128, 128, 32, 4, 256, 0x6, 1, 1, "mfma32x32_128x128x32"}, kMfma32x32},
    {{4, 256, 256, 32, 4, 512, 0x6, 1, 1, "mfma32x32_256x256x32_w8"}, kMfma32x32},
    {{5, 256, 256, 64, 4, 256, 0x6, 1, 1, "mfma32x32_256x256x64"}, kMfma32x32},
    {{6, 256, 256, 32, 4, 256, 0x6, 1, 1, "mfma16x16_256x256x32"}, kMfma16x16},
    {{7, 256, 128, 32, 4, 256, 0x6, 1, 1, "mfma16x16_256x128x32"}, kMfma16x16},
    {{8, 256, 256, 64, 4, 256, 0x6, 1, 1, "mfma16x16_256x256x64"}, kMfma16x16},
    {{9, 256, 128, 64, 4, 256, 0x6, 1, 1, "mfma16x16_256x128x64"}, kMfma16x16},
};
constexpr int kTableSize = sizeof(kTable) / sizeof(kTable[0]);

inline int64_t elem_bytes(int32_t dtype) { return dtype == kF32 ? 4 : 2; }

inline bool overlaps(const void* p, int64_t pbytes, const void* q, int64_t qbytes)
{
    if (pbytes <= 0 || qbytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), a1 = a0 + (uintptr_t)pbytes;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(q), b1 = b0 + (uintptr_t)qbytes;
    return a0 < b1 && b0 < a1;
}

gemm_status_t check_args(const void* A, const void* B, const void* C,
                         int64_t M, int64_t N, int64_t K, int32_t dtype)
{
    if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_VALUE;
    if (dtype != kF32 && dtype != kF16 && dtype != kBF16) return GEMM_ERR_UNSUPPORTED_DTYPE;
    const int64_t lim = INT32_MAX;
    if (M > lim || N > lim || K > lim) return GEMM_ERR_TOO_LARGE;
    const int64_t s = elem_bytes(dtype);
    // each matrix must stay below 2^31 bytes (32-bit byte offsets in the kernels);
    // products of two sizes <= 2^31-1 fit in int64
    const int64_t max_elems = ((int64_t)1 << 31) / s;
    const int64_t a_elems = M * K, b_elems = K * N, c_elems = M * N;
    if (a_elems >= max_elems || b_elems >= max_elems || c_elems >= max_elems)
        return GEMM_ERR_TOO_LARGE;
    if ((a_elems && !A) || (b_elems && !B) || (c_elems && !C)) return GEMM_ERR_INVALID_VALUE;
    if (overlaps(C, c_elems * s, A, a_elems * s) || overlaps(C, c_elems * s, B, b_elems * s))
        return GEMM_ERR_ALIASING;
    return GEMM_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Whether configuration e can run these (already checked) arguments.
bool accepts(const Entry& e, const void* A, const void* B, const void* C,
             int64_t N, int64_t K, int32_t dtype)
{
    if (!((e.cfg.dtype_mask >> dtype) & 1)) return false;
    if (e.cfg.needs_vec_align) {
        const int64_t per16 = 16 / elem_bytes(dtype);
        if (K % per16 || N % per16) return false;
        if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return false;
    }
    return true;
}

// Shape classes.  Small or oddly aligned problems take the generic kernel;
// aligned fp16/bf16 problems take an MFMA kernel with the largest tile that
// still gives every CU work.  For 256x256 tiles that is the 16x16x32 kernel
// (measured 6-9 % faster than the 32x32x16 one at 4096^3 and 8192^3: it runs
// at a higher clock under the power limit).
int select(const void* A, const void* B, const void* C, int64_t M, int64_t N, int64_t K,
           int32_t dtype)
{
    if (M == 0 || N == 0 || K == 0) return 0;
    if (dtype == kF32) return 0;
    if (!accepts(kTable[1], A, B, C, N, K, dtype)) return 0;
    if (M * N * K < (int64_t)128 * 128 * 128) return 0;
    // largest tile that still leaves at least one tile per CU (256 CUs)
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    if (t256 >= 256) return 6;
    const int64_t t128 = ((M + 255) / 256) * ((N + 127) / 128);
    if (t128 >= 256) return 2;
    return 3;
}

gemm_status_t launch(const Entry& e, gemm_handle_t h, const void* A, const void* B, void* C,
                     int64_t M, int64_t N, int64_t K, int32_t dtype, void* stream)
{
    if (!h) return GEMM_ERR_INVALID_VALUE;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return GEMM_ERR_HIP;
    if (cur != h->device) return GEMM_ERR_INVALID_VALUE;
    if (M == 0 || N == 0) return GEMM_OK;
    LaunchArgs la{A, B, C, (int)M, (int)N, (int)K, dtype, static_cast<hipStream_t>(stream)};
    hipError_t err = hipSuccess;
    switch (e.kind) {
    case kGeneric: err = launch_generic(e.cfg, la); break;
    case kMfma32x32: err = launch_mfma32x32(e.cfg, la); break;
    case kMfma16x16: err = launch_mfma16x16(e.cfg, la); break;
    }
    return err == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
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
    gemm_ctx* h = new (std::nothrow) gemm_ctx;
    if (!h) return GEMM_ERR_HIP;
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
    case GEMM_ERR_ALIASING: return "C overlaps A or B";
    case GEMM_ERR_HIP: return "HIP runtime error";
    case GEMM_ERR_CONFIG_MISMATCH: return "configuration does not accept these arguments";
    default: return "unknown status";
    }
}

gemm_status_t gemm_check_args(const void* A, const void* B, const void* C,
                              int64_t M, int64_t N, int64_t K, int32_t dtype)
{
    return check_args(A, B, C, M, N, K, dtype);
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
    if (check_args(A, B, C, M, N, K, dtype) != GEMM_OK) return -1;
    return select(A, B, C, M, N, K, dtype);
}

gemm_status_t gemm_tile_of_block(int32_t id, int64_t M, int64_t N, int64_t block,
                                 int64_t* tile_m, int64_t* tile_n)
{
    if (id < 0 || id >= kTableSize || !tile_m || !tile_n || M <= 0 || N <= 0 ||
        M > INT32_MAX || N > INT32_MAX)
        return GEMM_ERR_INVALID_VALUE;
    const Config& c = kTable[id].cfg;
    const int tiles_m = cdiv_i((int)M, c.bm), tiles_n = cdiv_i((int)N, c.bn);
    if (block < 0 || block >= (int64_t)tiles_m * tiles_n) return GEMM_ERR_INVALID_VALUE;
    int tm, tn;
    tile_of_block((int)block, tiles_m, tiles_n, c.group_m, c.xcd_remap != 0, tm, tn);
    *tile_m = tm;
    *tile_n = tn;
    return GEMM_OK;
}

gemm_status_t gemm_run(gemm_handle_t h, const void* A, const void* B, void* C,
                       int64_t M, int64_t N, int64_t K, int32_t dtype, void* stream)
{
    const gemm_status_t st = check_args(A, B, C, M, N, K, dtype);
    if (st != GEMM_OK) return st;
    return launch(kTable[select(A, B, C, M, N, K, dtype)], h, A, B, C, M, N, K, dtype, stream);
}

gemm_status_t gemm_run_config(gemm_handle_t h, const void* A, const void* B, void* C,
                              int64_t M, int64_t N, int64_t K, int32_t dtype,
                              int32_t config_id, void* stream)
{
    const gemm_status_t st = check_args(A, B, C, M, N, K, dtype);
    if (st != GEMM_OK) return st;
    if (config_id < 0 || config_id >= kTableSize) return GEMM_ERR_INVALID_VALUE;
    const Entry& e = kTable[config_id];
    if (!accepts(e, A, B, C, N, K, dtype)) return GEMM_ERR_CONFIG_MISMATCH;
    return launch(e, h, A, B, C, M, N, K, dtype, stream);
}

}  // extern "C"
