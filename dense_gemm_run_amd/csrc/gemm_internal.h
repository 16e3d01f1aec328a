// Internal declarations shared by the host library and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgr {

// MI355X hands consecutive workgroup ids to its 8 XCDs in turn (id % 8 picks
// the XCD); each XCD has its own L2.
constexpr int kNumXcd = 8;

__host__ __device__ inline int cdiv_i(int a, int b) { return (a + b - 1) / b; }

// Batch index and output tile owned by workgroup `bid` of a grid of
// batch * tiles_m * tiles_n workgroups.
//
// Step 1 (optional, xcd_remap): turn the hardware id into a logical id so
// that the workgroups one XCD runs get consecutive logical ids.  Of the
// first 8*q ids (q = total/8), XCD x runs ids x, x+8, x+16, ...; those become
// logical ids x*q, x*q+1, ...  The last total%8 ids keep their value.
//
// Step 2: logical id p belongs to batch p / (tiles_m*tiles_n) (the third
// program axis of notebook "Triton tiled matmul", the exercises), so the
// consecutive ids of one XCD stay in one or two matrices of the batch.
//
// Step 3: the grouped order of the pages (kernels-book chapter "Matrix
// Multiplication", section "The naive version"; lesson "Matrix
// multiplication", section "Connect to the real implementation"): within a
// matrix, ids fill a band of group_m tile-rows going down the band first,
// then one tile-column to the right, so the workgroups that run together
// share B tiles (and A tiles) in L2.  The last band holds the remaining
// tile-rows.
__host__ __device__ inline void tile_of_block(int bid, int tiles_m, int tiles_n, int batch,
                                              int group_m, bool xcd_remap, int& b, int& tm, int& tn)
{
    const int tiles = tiles_m * tiles_n;
    int p = bid;
    if (xcd_remap) {
        const int total = tiles * batch;
        const int q = total / kNumXcd;
        if (bid < q * kNumXcd) p = (bid % kNumXcd) * q + bid / kNumXcd;
    }
    b = p / tiles;
    p -= b * tiles;
    const int band_size = group_m * tiles_n;
    const int band = p / band_size;
    const int within = p - band * band_size;
    const int top = band * group_m;
    const int rows_left = tiles_m - top;
    const int height = rows_left < group_m ? rows_left : group_m;
    tn = within / height;
    tm = top + (within - tn * height);
}

// Element types.  The 8-bit formats are inputs only: their products are
// written as bf16.
enum Dtype : int32_t { kF32 = 0, kF16 = 1, kBF16 = 2, kFP8E4M3 = 3, kFP8E5M2 = 4 };

struct Config {
    int32_t id;
    int32_t bm, bn, bk;
    int32_t group_m;
    int32_t threads;
    int32_t dtype_mask;
    int32_t needs_vec_align;
    int32_t xcd_remap;
    const char* name;
    int32_t sched;   // pipeline variant of the kernel family (0: its default)
};

// The batch a launch covers: `count` products, matrix b of A (B, C) starting
// `sa` (`sb`, `sc`) elements after matrix b-1.  count = 1 is a single product.
struct Batch {
    int count;
    long long sa, sb, sc;
};

struct LaunchArgs {
    const void* A;
    const void* B;
    void* C;
    int M, N, K;
    int dtype;
    hipStream_t stream;
    Batch batch;
    // split K (one product only): `splits` workgroups per tile, each writing
    // fp32 sums to its M x N slice of `ws`; 1 = the single-pass kernels
    int splits = 1;
    float* ws = nullptr;
    // compute units of the device (persistent grids)
    int cus = 0;
    // measurement aid: clock samples of workgroup 0 (the MFMA tile kernels)
    unsigned long long* clk = nullptr;
};

// Kernel launchers; each returns the hipError_t of the launch.
hipError_t launch_generic(const Config& cfg, const LaunchArgs& a);
hipError_t launch_mfma32x32(const Config& cfg, const LaunchArgs& a);
hipError_t launch_mfma16x16(const Config& cfg, const LaunchArgs& a);
hipError_t launch_gemv(const Config& cfg, const LaunchArgs& a);
hipError_t launch_fp8(const Config& cfg, const LaunchArgs& a);
hipError_t launch_skinny(const Config& cfg, const LaunchArgs& a);
hipError_t launch_fp32(const Config& cfg, const LaunchArgs& a);
hipError_t launch_shortk(const Config& cfg, const LaunchArgs& a);
hipError_t launch_fewrow(const Config& cfg, const LaunchArgs& a);
// Second pass of split K: C = the rounded sum of the `splits` slices of ws.
hipError_t launch_reduce_splits(const LaunchArgs& a);

}  // namespace dgr
