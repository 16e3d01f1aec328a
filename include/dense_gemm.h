/*
 * dense_gemm.h - dense matrix product C = A·B on an AMD Instinct MI355X
 * (gfx950), behind a plain C ABI.
 *
 * The operation (lesson "Matrix multiplication: reuse the inputs",
 * triton-cuda-lab, section "The three dimensions have different jobs"):
 * A has shape [M,K], B has shape [K,N], C has shape [M,N] and
 *     C[row,col] = sum over inner of A[row,inner] * B[inner,col].
 * A's column count must equal B's row count; that is why K is passed once.
 *
 * Layout: all three matrices are dense and row-major with no padding between
 * rows: element (r,c) of A is at A + r*K + c, of B at B + r*N + c, of C at
 * C + r*N + c (same lesson, "Connect to the real implementation").
 *
 * Types: A, B and C share one element type, fp32, fp16 or bf16 (the output
 * has the input's type, as in chapter "Fast matrix multiplication", the
 * Triton wrapper).  Products are summed in fp32 whatever the input type
 * (notebook "Triton tiled matmul", section "What"), and the fp32 sum is
 * rounded to the output type with round-to-nearest-even.  fp32 inputs are
 * multiplied at full fp32 precision (no reduced-precision input mode).
 * The 8-bit floating-point inputs (the FP8 input path of the same
 * notebook's exercises: the accumulator stays fp32) are the two OCP FP8
 * formats, E4M3 and E5M2, for both A and B; C is then bf16, which holds
 * every product's range, and the fp32 sum is rounded to bf16 (nearest
 * even).  Every product of two such values is exact in fp32.
 *
 * Edges: M, N and K need not be multiples of any tile size.  Out-of-range
 * input elements read as zero (zero padding is neutral for the sum) and only
 * rows < M and columns < N of C are written (chapter "Fast matrix
 * multiplication", section "The CUDA kernel", the zero-padded edges).
 * Alignment of A, B and C never affects results, only which kernel runs.
 *
 * Ownership: the caller allocates A, B and C in device memory of the device
 * the handle was created on and keeps them alive until the stream has
 * finished the call.  The library allocates no device memory and never
 * synchronises: gemm_run only enqueues work on the given stream and returns.
 *
 * Errors: every argument check happens on the host before anything is
 * enqueued; on an error status nothing has been launched and C is untouched.
 * A fault inside a kernel would surface at the caller's next synchronisation,
 * like any asynchronous HIP work.
 */
#ifndef DENSE_GEMM_H
#define DENSE_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of A and B; C has the same type, except for the 8-bit
 * inputs, whose C is bf16. */
typedef enum gemm_dtype {
    GEMM_F32 = 0,      /* IEEE binary32 */
    GEMM_F16 = 1,      /* IEEE binary16 */
    GEMM_BF16 = 2,     /* bfloat16: fp32's exponent, 8-bit significand */
    GEMM_FP8_E4M3 = 3, /* OCP E4M3: bias 7, 3 significand bits, max 448, NaN
                        * S.1111.111, no infinities; C is bf16 */
    GEMM_FP8_E5M2 = 4  /* OCP E5M2: bias 15, 2 significand bits, max 57344,
                        * IEEE-style infinities and NaNs; C is bf16 */
} gemm_dtype_t;

typedef enum gemm_status {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_VALUE = 1,      /* negative size, null pointer with data, null handle, wrong device, bad config id */
    GEMM_ERR_UNSUPPORTED_DTYPE = 2,  /* dtype is not one of gemm_dtype_t */
    GEMM_ERR_UNSUPPORTED_DEVICE = 3, /* no GPU, or the current device is not gfx950 */
    GEMM_ERR_TOO_LARGE = 4,          /* a dimension > 2^31-1, a matrix of 2^31 bytes or more, or a
                                      * launch grid beyond 2^31-1 workgroups or 2^32-1 lanes */
    GEMM_ERR_ALIASING = 5,           /* C's bytes overlap A's or B's (or, batched, another C matrix) */
    GEMM_ERR_HIP = 6,                /* a HIP runtime call failed */
    GEMM_ERR_CONFIG_MISMATCH = 7     /* forced kernel configuration cannot run these arguments */
} gemm_status_t;

/* Opaque, immutable after creation; safe to share between host threads and
 * to use for concurrent calls on different streams. */
typedef struct gemm_ctx* gemm_handle_t;

/* Bind a handle to the device that is current on the calling thread.
 * *out receives the handle (NULL on error).  Fails with
 * GEMM_ERR_UNSUPPORTED_DEVICE when there is no GPU or it is not gfx950, and
 * with GEMM_ERR_INVALID_VALUE when out is NULL. */
gemm_status_t gemm_create(gemm_handle_t* out);

/* Enqueue C = A·B on `stream`.
 *   A      device pointer to M*K elements, row-major [M,K]    (read only)
 *   B      device pointer to K*N elements, row-major [K,N]    (read only)
 *   C      device pointer to M*N elements, row-major [M,N]    (written)
 *   M,N,K  sizes, each >= 0.  M == 0 or N == 0: nothing is written.
 *          K == 0: C is filled with zeros (an empty sum).
 *   dtype  a gemm_dtype_t value, the type of A and B and (8-bit inputs
 *          aside, whose C is bf16) of C.
 *   stream a hipStream_t, or NULL for the null stream.
 * A pointer may be NULL only when its matrix has no elements.  C may not
 * overlap A or B.  The device current on the calling thread must be the
 * handle's device.  Returns GEMM_OK once the work is enqueued. */
gemm_status_t gemm_run(gemm_handle_t h, const void* A, const void* B, void* C,
                       int64_t M, int64_t N, int64_t K, int32_t dtype, void* stream);

/* Enqueue C[b] = A[b]·B[b] for b = 0 .. batch-1 on `stream`: the product
 * above over an outer batch dimension, run as one launch whose workgroups
 * cover every (batch, tile) pair (notebook "Triton tiled matmul", the
 * exercises: a third program axis over the batch).
 *   A, B, C  device pointers to the first matrix of each operand; matrix b
 *            starts at A + b*stride_a, B + b*stride_b, C + b*stride_c
 *            elements, and each matrix is row-major as in gemm_run.
 *   batch    number of products, >= 0 (0: nothing is done).
 *   strides  in elements of their own matrix (one byte for 8-bit A and B,
 *            bf16 elements for their C), >= 0.  A stride of 0 uses the same
 *            matrix for every b (one weight matrix B for a batch of
 *            activations, say).
 *   M,N,K, dtype, stream  as in gemm_run, for every matrix of the batch.
 * Each matrix must stay below 2^31 bytes; strides may be larger.  The C
 * matrices may not overlap each other (stride_c >= M*N when batch > 1), and
 * the span of C (from C to the end of matrix batch-1) may not overlap the
 * span of A or of B: GEMM_ERR_ALIASING.  Other errors and ownership as in
 * gemm_run; gemm_run(h, A, B, C, M, N, K, ...) is the batch = 1 case. */
gemm_status_t gemm_run_batched(gemm_handle_t h, const void* A, const void* B, void* C,
                               int64_t batch, int64_t M, int64_t N, int64_t K,
                               int64_t stride_a, int64_t stride_b, int64_t stride_c,
                               int32_t dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Split K with a caller-provided workspace.
 *
 * A product with few output tiles and a long K (a few hundred rows times a
 * few thousand columns, say) leaves most CUs idle when each tile is one
 * workgroup.  gemm_run_ws may split K over several workgroups per tile: each
 * writes its fp32 sums, unrounded, to its own M x N slice of the workspace,
 * and a second kernel adds the slices in split order and rounds once (the
 * blocked K-loop of lesson "Matrix multiplication", section "Tiles are small
 * rectangles of work", with the per-block contributions summed across
 * workgroups).  The result is bitwise the same on every call for a given
 * configuration and split count, and meets gemm_run's accuracy (fp32 sums,
 * one rounding).  Only products of one matrix split: fp16/bf16 ones, and
 * 8-bit ones of up to 128 rows (their C is bf16 as always).
 * ------------------------------------------------------------------------- */

/* Bytes of workspace gemm_run_ws uses for this product when A, B and C are
 * 16-byte aligned and the workspace is large enough (0: it runs as gemm_run
 * and needs none).  -1 for negative sizes or an unknown dtype. */
int64_t gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t dtype);

/* gemm_run with `workspace` available as scratch:
 *   workspace        device memory on the handle's device, 16-byte aligned,
 *                    owned by the caller, overlapping none of A, B and C;
 *                    NULL when workspace_bytes is 0.
 *   workspace_bytes  its size; when the split this product would use needs
 *                    more (gemm_workspace_size), the call runs as gemm_run.
 * The workspace's contents are overwritten and have no meaning afterwards;
 * calls that may run at the same time (other streams) need distinct
 * workspaces.  Errors as gemm_run, plus GEMM_ERR_INVALID_VALUE for a negative
 * workspace_bytes, a NULL workspace with a nonzero size, or a misaligned
 * workspace, and GEMM_ERR_ALIASING when it overlaps A, B or C. */
gemm_status_t gemm_run_ws(gemm_handle_t h, const void* A, const void* B, void* C,
                          int64_t M, int64_t N, int64_t K, int32_t dtype,
                          void* workspace, int64_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * For callers that cannot allocate: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.
 *
 * gemm_run_noalloc is gemm_run_ws with the library's own scratch in place of
 * the workspace argument: a file-scope device array of
 * GEMM_NOALLOC_SCRATCH_BYTES (16 MiB) in the library, of which every device
 * the library runs on holds one copy until the process ends (gemm_create
 * looks up its address once per device).  The call allocates nothing (no
 * hipMalloc, no allocating library routine) and never synchronises.
 * Arguments, results and errors are gemm_run_ws's with a 16 MiB workspace:
 * the same kernels, split count and bitwise result, except that a product
 * whose split would need more than the array holds is refused with
 * GEMM_ERR_TOO_LARGE before anything is enqueued (the split rule asks for at
 * most 11 MiB: s * M * N * 4 bytes for about 256 workgroups of 64 x 128
 * outputs).  Products that do not split run as gemm_run.
 * Every call on one device shares that device's array, which keeps the last
 * call's contents; nothing in it has to start at zero (each split writes
 * every element of its slice before the reduction reads it).  Calls that may
 * overlap in time on one device (other streams, other host threads) race on
 * the array and must be serialised by the caller.
 * ------------------------------------------------------------------------- */
#define GEMM_NOALLOC_SCRATCH_BYTES (16u << 20)

gemm_status_t gemm_run_noalloc(gemm_handle_t h, const void* A, const void* B, void* C,
                               int64_t M, int64_t N, int64_t K, int32_t dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Measurement aid: the clock a product ran at, which the fraction of the
 * nominal peak needs beside it (notebook "Triton tiled matmul", section
 * "Performance"; under the board's power limit the shader clock of a long
 * MFMA-bound product sits well below the nominal 2.4 GHz, and it moves within
 * microseconds of the load changing, so it has to be read from inside the
 * kernel).
 *
 * gemm_run_clocked is gemm_run (same selection, kernels and result), except
 * that in the MFMA tile kernels (16-bit, 8-bit and fp32 inputs) thread 0 of
 * workgroup 0 samples the counter that ticks with the shader clock and the
 * constant 100 MHz counter at entry and after its last store, and writes
 * clk = {clock0, clock1, real0, real1}: the shader clock in MHz is
 * 100 * (clock1 - clock0) / (real1 - real0).  The other kernels (generic,
 * strip, few-row, matrix-vector, short-K) leave clk untouched, so a caller
 * clears it first.  clk: device memory on the handle's device, 8-byte aligned,
 * 4 x uint64.  Errors as gemm_run, and GEMM_ERR_INVALID_VALUE for a NULL or
 * misaligned clk.
 * ------------------------------------------------------------------------- */
gemm_status_t gemm_run_clocked(gemm_handle_t h, const void* A, const void* B, void* C,
                               int64_t M, int64_t N, int64_t K, int32_t dtype, void* clk, void* stream);

/* Release a handle.  NULL is accepted and ignored.  No work may still be
 * using the handle (enqueued work does not refer to it). */
gemm_status_t gemm_destroy(gemm_handle_t h);

/* Static English text for a status code (never NULL). */
const char* gemm_status_string(int32_t status);

/* ---------------------------------------------------------------------------
 * Introspection.  These touch no device and are safe without a GPU.
 * ------------------------------------------------------------------------- */

/* The status gemm_run would return for these arguments before launching
 * (handle and device checks excluded).  Pointers are only compared, never
 * dereferenced. */
gemm_status_t gemm_check_args(const void* A, const void* B, const void* C,
                              int64_t M, int64_t N, int64_t K, int32_t dtype);

/* As gemm_check_args, for gemm_run_batched's arguments. */
gemm_status_t gemm_check_args_batched(const void* A, const void* B, const void* C, int64_t batch,
                                      int64_t M, int64_t N, int64_t K, int64_t stride_a,
                                      int64_t stride_b, int64_t stride_c, int32_t dtype);

/* Kernel configurations.  A configuration fixes the output tile BM x BN, the
 * K-step BK, the band height GROUP_M of the tile order, the workgroup size,
 * and which element types and alignments it accepts. */
typedef struct gemm_config_info {
    int32_t id;
    int32_t bm, bn, bk;        /* output tile and K-step (the persistent short-K configuration: the largest
                                * K it accepts, staged whole) */
    int32_t group_m;           /* tile-rows walked before moving right */
    int32_t threads;           /* workgroup size */
    int32_t dtype_mask;        /* bit d set: accepts gemm_dtype_t d */
    int32_t needs_vec_align;   /* 1: needs 16-byte aligned A, B, C, and K, N and batch strides that keep every
                                * row of A, B and C a multiple of 16 bytes (in each matrix's element size) */
    int32_t xcd_remap;         /* 1: workgroup ids are remapped so each XCD gets a compact block of tiles */
    char name[40];
} gemm_config_info_t;

/* Number of configurations; ids run from 0 to count-1. */
int32_t gemm_config_count(void);

/* Describe configuration `id`.  GEMM_ERR_INVALID_VALUE for a bad id or NULL. */
gemm_status_t gemm_config_info(int32_t id, gemm_config_info_t* out);

/* The configuration gemm_run picks for these arguments (alignment is read
 * from the pointer values), or -1 when gemm_check_args would fail. */
int32_t gemm_select_config(const void* A, const void* B, const void* C,
                           int64_t M, int64_t N, int64_t K, int32_t dtype);

/* As gemm_select_config, for gemm_run_batched's arguments (the shape class
 * counts the tiles of the whole batch). */
int32_t gemm_select_config_batched(const void* A, const void* B, const void* C, int64_t batch,
                                   int64_t M, int64_t N, int64_t K, int64_t stride_a,
                                   int64_t stride_b, int64_t stride_c, int32_t dtype);

/* Output tile (tile_m, tile_n) computed by workgroup `block` of
 * configuration `id` for an M x N output, evaluated on the host with the
 * same function the kernels use.  Used to test the tile order.  (For the
 * persistent short-K configuration `block` indexes the walk of tiles: its
 * workgroup g of G takes indices g, g + G, g + 2G, ...) */
gemm_status_t gemm_tile_of_block(int32_t id, int64_t M, int64_t N, int64_t block,
                                 int64_t* tile_m, int64_t* tile_n);

/* Batch index and output tile of workgroup `block` of configuration `id`
 * in a batched launch of `batch` M x N outputs (block < batch * tiles). */
gemm_status_t gemm_tile_of_block_batched(int32_t id, int64_t M, int64_t N, int64_t batch,
                                         int64_t block, int64_t* batch_index, int64_t* tile_m,
                                         int64_t* tile_n);

/* ---------------------------------------------------------------------------
 * gemm_run with a forced configuration, for measuring the alternatives.
 * GEMM_ERR_CONFIG_MISMATCH when that configuration does not accept the
 * dtype or the alignment of these arguments; otherwise as gemm_run.
 * ------------------------------------------------------------------------- */
gemm_status_t gemm_run_config(gemm_handle_t h, const void* A, const void* B, void* C,
                              int64_t M, int64_t N, int64_t K, int32_t dtype,
                              int32_t config_id, void* stream);

/* The configuration and split count gemm_run_ws would use with
 * workspace_bytes of workspace (*splits = 1 when it does not split); -1 when
 * the arguments are invalid.  splits may be NULL. */
int32_t gemm_select_config_ws(const void* A, const void* B, const void* C,
                              int64_t M, int64_t N, int64_t K, int32_t dtype,
                              int64_t workspace_bytes, int32_t* splits);

/* gemm_run_ws with a forced configuration and split count.  splits = 1 is
 * gemm_run_config.  splits in 2 .. 64 needs a tile configuration of the
 * 16x16x32 or the 8-bit kernel
 * (GEMM_ERR_CONFIG_MISMATCH otherwise) and splits*M*N*4 bytes of workspace
 * (GEMM_ERR_INVALID_VALUE otherwise); the count actually used is lowered
 * until no split is left without K-steps (K-steps of the configuration's
 * bk).  Other errors as gemm_run_ws. */
gemm_status_t gemm_run_ws_config(gemm_handle_t h, const void* A, const void* B, void* C,
                                 int64_t M, int64_t N, int64_t K, int32_t dtype,
                                 int32_t config_id, int32_t splits,
                                 void* workspace, int64_t workspace_bytes, void* stream);

/* gemm_run_batched with a forced configuration (alignment also covers the
 * strides: with batch > 1 they must be multiples of 16 bytes). */
gemm_status_t gemm_run_batched_config(gemm_handle_t h, const void* A, const void* B, void* C,
                                      int64_t batch, int64_t M, int64_t N, int64_t K,
                                      int64_t stride_a, int64_t stride_b, int64_t stride_c,
                                      int32_t dtype, int32_t config_id, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_GEMM_H */
