// Device-side helpers shared by the MFMA kernels: vector types, buffer
// resources, wait-count immediates and fp32 -> fp16/bf16 packing.
#pragma once

#include <hip/hip_runtime.h>

namespace dgr {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_byte;

// Byte offset past the end of any buffer the kernels build (every matrix is
// below 2^31 bytes): a buffer load at this offset returns zeros.
constexpr unsigned kOOB = 0x80000000u;

// Raw buffer resource over [p, p + bytes); loads outside it return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wavefront are outstanding (gfx9 encoding: vmcnt bits 3:0 and 15:14,
// expcnt and lgkmcnt left at their maximum, i.e. not waited for).
constexpr unsigned waitcnt_vm(unsigned n)
{
    return (n & 15u) | (7u << 4) | (15u << 8) | ((n >> 4) << 14);
}
// ... and the one that waits for all of this wavefront's LDS operations.
constexpr unsigned kWaitLgkm0 = 15u | (7u << 4) | (0u << 8) | (3u << 14);
// ... and the one that waits until at most n (<= 15) of them are outstanding.
constexpr unsigned waitcnt_lgkm(unsigned n) { return 15u | (7u << 4) | ((n > 15u ? 15u : n) << 8) | (3u << 14); }

// Measurement aid: when `clk` is set, thread 0 of workgroup 0 records the
// counter that ticks with the shader clock and the constant 100 MHz counter,
// at entry (at = 0) and after its last store (at = 1), as clk = {clock0,
// clock1, real0, real1}: the clock the kernel ran at, from inside it.
__device__ __forceinline__ void clock_sample(unsigned long long* clk, int at)
{
    if (clk != nullptr && blockIdx.x == 0 && threadIdx.x == 0) {
        const unsigned long long c = __builtin_readcyclecounter();
        const unsigned long long r = __builtin_amdgcn_s_memrealtime();
        clk[at] = c;
        clk[2 + at] = r;
    }
}

// Two fp32 values -> two 16-bit floats (round to nearest even), packed low
// half first.
template <typename T> __device__ __forceinline__ unsigned pack2(float a, float b);
template <> __device__ __forceinline__ unsigned pack2<_Float16>(float a, float b)
{
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(unsigned, v);
}
template <> __device__ __forceinline__ unsigned pack2<__bf16>(float a, float b)
{
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    b2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(unsigned, v);
}

// Epilogue: one wavefront's WM x WN block of fp32 accumulators (tile (bi,
// bj): lane l holds row 16*bi + l%16, columns 16*bj + 4*(l/16) .. +3) is
// rounded to the output type and written to C at (row0, col0) through the
// wavefront's own LDS region `cw` of CW_BYTES: RP rows at a time are staged
// there and read back as whole row segments for 16-byte stores, skipping
// rows >= M and columns >= N.
template <typename T, int WM, int WN, int CW_BYTES>
__device__ __forceinline__ void store_c_block(const f32x4 (&acc)[WM / 16][WN / 16], lds_byte* cw,
                                              int lane, int row0, int col0, int M, int N, T* C)
{
    constexpr int FN = WN / 16;
    constexpr int PR = WN / 8;           // 16-byte pieces per C row
    constexpr int W = 128 / WN;          // C rows per 256-byte bank window
    constexpr int RP = CW_BYTES / (WN * 2);   // rows per pass
    static_assert(W >= 1 && PR <= 16, "wavefront block too wide");
    static_assert(RP % 16 == 0 && WM % RP == 0, "passes must hold whole tile rows");
    // piece p of row r sits at p ^ ((r / W) % PR): the 16 rows one
    // half-wavefront writes (8 bytes per lane, two lanes per piece) and the
    // rows one 16-lane group reads back each cover 16 different bank groups.
    const int q = lane % PR;
    const int col = col0 + q * 8;
#pragma unroll
    for (int pass = 0; pass < WM / RP; ++pass) {
        if (pass) __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // previous pass read back
#pragma unroll
        for (int bi = pass * RP / 16; bi < (pass + 1) * RP / 16; ++bi) {
            const int r = 16 * bi + (lane & 15) - pass * RP;
            const int sw = (r / W) & (PR - 1);
#pragma unroll
            for (int bj = 0; bj < FN; ++bj) {
                const int p = (2 * bj + (lane >> 5)) ^ sw;
                const int h = (lane >> 4) & 1;
                u32x2 v;
                v[0] = pack2<T>(acc[bi][bj][0], acc[bi][bj][1]);
                v[1] = pack2<T>(acc[bi][bj][2], acc[bi][bj][3]);
                *(u32x2 __attribute__((address_space(3)))*)(cw + r * (WN * 2) + p * 16 + h * 8) = v;
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // this wavefront's LDS writes done
#pragma unroll 4
        for (int it = 0; it < RP * PR / 64; ++it) {
            const int r = it * (64 / PR) + lane / PR;
            const int p = q ^ ((r / W) & (PR - 1));
            const u32x4 v = *(const u32x4 __attribute__((address_space(3)))*)(cw + r * (WN * 2) + p * 16);
            const int row = row0 + pass * RP + r;
            // non-temporal: C is not read again, and streaming it past the
            // caches leaves them to the A and B tiles other workgroups still
            // need (bf16 8192^3: 760 against 787 us)
            if (row < M && col < N) __builtin_nontemporal_store(v, (u32x4*)(C + (size_t)row * N + col));
        }
    }
}

// Epilogue of the 32x32 MFMA kernels: one wavefront's WM x WN block of fp32
// accumulators (lane l holds row 32*bi + l%32, columns 32*bj + 8g + 4*(l/32)
// .. +3 of tile (bi, bj) in registers 4g..4g+3) is rounded to the output type
// (round to nearest even) and written to C at (row0, col0) through the
// wavefront's own LDS region `cw` of CW_BYTES: RP rows at a time are staged
// there and read back as whole row segments for 16-byte stores, skipping
// rows >= M and columns >= N.  The caller makes sure no other use of `cw` is
// in flight.
template <typename T, int WM, int WN, int CW_BYTES = WM * WN * 2>
__device__ __forceinline__ void store_c_block_32x32(const f32x16 (&acc)[WM / 32][WN / 32], lds_byte* cw,
                                                    int lane, int row0, int col0, int M, int N, T* C)
{
    constexpr int FN = WN / 32;
    constexpr int RP = CW_BYTES / (WN * 2);   // rows per pass
    static_assert(RP % 32 == 0 && WM % RP == 0, "passes must hold whole tile rows");
    // Row-major in LDS with 16-byte pieces swizzled: piece p of row r sits at
    // p ^ (r % PR) and its two 8-byte halves are swapped when (r / PR) is
    // odd, so the 8-byte writes of 32 lanes (32 rows, one piece-half each)
    // land on distinct banks.
    constexpr int PR = WN / 8;                    // 16-byte pieces per C row
    const int q = lane % PR;
    const int col = col0 + q * 8;
#pragma unroll
    for (int pass = 0; pass < WM / RP; ++pass) {
        if (pass) __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // previous pass read back
#pragma unroll
        for (int bi = pass * RP / 32; bi < (pass + 1) * RP / 32; ++bi) {
            const int r = 32 * bi + (lane & 31) - pass * RP;
#pragma unroll
            for (int bj = 0; bj < FN; ++bj) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int p = (4 * bj + g) ^ (r & (PR - 1));
                    const int h = (lane >> 5) ^ ((r / PR) & 1);
                    u32x2 v;
                    v[0] = pack2<T>(acc[bi][bj][4 * g + 0], acc[bi][bj][4 * g + 1]);
                    v[1] = pack2<T>(acc[bi][bj][4 * g + 2], acc[bi][bj][4 * g + 3]);
                    *(u32x2 __attribute__((address_space(3)))*)(cw + r * (WN * 2) + p * 16 + h * 8) = v;
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // this wavefront's LDS writes done
        // Read back whole row segments: lane -> row it*(64/PR) + lane/PR, piece lane%PR.
#pragma unroll 4
        for (int it = 0; it < RP * PR / 64; ++it) {
            const int r = it * (64 / PR) + lane / PR;
            const int p = q ^ (r & (PR - 1));
            u32x4 v = *(const u32x4 __attribute__((address_space(3)))*)(cw + r * (WN * 2) + p * 16);
            if ((r / PR) & 1) v = __builtin_shufflevector(v, v, 2, 3, 0, 1);
            const int row = row0 + pass * RP + r;
            // non-temporal: C is not read again (see the 16x16 epilogue)
            if (row < M && col < N) __builtin_nontemporal_store(v, (u32x4*)(C + (size_t)row * N + col));
        }
    }
}

}  // namespace dgr
