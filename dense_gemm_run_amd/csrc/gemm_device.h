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

}  // namespace dgr
