// fa_device.h -- device-side building blocks shared by the forward and backward kernels:
// vector types, the 32x32x16 MFMA and fp32 -> fp16/bf16 packing per element type, and the
// direct buffer-to-LDS load.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// ---------------------------------------------------------------- element types

template <typename T> struct Elem;

template <> struct Elem<_Float16> {
    static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    }
    // round-to-nearest-even fp32 -> fp16, two values packed in one dword (x in the low half)
    static __device__ __forceinline__ unsigned pack2(float x, float y)
    {
        const f32x2 v = {x, y};
        return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2));
    }
    // the two fp16 values of a dword (low half first), widened exactly
    static __device__ __forceinline__ f32x2 unpack2(unsigned w)
    {
        return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
    }
};

template <> struct Elem<__bf16> {
    static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
    static __device__ __forceinline__ unsigned pack2(float x, float y)
    {
        const f32x2 v = {x, y};
        return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
    }
    static __device__ __forceinline__ f32x2 unpack2(unsigned w)
    {
        return __builtin_convertvector(__builtin_bit_cast(bf16x2, w), f32x2);
    }
};

// 16 bytes per lane from a buffer straight into LDS: lane i writes dst + 16 i (dst is uniform).
// The builtin only exists for the device; the host pass never sees the call.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rs, lds_void *dst, unsigned voffset)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voffset, 0, 0, 0);
#endif
}

}  // namespace fa
