// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 is carried as its 16 raw bits.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));

// Two fp32 values -> one packed bf16 pair (a in the low half), round to
// nearest even (the default rounding mode; denormals kept), with one
// v_cvt_pk_bf16_f32; a NaN stays a NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const floatx2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Element i of an activation vector as fp32 (exact for both dtypes).
template <bool BF16>
__device__ __forceinline__ float load_act(const void* p, int64_t i) {
    if constexpr (BF16) return bf16_bits_to_f32(((const uint16_t*)p)[i]);
    else return ((const float*)p)[i];
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

}  // namespace moe
