// hstu_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// Wavefronts are 64 lanes; the MFMA layouts the kernels use are described
// with the 32x32x16 helper in tile_ops.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// SiLU(x) = x / (1 + 2^(-x log2 e)) with the hardware exp2 and reciprocal
// (both ~1 ulp).  x -> -inf gives -0, x -> +inf gives x.
__device__ __forceinline__ float silu_fast(float x) {
    float e = __builtin_amdgcn_exp2f(-x * kLog2e);
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// Accurate SiLU for the fp32 path.
__device__ __forceinline__ float silu_precise(float x) { return x / (1.0f + expf(-x)); }

// |a - b| + c on unsigned 32-bit values in one VALU instruction.
__device__ __forceinline__ uint32_t sad_u32(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    asm("v_sad_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Pack two floats into two bf16 (round to nearest even) in one dword.
// (A vector conversion, so that it becomes a single v_cvt_pk_bf16_f32.)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t bits) {
    return __uint_as_float((uint32_t)bits << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Number of significant bits of a 64-bit value (0 for 0).
__device__ __forceinline__ int bit_length_u64(uint64_t x) { return x == 0 ? 0 : 64 - __clzll(x); }

// Wave-wide sum over 64 lanes.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

}  // namespace hstu
