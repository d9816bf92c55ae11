// Device helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even; inputs are finite by contract.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t x = __float_as_uint(f);
    x += 0x7FFFu + ((x >> 16) & 1u);
    return (uint16_t)(x >> 16);
}

// Element access for the two storage types (float, or bf16 bits in uint16_t).
__device__ __forceinline__ float ld_f32(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld_f32(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ void st_f32(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st_f32(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        unsigned long long w = __shfl_xor(v, o);
        v = w > v ? w : v;
    }
    return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Map a workgroup id to a logical tile id so that the workgroups that run on one XCD
// (ids b with equal b % 8, dispatched round-robin) take consecutive logical tiles and
// share operands through that XCD's L2.  nb must be a multiple of 8.
__device__ __forceinline__ int xcd_remap(int b, int nb) { return (b & 7) * (nb >> 3) + (b >> 3); }

}  // namespace moe
