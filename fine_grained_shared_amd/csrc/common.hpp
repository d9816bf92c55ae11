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

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32); inputs are finite by contract.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two values in one conversion: lo in bits 15:0, hi in bits 31:16.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 16 bytes read once (routed rows and residual in the combine), with the non-temporal cache policy:
// streaming them past the caches raises the read rate (V3 fused combine 0.96 -> 0.92 ms).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_once16(const void* q) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q));
    return make_uint4(v.x, v.y, v.z, v.w);
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

// SiLU of the bf16 path with the hardware reciprocal (about 1 ulp of fp32) in place of an IEEE
// division: the result is rounded to bf16 (8 significant bits) right after.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Map a workgroup id to a logical tile id so that the workgroups that run on one XCD
// (ids b with equal b % 8, dispatched round-robin) take consecutive logical tiles and
// share operands through that XCD's L2.  nb must be a multiple of 8.
__device__ __forceinline__ int xcd_remap(int b, int nb) { return (b & 7) * (nb >> 3) + (b >> 3); }

}  // namespace moe
