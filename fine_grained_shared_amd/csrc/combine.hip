// Combine and the balance controller.
//
// Combine (llm-infra-atlas "02 Fine-grained MoE", section 3.1, DeepSeekMoE Eq. 9):
//   out[t] = u[t] + y_shared[t] + sum_k g[t,k] * y_perm[pair_row[t,k]]
// accumulated in fp32 in that fixed order, so the result does not depend on where the rows
// of a token sit in the permuted buffer.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

template <typename E>
__device__ __forceinline__ void load8(const E* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&v)[8]) {
    const uint4 q = ld_once16(p);   // every input row of the combine is read once
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <typename E>
__device__ __forceinline__ void store8(E* p, const float (&v)[8]);
template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* p, const float (&v)[8]) {
    uint4 q;
    q.x = pack2_bf16(v[0], v[1]);
    q.y = pack2_bf16(v[2], v[3]);
    q.z = pack2_bf16(v[4], v[5]);
    q.w = pack2_bf16(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = q;
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&v)[8]) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// grid: (ceil(H / 2048), T); each thread owns 8 consecutive features of one token.
template <typename E>
__global__ __launch_bounds__(256) void k_combine(const E* __restrict__ residual, const E* __restrict__ y_shared,
                                                 const E* __restrict__ y_perm, const int32_t* __restrict__ pair_row,
                                                 const float* __restrict__ topk_w, E* __restrict__ out, int T,
                                                 int H, int K) {
    const int t = blockIdx.y;
    const int h = (blockIdx.x * 256 + threadIdx.x) * 8;
    if (h >= H) return;
    const size_t R = (size_t)T * K;
    float acc[8], v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    if (residual) {
        load8<E>(residual + (size_t)t * H + h, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    if (y_shared) {
        load8<E>(y_shared + (size_t)t * H + h, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    for (int k = 0; k < K; ++k) {
        size_t row = (size_t)(uint32_t)pair_row[(size_t)t * K + k];
        row = row < R ? row : R - 1;
        const float g = topk_w[(size_t)t * K + k];
        load8<E>(y_perm + row * H + h, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, v[i], acc[i]);
    }
    store8<E>(out + (size_t)t * H + h, acc);
}

hipError_t launch_combine(int dtype, const void* residual, const void* y_shared, const void* y_perm,
                          const int32_t* pair_row, const float* topk_w, void* out, int T, int H, int K,
                          hipStream_t s) {
    if (T == 0) return hipSuccess;
    dim3 grid((H + 2047) / 2048, T);
    if (dtype == 0)
        hipLaunchKernelGGL(k_combine<float>, grid, dim3(256), 0, s, (const float*)residual, (const float*)y_shared,
                           (const float*)y_perm, pair_row, topk_w, (float*)out, T, H, K);
    else
        hipLaunchKernelGGL(k_combine<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)residual,
                           (const uint16_t*)y_shared, (const uint16_t*)y_perm, pair_row, topk_w, (uint16_t*)out, T,
                           H, K);
    return hipGetLastError();
}

// Aux-loss-free balance controller (ibossgateway chapter 7, section 7.4): overloaded experts
// (load above the mean T*K/N) get b - gamma, underloaded ones b + gamma; the comparison is
// done in integers (load * N against T * K).
__global__ __launch_bounds__(256) void k_bias_update(const int32_t* __restrict__ offsets, int N, long long T,
                                                     int K, float gamma, float* __restrict__ bias,
                                                     int32_t* __restrict__ counts) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= N) return;
    const int c = offsets[e + 1] - offsets[e];
    if (counts) counts[e] = c;
    const long long lhs = (long long)c * N, total = T * (long long)K;
    float b = bias[e];
    if (lhs > total) b = b - gamma;
    else if (lhs < total) b = b + gamma;
    bias[e] = b;
}

hipError_t launch_bias_update(const int32_t* offsets, int N, long long T, int K, float gamma, float* bias,
                              int32_t* counts, hipStream_t s) {
    if (N == 0) return hipSuccess;
    hipLaunchKernelGGL(k_bias_update, dim3((N + 255) / 256), dim3(256), 0, s, offsets, N, T, K, gamma, bias, counts);
    return hipGetLastError();
}

}  // namespace moe
