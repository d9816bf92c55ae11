// Router: logits, scores, top-k selection and gate weights.
//
// llm-infra-atlas "02 Fine-grained MoE", section 2.1 (DeepSeekMoE Eq. 7-8): l = u_t . e_i,
// s = softmax(l), g = s on the top-K set.  Section 3.1 (DeepSeek-V3 Eq. 12-15): s = sigmoid(l),
// g = s / sum of the selected s.  ibossgateway chapter 7, section 7.4: the ranking uses
// s + b_i, the weights the raw s.  tomabc explainer: the masked softmax gate.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// ---------------------------------------------------------------- logits, bf16 (MFMA)
// Tile: TB*16 tokens x 64 experts per workgroup.  Wave w owns experts [e0 + 16 w, +16) and all
// TB token blocks; v_mfma_f32_16x16x32_bf16 with both operands read straight from global
// memory as 16-byte rows (u and the centroids are both K-contiguous).
template <int TB>
__global__ __launch_bounds__(256) void k_logits_bf16(const uint16_t* __restrict__ u,
                                                     const uint16_t* __restrict__ e,
                                                     float* __restrict__ logits, int T, int H, int N) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int t0 = blockIdx.x * (TB * 16);
    const int e0 = blockIdx.y * 64 + w * 16;
    if (e0 >= N) return;
    const int r = lane & 15;
    const int kq = (lane >> 4) * 8;
    const uint16_t* ap[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) {
        int t = min(t0 + b * 16 + r, T - 1);
        ap[b] = u + (size_t)t * H + kq;
    }
    const int ex = min(e0 + r, N - 1);
    const uint16_t* bp = e + (size_t)ex * H + kq;
    f32x4 acc[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < H; k += 32) {
        uint4 bv = *reinterpret_cast<const uint4*>(bp + k);
#pragma unroll
        for (int b = 0; b < TB; ++b) {
            uint4 av = *reinterpret_cast<const uint4*>(ap[b] + k);
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                             __builtin_bit_cast(bf16x8, bv), acc[b], 0, 0, 0);
        }
    }
    // D[i][j]: j = lane % 16 (expert), i = 4 * (lane / 16) + q (token)
    const int col = e0 + r;
    if (col < N) {
#pragma unroll
        for (int b = 0; b < TB; ++b)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                int t = t0 + b * 16 + (lane >> 4) * 4 + q;
                if (t < T) logits[(size_t)t * N + col] = acc[b][q];
            }
    }
}

// ---------------------------------------------------------------- logits, bf16, few tokens
// Decode-sized T: a workgroup computes 16 tokens x 16 experts; its four waves take contiguous
// quarters of H and keep eight 32-wide k-chunks of loads in flight (latency, not bandwidth, bounds
// this shape), then the four partial sums are added in a fixed order through LDS.
__global__ __launch_bounds__(256) void k_logits_bf16_sk(const uint16_t* __restrict__ u,
                                                        const uint16_t* __restrict__ e,
                                                        float* __restrict__ logits, int T, int H, int N) {
    __shared__ f32x4 part[4][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, kq = (lane >> 4) * 8;
    const int t = min((int)blockIdx.x * 16 + r, T - 1);
    const int ex = min((int)blockIdx.y * 16 + r, N - 1);
    const uint16_t* ap = u + (size_t)t * H + kq;
    const uint16_t* bp = e + (size_t)ex * H + kq;
    const int nch = H / 32;
    const int c0 = nch * w / 4, c1 = nch * (w + 1) / 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int c = c0;
    for (; c + 8 <= c1; c += 8) {
        uint4 av[8], bv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            av[j] = *reinterpret_cast<const uint4*>(ap + (c + j) * 32);
            bv[j] = *reinterpret_cast<const uint4*>(bp + (c + j) * 32);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[j]),
                                                          __builtin_bit_cast(bf16x8, bv[j]), acc, 0, 0, 0);
    }
    for (; c < c1; ++c) {
        const uint4 av = *reinterpret_cast<const uint4*>(ap + c * 32);
        const uint4 bv = *reinterpret_cast<const uint4*>(bp + c * 32);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv),
                                                      acc, 0, 0, 0);
    }
    part[w][lane] = acc;
    __syncthreads();
    if (w == 0) {
        f32x4 v = part[0][lane];
#pragma unroll
        for (int q = 1; q < 4; ++q) v += part[q][lane];
        // D[i][j]: j = lane % 16 (expert), i = 4 * (lane / 16) + q (token)
        const int col = blockIdx.y * 16 + r;
        if (col < N) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int tt = blockIdx.x * 16 + (lane >> 4) * 4 + q;
                if (tt < T) logits[(size_t)tt * N + col] = v[q];
            }
        }
    }
}

// ---------------------------------------------------------------- logits, fp32 (VALU)
__global__ __launch_bounds__(256) void k_logits_f32(const float* __restrict__ u, const float* __restrict__ e,
                                                    float* __restrict__ logits, int T, int H, int N) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)T * N) return;
    const int t = (int)(idx / N), i = (int)(idx % N);
    const float* a = u + (size_t)t * H;
    const float* b = e + (size_t)i * H;
    float acc = 0.f;
    for (int h = 0; h < H; ++h) acc = fmaf(a[h], b[h], acc);
    logits[idx] = acc;
}

// Below 32768 tokens the 128 x 128 tiles of the logits GEMM (T / 128 x N / 128 of them) leave half of
// its two-workgroups-per-CU slots empty; two reduction halves fill them.
bool logits_split(int dtype, int T, int H, int N) {
    return dtype != 0 && T >= 1024 && T < 32768 && N % 64 == 0 && H % 128 == 0;
}

hipError_t launch_logits(int dtype, const void* u, const void* e, float* logits, int T, int H, int N,
                         hipStream_t s) {
    if (T == 0 || N == 0) return hipSuccess;
    if (dtype == 0) {
        long long n = (long long)T * N;
        hipLaunchKernelGGL(k_logits_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)u,
                           (const float*)e, logits, T, H, N);
    } else if (T >= 1024 && N % 64 == 0) {
        // prefill: the tiled MFMA GEMM (LDS-staged, fp32 output) over u [T, H] x e [N, H]^T; split, the
        // two halves of H are two dense groups writing [T, 2N] side by side
        const bool split = logits_split(dtype, T, H, N);
        GemmParams p{};
        p.A = u;
        p.lda = H;
        p.a_nrows = T;
        p.B = e;
        p.ldb = H;
        p.K = split ? H / 2 : H;
        p.Kseg = p.K;
        p.sA_group = split ? H / 2 : 0;
        p.sB_group = split ? H / 2 : 0;
        p.N = N;
        p.M_dense = T;
        p.G = split ? 2 : 1;
        p.max_rows = T;
        p.C = logits;
        p.ldc = split ? 2 * N : N;
        p.sC_group = N;
        return launch_gemm(1, GM_F32OUT, p, s);
    } else if (T < 1024) {
        // one kernel (one summation order) for every T below the GEMM path, so a token's logits do
        // not depend on how the tokens are batched
        dim3 grid((T + 15) / 16, (N + 15) / 16);
        hipLaunchKernelGGL(k_logits_bf16_sk, grid, dim3(256), 0, s, (const uint16_t*)u, (const uint16_t*)e,
                           logits, T, H, N);
    } else if (T >= 2048) {
        dim3 grid((T + 63) / 64, (N + 63) / 64);
        hipLaunchKernelGGL(k_logits_bf16<4>, grid, dim3(256), 0, s, (const uint16_t*)u, (const uint16_t*)e,
                           logits, T, H, N);
    } else {
        dim3 grid((T + 15) / 16, (N + 63) / 64);
        hipLaunchKernelGGL(k_logits_bf16<1>, grid, dim3(256), 0, s, (const uint16_t*)u, (const uint16_t*)e,
                           logits, T, H, N);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- selection (one wavefront per token)
// Keys are packed as (order-preserving key bits << 32) | (~index) so that one 64-bit max picks
// the largest key and, among equal keys, the lower expert index.
__device__ __forceinline__ uint32_t order_bits(float f) {
    uint32_t b = __float_as_uint(f + 0.0f);  // -0 -> +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ unsigned long long pack_key(float key, int idx) {
    return ((unsigned long long)order_bits(key) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ __forceinline__ int unpack_idx(unsigned long long p) {
    return (int)(0xFFFFFFFFu - (uint32_t)(p & 0xFFFFFFFFull));
}

// Wave-wide maximum of a 32-bit value, left in a scalar register: DPP permutes inside each row of 16
// lanes (pairs, quads, half-rows, rows), then the four row maxima read out with readlane.  Every lane
// of the wave must be active.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));   // row_mirror
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// Index of the largest packed key of the wave (each lane offers its own best; 0 = nothing): the
// largest key bits first, then, only when several lanes hold them, the largest ~index among those.
__device__ __forceinline__ int wave_argmax(unsigned long long best) {
    const uint32_t hi = (uint32_t)(best >> 32), lo = (uint32_t)best;
    const uint32_t mh = wave_max_u32(hi);
    const unsigned long long m = __ballot(hi == mh);
    uint32_t ml;
    if (__popcll(m) == 1) ml = __builtin_amdgcn_readlane(lo, __ffsll((long long)m) - 1);
    else ml = wave_max_u32(hi == mh ? lo : 0u);
    return (int)(0xFFFFFFFFu - ml);
}

// One selection round over the packed keys pk (entry j of a lane: expert lane + 64 j; 0 = taken or
// absent): returns the winner and clears its entry.
template <int NPL>
__device__ __forceinline__ int take_best(unsigned long long (&pk)[NPL], int lane) {
    unsigned long long b = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) b = pk[j] > b ? pk[j] : b;
    const int idx = wave_argmax(b);
    const int slot = idx >> 6;   // wave-uniform
#pragma unroll
    for (int j = 0; j < NPL; ++j)
        if (j == slot && lane == (idx & 63)) pk[j] = 0;
    return idx;
}

template <int NPL>
__global__ __launch_bounds__(256) void k_select(SelectArgs a) {
    __shared__ float sh_key[4][NPL * 64];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int t_raw = blockIdx.x * 4 + wv;
    const bool active = t_raw < a.T;
    const int t = active ? t_raw : a.T - 1;
    const int N = a.N;

    float l[NPL], key[NPL], s[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int i = lane + 64 * j;
        l[j] = i >= N ? -INFINITY
                      : a.split ? a.logits[(size_t)t * 2 * N + i] + a.logits[(size_t)t * 2 * N + N + i]
                                : a.logits[(size_t)t * N + i];
    }
    float lmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < NPL; ++j) lmax = fmaxf(lmax, l[j]);
    lmax = wave_max(lmax);
    float z = 0.f;
    if (a.gating == 1) {
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            const int i = lane + 64 * j;
            s[j] = 1.0f / (1.0f + expf(-l[j]));
            key[j] = s[j] + ((a.bias && i < N) ? a.bias[i] : 0.0f);
        }
    } else {
        // softmax modes rank by the logits (softmax is monotone)
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            s[j] = (lane + 64 * j < N) ? expf(l[j] - lmax) : 0.0f;
            key[j] = l[j];
            z += s[j];
        }
        z = wave_sum(z);
    }
    unsigned long long pk[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) pk[j] = lane + 64 * j < N ? pack_key(key[j], lane + 64 * j) : 0ull;

    if (a.n_group > 0) {
        // group scores: sum of the keys of each contiguous group, in index order
        // (softmax modes: the probabilities s, as ranked; sigmoid mode: s + b)
#pragma unroll
        for (int j = 0; j < NPL; ++j) sh_key[wv][lane + 64 * j] = a.gating == 1 ? key[j] : s[j] / z;
        __syncthreads();
        const int per = N / a.n_group;
        float gs = 0.f;
        if (lane < a.n_group)
            for (int q = 0; q < per; ++q) gs += sh_key[wv][lane * per + q];
        unsigned long long gpk[1] = {lane < a.n_group ? pack_key(gs, lane) : 0ull};
        unsigned long long chosen = 0;
        for (int r = 0; r < a.topk_group; ++r) chosen |= 1ull << take_best<1>(gpk, lane);
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            const int i = lane + 64 * j;
            if (!((chosen >> (i / per)) & 1ull)) pk[j] = 0;
        }
    }
    for (int r = 0; r < a.mask_r; ++r) take_best<NPL>(pk, lane);

    int my_idx = 0;
    for (int k = 0; k < a.K; ++k) {
        const int idx = take_best<NPL>(pk, lane);
        if (lane == k) my_idx = idx;
    }
    // the logit and score of this lane's pick, from its owner lane
    float my_l = 0.f, my_s = 0.f;
    {
        const int src = my_idx & 63, slot = my_idx >> 6;
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            const float lj = __shfl(l[j], src), sj = __shfl(s[j], src);
            if (slot == j) {
                my_l = lj;
                my_s = sj;
            }
        }
    }
    const bool mine = lane < a.K;
    float g;
    if (a.gating == 0) {
        g = my_s / z;
    } else if (a.gating == 1) {
        const float sum = wave_sum(mine ? my_s : 0.0f);
        g = sum > 0.0f ? my_s / sum : 1.0f / (float)a.K;
    } else {
        const float m0 = __shfl(my_l, 0);
        const float ex = mine ? expf(my_l - m0) : 0.0f;
        g = ex / wave_sum(ex);
    }
    if (active && mine) {
        a.topk_idx[(size_t)t * a.K + lane] = my_idx;
        a.topk_w[(size_t)t * a.K + lane] = g;
    }
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
    if (a.T == 0 || a.K == 0) return hipSuccess;
    dim3 grid((a.T + 3) / 4), block(256);
    const int npl = (a.N + 63) / 64;
    if (npl <= 1) hipLaunchKernelGGL(k_select<1>, grid, block, 0, s, a);
    else if (npl <= 2) hipLaunchKernelGGL(k_select<2>, grid, block, 0, s, a);
    else if (npl <= 4) hipLaunchKernelGGL(k_select<4>, grid, block, 0, s, a);
    else if (npl <= 8) hipLaunchKernelGGL(k_select<8>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(k_select<16>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
