// Router: logits, scores, top-k selection and gate weights.
//
// llm-infra-atlas "02 Fine-grained MoE", section 2.1 (DeepSeekMoE Eq. 7-8): l = u_t . e_i,
// s = softmax(l), g = s on the top-K set.  Section 3.1 (DeepSeek-V3 Eq. 12-15): s = sigmoid(l),
// g = s / sum of the selected s.  ibossgateway chapter 7, section 7.4: the ranking uses
// s + b_i, the weights the raw s.  tomabc explainer: the masked softmax gate.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// ---------------------------------------------------------------- logits, bf16
// Every bf16 logit l[t,i] = u_t . e_i is summed in one fixed order, whatever T is and whichever kernel
// computes it, so a token's logits - and its routing, near ties included - do not depend on how the
// tokens are batched:
//   H is cut into G equal reduction groups - two for long hidden sizes (H >= 4096, H % 128 == 0),
//   else one - each summed as one fp32 chain of v_mfma_f32_32x32x16_bf16 over its 16-deep k-chunks in
//   ascending order, with the token in the A operand and the expert in the B operand; the groups are
//   written side by side as [T, G N] and added by the selection kernel in group order.
// G depends on the layer's shape only, never on T.  Two groups halve the k-loop of the GEMM's few
// 128 x 128 tiles (V3-style prefill router 0.165 -> 0.116 ms) and the chain of the small-batch kernel;
// for H = 2048 one group is faster on both (the partial sums cost traffic: four groups at 512 experts
// and 32768 tokens would write and re-read 268 MB).
// That is the order of the tiled GEMM kernels (GM_F32OUT mode), which compute it for many tokens; the
// kernel below computes it for a few (a decode step) or for expert counts that are not multiples of 64.
int logits_groups(int H) { return H >= 4096 && H % 128 == 0 ? 2 : 1; }

// One wave per 32 tokens x 32 experts of one reduction group: the chain of its k-chunks, operands loaded
// from global memory sixteen chunks ahead (latency bounds this shape: the more bytes in flight per wave,
// the faster).  Lane l feeds row l % 32 (token for A, expert for B) and the k-half l / 32 of each
// 16-deep chunk, as the tiled kernels do.
__global__ __launch_bounds__(64) void k_logits_bf16_dec(const uint16_t* __restrict__ u, const uint16_t* __restrict__ e,
                                                        float* __restrict__ logits, int T, int H, int N, int G) {
    const int lane = threadIdx.x;
    const int g = blockIdx.z, Kg = H / G;
    const int t = min((int)blockIdx.x * 32 + (lane & 31), T - 1);
    const int ex = min((int)blockIdx.y * 32 + (lane & 31), N - 1);
    const uint16_t* ap = u + (size_t)t * H + (size_t)g * Kg + (lane >> 5) * 8;
    const uint16_t* bp = e + (size_t)ex * H + (size_t)g * Kg + (lane >> 5) * 8;
    const int nc = Kg / 16;
    f32x16 acc;
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.f;
    constexpr int D = 16;   // chunks in flight
    uint4 av[D], bv[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {
        const int c = min(j, nc - 1);
        av[j] = *reinterpret_cast<const uint4*>(ap + c * 16);
        bv[j] = *reinterpret_cast<const uint4*>(bp + c * 16);
    }
    for (int c0 = 0; c0 < nc; c0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            if (c0 + j < nc)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[j]),
                                                              __builtin_bit_cast(bf16x8, bv[j]), acc, 0, 0, 0);
            const int c = min(c0 + D + j, nc - 1);   // the next round's chunk (clamped: re-read, unused)
            av[j] = *reinterpret_cast<const uint4*>(ap + c * 16);
            bv[j] = *reinterpret_cast<const uint4*>(bp + c * 16);
        }
    }
    // D[i][j] of the 32 x 32 block: j = lane % 32 (expert), i = 8 (q / 4) + 4 (lane / 32) + q % 4 (token)
    const int col = blockIdx.y * 32 + (lane & 31);
    if (col >= N) return;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int tt = blockIdx.x * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        if (tt < T) logits[(size_t)tt * G * N + (size_t)g * N + col] = acc[q];
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

hipError_t launch_logits(int dtype, const void* u, const void* e, float* logits, int T, int H, int N,
                         hipStream_t s) {
    if (T == 0 || N == 0) return hipSuccess;
    if (dtype == 0) {
        long long n = (long long)T * N;
        hipLaunchKernelGGL(k_logits_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)u,
                           (const float*)e, logits, T, H, N);
        return hipGetLastError();
    }
    const int G = logits_groups(H);
    // The two kernels give the same bits, so the choice is by speed only: the tiled GEMM once its 128 x 128
    // output tiles fill the GPU, else the small-batch kernel (many more, shorter waves).
    const long long gemm_tiles = (long long)((T + 127) / 128) * ((N + 127) / 128) * G;
    if (T >= 1024 && N % 64 == 0 && gemm_tiles >= 256) {
        // many tokens: the tiled MFMA GEMM (fp32 output) over u [T, H] x e [N, H]^T, the reduction groups
        // as dense groups writing [T, G N] side by side
        GemmParams p{};
        p.A = u;
        p.lda = H;
        p.a_nrows = T;
        p.B = e;
        p.ldb = H;
        p.K = H / G;
        p.Kseg = p.K;
        p.sA_group = H / G;
        p.sB_group = H / G;
        p.N = N;
        p.M_dense = T;
        p.G = G;
        p.max_rows = T;
        p.C = logits;
        p.ldc = (long long)G * N;
        p.sC_group = N;
        return launch_gemm(1, GM_F32OUT, p, s);
    }
    dim3 grid((T + 31) / 32, (N + 31) / 32, G);
    hipLaunchKernelGGL(k_logits_bf16_dec, grid, dim3(64), 0, s, (const uint16_t*)u, (const uint16_t*)e, logits, T, H,
                       N, G);
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

// Scores, selection and gate weights of token t from its logits l (entry j of a lane: expert
// lane + 64 j; -inf past N), by one whole wavefront; the results go to a.topk_idx / a.topk_w when
// `active`.  sh_key: NPL * 64 floats of LDS for this wave (group-limited routing).  Every wave of the
// workgroup calls this the same number of times (a barrier orders sh_key's writes and reads).
template <int NPL>
__device__ __forceinline__ void select_token(const SelectArgs& a, int t, bool active, float (&l)[NPL],
                                             float* sh_key, int lane) {
    const int N = a.N;
    float key[NPL], s[NPL];
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
        for (int j = 0; j < NPL; ++j) sh_key[lane + 64 * j] = a.gating == 1 ? key[j] : s[j] / z;
        __syncthreads();
        const int per = N / a.n_group;
        float gs = 0.f;
        if (lane < a.n_group)
            for (int q = 0; q < per; ++q) gs += sh_key[lane * per + q];
        __syncthreads();   // sh_key is rewritten by this wave's next token
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

// One wavefront per token, logits read from a.logits [T, N].
template <int NPL>
__global__ __launch_bounds__(256) void k_select(SelectArgs a) {
    __shared__ float sh_key[4][NPL * 64];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int t_raw = blockIdx.x * 4 + wv;
    const bool active = t_raw < a.T;
    const int t = active ? t_raw : a.T - 1;
    float l[NPL];
    const float* row = a.logits + (size_t)t * a.groups * a.N;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int i = lane + 64 * j;
        float v = -INFINITY;
        if (i < a.N) {
            v = row[i];
            for (int g = 1; g < a.groups; ++g) v += row[(size_t)g * a.N + i];
        }
        l[j] = v;
    }
    select_token<NPL>(a, t, active, l, sh_key[wv], lane);
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
