// Dispatch: per-expert histogram, exclusive prefix sum and a stable scatter of the
// (token, slot) pairs into contiguous per-expert segments (llm-infra-atlas "02 Fine-grained
// MoE", section 4: no token dropping, so every selected pair gets a row).
//
// Determinism: positions inside a segment follow (token, slot) order.  Tokens are cut into
// chunks of kChunk; the position of pair (t, k) in expert e's segment is
//   offsets[e] + (pairs of e in earlier chunks) + (tokens of this chunk before t that chose e),
// the last term read from an LDS bitmap with popcounts.  No atomics touch global memory.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// chunk_counts[c * N + e] = number of pairs of chunk c routed to e
__global__ __launch_bounds__(256) void k_count(const int32_t* __restrict__ idx, int T, int K, int N,
                                               int32_t* __restrict__ chunk_counts) {
    extern __shared__ int32_t hist[];
    const int c = blockIdx.x;
    for (int e = threadIdx.x; e < N; e += 256) hist[e] = 0;
    __syncthreads();
    const int t = c * kChunk + threadIdx.x;
    if (t < T) {
        for (int k = 0; k < K; ++k) {
            const int e = idx[(size_t)t * K + k];
            if ((unsigned)e < (unsigned)N) atomicAdd(&hist[e], 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < N; e += 256) chunk_counts[(size_t)c * N + e] = hist[e];
}

// Column-wise exclusive prefix over chunks, as absolute segment bases (bases[c][e] = offsets[e] + pairs
// of e in chunks before c), and offsets = exclusive prefix of the per-expert totals (N <= 1024).
// Workgroup b writes the columns of experts [64 b, 64 b + 64): its 1024 threads take 16 contiguous
// chunk ranges of each of those experts.  Every workgroup first computes all the totals (a table of
// nchunk x N counts, read from L2) and their prefix; workgroup 0 writes offsets.  The counts are only
// read, so the workgroups do not race.  Integer sums: the order does not matter.
__global__ __launch_bounds__(1024) void k_scan(const int32_t* __restrict__ cc, int32_t* __restrict__ bases,
                                               int nchunk, int N, int32_t* __restrict__ offsets) {
    __shared__ int32_t base[1024];      // per-expert totals, then their exclusive prefix
    __shared__ int32_t part[16][64];    // this workgroup's experts: sums of the 16 chunk ranges
    __shared__ int32_t wsum[16];
    const int tid = threadIdx.x;
    if (N <= 0) {
        if (tid == 0 && blockIdx.x == 0) offsets[0] = 0;
        return;
    }
    // 1. totals: thread (e, q) with e = tid % N sums chunks q, q + P, ... (P = 1024 / N of them per expert)
    if (tid < N) base[tid] = 0;
    __syncthreads();
    const int P = 1024 / N;
    if (tid < P * N) {
        const int e = tid % N, q = tid / N;
        int sum = 0, c = q;
        for (; c + 7 * P < nchunk; c += 8 * P) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = cc[(size_t)(c + u * P) * N + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) sum += v[u];
        }
        for (; c < nchunk; c += P) sum += cc[(size_t)c * N + e];
        atomicAdd(&base[e], sum);
    }
    __syncthreads();
    // 2. exclusive prefix of the totals over the experts (thread e holds expert e)
    const int lane = tid & 63, w = tid >> 6;
    const int run = tid < N ? base[tid] : 0;
    int incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int q = 0; q < 16; ++q) {
            const int v = wsum[q];
            wsum[q] = acc;
            acc += v;
        }
        if (blockIdx.x == 0) offsets[N] = acc;
    }
    __syncthreads();
    const int excl = incl - run + wsum[w];
    if (tid < N) {
        base[tid] = excl;
        if (blockIdx.x == 0) offsets[tid] = excl;
    }
    // 3. this workgroup's experts: chunk range r of expert e = 64 b + el
    const int el = tid & 63, r = tid >> 6;
    const int e = blockIdx.x * 64 + el;
    const int L = (nchunk + 15) / 16;
    const int c0 = min(r * L, nchunk), c1 = min(c0 + L, nchunk);
    int rsum = 0;
    if (e < N) {
        int c = c0;
        for (; c + 8 <= c1; c += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = cc[(size_t)(c + u) * N + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) rsum += v[u];
        }
        for (; c < c1; ++c) rsum += cc[(size_t)c * N + e];
    }
    part[r][el] = rsum;
    __syncthreads();
    if (e < N) {
        int start = base[e];
        for (int q = 0; q < r; ++q) start += part[q][el];
        int c = c0;
        for (; c + 8 <= c1; c += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = cc[(size_t)(c + u) * N + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                bases[(size_t)(c + u) * N + e] = start;
                start += v[u];
            }
        }
        for (; c < c1; ++c) {
            const int v = cc[(size_t)c * N + e];
            bases[(size_t)c * N + e] = start;
            start += v;
        }
    }
}

__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ idx, int T, int K, int N,
                                                 const int32_t* __restrict__ chunk_base,
                                                 int32_t* __restrict__ row_token, int32_t* __restrict__ pair_row) {
    extern __shared__ uint32_t bits[];  // [N][kChunk / 32]
    constexpr int W = kChunk / 32;
    const int c = blockIdx.x;
    for (int q = threadIdx.x; q < N * W; q += 256) bits[q] = 0u;
    __syncthreads();
    const int tl = threadIdx.x;
    const int t = c * kChunk + tl;
    if (t < T) {
        for (int k = 0; k < K; ++k) {
            const int e = idx[(size_t)t * K + k];
            if ((unsigned)e < (unsigned)N) atomicOr(&bits[e * W + (tl >> 5)], 1u << (tl & 31));
        }
    }
    __syncthreads();
    if (t < T) {
        for (int k = 0; k < K; ++k) {
            const int e = idx[(size_t)t * K + k];
            if ((unsigned)e >= (unsigned)N) continue;
            int rank = __popc(bits[e * W + (tl >> 5)] & ((1u << (tl & 31)) - 1u));
            for (int q = 0; q < (tl >> 5); ++q) rank += __popc(bits[e * W + q]);
            const int pos = chunk_base[(size_t)c * N + e] + rank;
            row_token[pos] = t;
            pair_row[(size_t)t * K + k] = pos;
        }
    }
}

// The whole dispatch of one chunk (T <= kChunk tokens, a decode step) in one workgroup: the histogram,
// the exclusive prefix over the experts (offsets) and the stable scatter, all through LDS, in place of
// the three launches above.  Positions are the same: offsets[e] + tokens before t in the chunk that
// chose e.
__global__ __launch_bounds__(256) void k_dispatch1(const int32_t* __restrict__ idx, int T, int K, int N,
                                                   int32_t* __restrict__ offsets, int32_t* __restrict__ row_token,
                                                   int32_t* __restrict__ pair_row) {
    constexpr int W = kChunk / 32;
    extern __shared__ uint32_t sh1[];
    int32_t* base = reinterpret_cast<int32_t*>(sh1);   // [N]: counts, then segment starts
    uint32_t* bits = sh1 + N;                          // [N][W]: tokens of the chunk per expert
    __shared__ int32_t wsum[4];
    const int tid = threadIdx.x;
    for (int q = tid; q < N * (W + 1); q += 256) sh1[q] = 0u;
    __syncthreads();
    if (tid < T) {
        for (int k = 0; k < K; ++k) {
            const int e = idx[(size_t)tid * K + k];
            if ((unsigned)e < (unsigned)N) {
                atomicAdd(&base[e], 1);
                atomicOr(&bits[e * W + (tid >> 5)], 1u << (tid & 31));
            }
        }
    }
    __syncthreads();
    // exclusive prefix over the experts: thread tid sums experts [per tid, per (tid + 1)), then a block scan
    const int per = (N + 255) / 256;
    const int e0 = min(tid * per, N), e1 = min(e0 + per, N);
    int run = 0;
    for (int e = e0; e < e1; ++e) run += base[e];
    const int lane = tid & 63, w = tid >> 6;
    int incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int acc = 0;
    for (int q = 0; q < w; ++q) acc += wsum[q];
    int start = acc + incl - run;
    if (tid == 255) offsets[N] = acc + incl;
    __syncthreads();   // every count read before the starts overwrite them
    for (int e = e0; e < e1; ++e) {
        const int c = base[e];
        base[e] = start;
        offsets[e] = start;
        start += c;
    }
    __syncthreads();
    if (tid < T) {
        for (int k = 0; k < K; ++k) {
            const int e = idx[(size_t)tid * K + k];
            if ((unsigned)e >= (unsigned)N) continue;
            int rank = __popc(bits[e * W + (tid >> 5)] & ((1u << (tid & 31)) - 1u));
            for (int q = 0; q < (tid >> 5); ++q) rank += __popc(bits[e * W + q]);
            const int pos = base[e] + rank;
            row_token[pos] = tid;
            pair_row[(size_t)tid * K + k] = pos;
        }
    }
}

// x_perm[r] = u[row_token[r]].  Rows past the last segment (pairs skipped for an out-of-range expert id)
// hold whatever the caller's row_token buffer held: every token index is clamped into [0, T), so the
// gather never reads outside u.
template <typename E>
__global__ __launch_bounds__(256) void k_gather(const E* __restrict__ u, const int32_t* __restrict__ row_token,
                                                int T, int R, int H, E* __restrict__ x_perm) {
    // one row per workgroup, 16-byte vectors
    const int r = blockIdx.x;
    if (r >= R) return;
    const int t = min(max(row_token[r], 0), T - 1);
    const uint4* src = reinterpret_cast<const uint4*>(u + (size_t)t * H);
    uint4* dst = reinterpret_cast<uint4*>(x_perm + (size_t)r * H);
    const int nv = H * (int)sizeof(E) / 16;
    for (int v = threadIdx.x; v < nv; v += 256) dst[v] = src[v];
}

hipError_t launch_count(const int32_t* idx, int T, int K, int N, int32_t* chunk_counts, hipStream_t s) {
    const int nchunk = (T + kChunk - 1) / kChunk;
    if (nchunk == 0) return hipSuccess;
    hipLaunchKernelGGL(k_count, dim3(nchunk), dim3(256), N * sizeof(int32_t), s, idx, T, K, N, chunk_counts);
    return hipGetLastError();
}

hipError_t launch_scan(const int32_t* chunk_counts, int32_t* chunk_base, int nchunk, int N, int32_t* offsets,
                       hipStream_t s) {
    hipLaunchKernelGGL(k_scan, dim3(N > 64 ? (N + 63) / 64 : 1), dim3(1024), 0, s, chunk_counts, chunk_base, nchunk,
                       N, offsets);
    return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* idx, int T, int K, int N, const int32_t* chunk_base,
                          int32_t* row_token, int32_t* pair_row, hipStream_t s) {
    const int nchunk = (T + kChunk - 1) / kChunk;
    if (nchunk == 0 || K == 0) return hipSuccess;
    hipLaunchKernelGGL(k_scatter, dim3(nchunk), dim3(256), (size_t)N * (kChunk / 32) * sizeof(uint32_t), s, idx,
                       T, K, N, chunk_base, row_token, pair_row);
    return hipGetLastError();
}

hipError_t launch_dispatch1(const int32_t* idx, int T, int K, int N, int32_t* offsets, int32_t* row_token,
                            int32_t* pair_row, hipStream_t s) {
    hipLaunchKernelGGL(k_dispatch1, dim3(1), dim3(256), (size_t)N * (kChunk / 32 + 1) * sizeof(uint32_t), s, idx, T,
                       K, N, offsets, row_token, pair_row);
    return hipGetLastError();
}

hipError_t launch_gather(int dtype, const void* u, const int32_t* row_token, int T, int R, int H, void* x_perm,
                         hipStream_t s) {
    if (R == 0 || T == 0) return hipSuccess;
    if (dtype == 0)
        hipLaunchKernelGGL(k_gather<float>, dim3(R), dim3(256), 0, s, (const float*)u, row_token, T, R, H,
                           (float*)x_perm);
    else
        hipLaunchKernelGGL(k_gather<uint16_t>, dim3(R), dim3(256), 0, s, (const uint16_t*)u, row_token, T, R, H,
                           (uint16_t*)x_perm);
    return hipGetLastError();
}

}  // namespace moe
