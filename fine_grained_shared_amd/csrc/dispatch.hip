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

// One workgroup: column-wise exclusive prefix over chunks (in place, turned into absolute
// segment bases), per-expert totals, and offsets = exclusive prefix of the totals.
__global__ __launch_bounds__(1024) void k_scan(int32_t* __restrict__ cc, int nchunk, int N,
                                               int32_t* __restrict__ offsets) {
    __shared__ int32_t tot[1024];
    __shared__ int32_t wsum[16];
    const int e = threadIdx.x;
    int run = 0;
    if (e < N) {
        for (int c = 0; c < nchunk; ++c) {
            const int v = cc[(size_t)c * N + e];
            cc[(size_t)c * N + e] = run;
            run += v;
        }
    }
    // block-wide exclusive scan of the totals (N <= 1024)
    const int lane = e & 63, w = e >> 6;
    int incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    if (e == 0) {
        int acc = 0;
        for (int q = 0; q < 16; ++q) {
            const int v = wsum[q];
            wsum[q] = acc;
            acc += v;
        }
        tot[0] = acc;
    }
    __syncthreads();
    const int excl = incl - run + wsum[w];
    if (e < N) {
        offsets[e] = excl;
        for (int c = 0; c < nchunk; ++c) cc[(size_t)c * N + e] += excl;
    }
    if (e == 0) offsets[N] = tot[0];
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

template <typename E>
__global__ __launch_bounds__(256) void k_gather(const E* __restrict__ u, const int32_t* __restrict__ row_token,
                                                int R, int H, E* __restrict__ x_perm) {
    // one row per workgroup, 16-byte vectors
    const int r = blockIdx.x;
    if (r >= R) return;
    const int t = row_token[r];
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

hipError_t launch_scan(int32_t* chunk_counts, int nchunk, int N, int32_t* offsets, hipStream_t s) {
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, chunk_counts, nchunk, N, offsets);
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

hipError_t launch_gather(int dtype, const void* u, const int32_t* row_token, int R, int H, void* x_perm,
                         hipStream_t s) {
    if (R == 0) return hipSuccess;
    if (dtype == 0)
        hipLaunchKernelGGL(k_gather<float>, dim3(R), dim3(256), 0, s, (const float*)u, row_token, R, H,
                           (float*)x_perm);
    else
        hipLaunchKernelGGL(k_gather<uint16_t>, dim3(R), dim3(256), 0, s, (const uint16_t*)u, row_token, R, H,
                           (uint16_t*)x_perm);
    return hipGetLastError();
}

}  // namespace moe
