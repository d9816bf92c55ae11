// Expert FFNs as grouped GEMMs.
//
// Routed experts (llm-infra-atlas "02 Fine-grained MoE", section 2.1: mN experts of width
// M/m) are groups of consecutive rows of the permuted pair list; the shared experts
// (section 3.1, Eq. 9) are dense groups over all tokens.  Each expert is
//   SwiGLU: y = W2 (SiLU(Wg x) * (Wu x))      ReLU: y = V ReLU(W x + b)   (tomabc explainer)
// computed as an "up" GEMM with the activation fused into its epilogue, then a "down" GEMM.
//
// bf16 path: 128 x 128 x 64 workgroup tiles, 4 waves of 64 x 64 on v_mfma_f32_32x32x16_bf16,
// operands staged through double-buffered LDS.  For SwiGLU the 128 weight rows of a tile are
// 64 gate rows and the 64 matching up rows, so the epilogue has both halves of every output
// element in the same lane.  fp32 path: plain VALU kernels (the tiny fp32 layer only).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDSW = BK + 8;  // padded LDS row (elements)

int gemm_bm(int dtype) { return dtype == 0 ? 1 : BM; }

// Compute units of the current device (cached per device id).
static int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// ---------------------------------------------------------------- tile plan
// tiles[g] = sum_{g' < g} ceil(rows(g') / bm); tiles[G] = total m-tiles.  One workgroup, G <= 1024.
__global__ __launch_bounds__(1024) void k_tile_plan(const int32_t* __restrict__ offsets, int G, int bm,
                                                    int32_t* __restrict__ tiles) {
    __shared__ int32_t wsum[16];
    const int g = threadIdx.x, lane = g & 63, w = g >> 6;
    int v = 0;
    if (g < G) {
        const int rows = offsets[g + 1] - offsets[g];
        v = rows > 0 ? (rows + bm - 1) / bm : 0;
    }
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int x = __shfl_up(incl, o);
        if (lane >= o) incl += x;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    if (g == 0) {
        int acc = 0;
        for (int q = 0; q < 16; ++q) {
            const int x = wsum[q];
            wsum[q] = acc;
            acc += x;
        }
        tiles[G] = acc;
    }
    __syncthreads();
    if (g < G) tiles[g] = wsum[w] + incl - v;
}

hipError_t launch_tile_plan(const int32_t* offsets, int G, int bm, int32_t* tiles, hipStream_t s) {
    hipLaunchKernelGGL(k_tile_plan, dim3(1), dim3(1024), 0, s, offsets, G, bm, tiles);
    return hipGetLastError();
}

// ---------------------------------------------------------------- tile decode
struct TileInfo {
    int g, row0, rows, nt;
};

__device__ __forceinline__ bool decode_tile(const GemmParams& p, int NT, int bm, int L, TileInfo& ti) {
    if (p.offsets) {
        const int total = p.tiles[p.G];
        if (L >= total * NT) return false;
        const int mt = L / NT;  // only for the binary search: tiles[g] * NT <= L  <=>  tiles[g] <= L / NT
        int lo = 0, hi = p.G;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (p.tiles[mid] <= mt) lo = mid;
            else hi = mid;
        }
        const int g = lo;
        const int t0 = p.tiles[g], nm = p.tiles[g + 1] - t0;
        const int Lg = L - t0 * NT;
        ti.g = g;
        ti.nt = Lg / nm;
        const int ml = Lg - ti.nt * nm;
        ti.row0 = p.offsets[g] + ml * bm;
        ti.rows = min(bm, p.offsets[g + 1] - ti.row0);
    } else {
        const int nm = (p.M_dense + bm - 1) / bm;
        const int per = nm * NT;
        if (L >= p.G * per) return false;
        ti.g = L / per;
        const int Lg = L - ti.g * per;
        ti.nt = Lg / nm;
        const int ml = Lg - ti.nt * nm;
        ti.row0 = ml * bm;
        ti.rows = min(bm, p.M_dense - ti.row0);
    }
    return true;
}

// ---------------------------------------------------------------- bf16 MFMA grouped GEMM
// Persistent: the grid holds two workgroups per CU; the workgroups of one XCD walk a
// contiguous range of the tile list (so concurrently running tiles of an XCD share weight
// and activation tiles in its L2), strided by the number of workgroups on that XCD.
// Pipeline: k-tile kt+2 is fetched into registers while k-tile kt is multiplied out of LDS
// and k-tile kt+1 waits in the other register set, so each global load has two iterations
// to arrive.  Epilogues stage the fp32 tile through LDS and store 16-byte vectors.
constexpr int EPW = BN + 4;  // fp32 staging row (floats)
constexpr int kSmemBytes = 2 * (BM + BN) * LDSW * 2;
static_assert(BM * EPW * 4 <= kSmemBytes, "epilogue staging must fit in the operand buffers");

// Global -> register staging of one k-tile (4 A rows and 4 weight rows of 16 bytes per
// thread), and register -> LDS.  Macros over named registers keep the staging in VGPRs.
#define MOE_STAGE_DECL(S) uint4 S##a0, S##a1, S##a2, S##a3, S##b0, S##b1, S##b2, S##b3
#define MOE_STAGE_LOAD(S, k, bo)                                   \
    do {                                                           \
        S##a0 = *reinterpret_cast<const uint4*>(ag0 + (k));        \
        S##a1 = *reinterpret_cast<const uint4*>(ag1 + (k));        \
        S##a2 = *reinterpret_cast<const uint4*>(ag2 + (k));        \
        S##a3 = *reinterpret_cast<const uint4*>(ag3 + (k));        \
        S##b0 = *reinterpret_cast<const uint4*>(bg0 + (bo));       \
        S##b1 = *reinterpret_cast<const uint4*>(bg1 + (bo));       \
        S##b2 = *reinterpret_cast<const uint4*>(bg2 + (bo));       \
        S##b3 = *reinterpret_cast<const uint4*>(bg3 + (bo));       \
    } while (0)
#define MOE_STAGE_STORE(S, buf)                                            \
    do {                                                                   \
        *reinterpret_cast<uint4*>(&sA[buf][lr][kc]) = S##a0;              \
        *reinterpret_cast<uint4*>(&sA[buf][lr + 32][kc]) = S##a1;         \
        *reinterpret_cast<uint4*>(&sA[buf][lr + 64][kc]) = S##a2;         \
        *reinterpret_cast<uint4*>(&sA[buf][lr + 96][kc]) = S##a3;         \
        *reinterpret_cast<uint4*>(&sB[buf][lr][kc]) = S##b0;              \
        *reinterpret_cast<uint4*>(&sB[buf][lr + 32][kc]) = S##b1;         \
        *reinterpret_cast<uint4*>(&sB[buf][lr + 64][kc]) = S##b2;         \
        *reinterpret_cast<uint4*>(&sB[buf][lr + 96][kc]) = S##b3;         \
    } while (0)

__device__ __forceinline__ void mma_tile(f32x16& c00, f32x16& c01, f32x16& c10, f32x16& c11,
                                         const uint16_t (*sa)[LDSW], const uint16_t (*sb)[LDSW], int arow, int br0,
                                         int br1, int lane) {
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
        const int ko = s * 16 + (lane >> 5) * 8;
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&sa[arow + (lane & 31)][ko]);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&sa[arow + 32 + (lane & 31)][ko]);
        const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(&sb[br0 + (lane & 31)][ko]);
        const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(&sb[br1 + (lane & 31)][ko]);
        c00 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c00, 0, 0, 0);
        c01 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, c01, 0, 0, 0);
        c10 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, c10, 0, 0, 0);
        c11 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c11, 0, 0, 0);
    }
}

__device__ __forceinline__ uint4 pack8_bf16(const float (&v)[8]) {
    uint4 o;
    o.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    o.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    o.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
    o.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
    return o;
}

__device__ __forceinline__ void add8_bf16(float (&v)[8], uint4 q) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] += __uint_as_float(w[e] << 16);
        v[2 * e + 1] += __uint_as_float(w[e] & 0xFFFF0000u);
    }
}

__device__ __forceinline__ void fma8_bf16(float (&v)[8], float g, uint4 q) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] = fmaf(g, __uint_as_float(w[e] << 16), v[2 * e]);
        v[2 * e + 1] = fmaf(g, __uint_as_float(w[e] & 0xFFFF0000u), v[2 * e + 1]);
    }
}

template <int MODE>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, const TileInfo& ti, unsigned char* smem) {
    auto sA = reinterpret_cast<uint16_t(*)[BM][LDSW]>(smem);
    auto sB = reinterpret_cast<uint16_t(*)[BN][LDSW]>(smem + 2 * BM * LDSW * 2);
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
    const int lr = tid >> 3;       // 0..31: row handled by this thread in each 32-row slab
    const int kc = (tid & 7) * 8;  // element offset of this thread's 16-byte chunk

    const uint16_t* A = (const uint16_t*)p.A;
    const uint16_t* Bg = (const uint16_t*)p.B + (size_t)ti.g * p.sB_group;
    const uint16_t* ag[4];
    const uint16_t* bg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = min(lr + 32 * i, ti.rows - 1);
        long long src = ti.row0 + r;
        if (p.a_rows) src = min(max((long long)p.a_rows[src], 0LL), p.a_nrows - 1);
        ag[i] = A + src * p.lda + kc;
        const int rb = lr + 32 * i;
        int wr;
        if (MODE == GM_UP_SWIGLU) {
            const int n0 = ti.nt * 64;
            wr = rb < 64 ? n0 + rb : p.up_off + n0 + (rb - 64);
        } else {
            wr = min(ti.nt * BN + rb, p.N - 1);
        }
        bg[i] = Bg + (size_t)wr * p.ldb + kc;
    }
    const uint16_t *ag0 = ag[0], *ag1 = ag[1], *ag2 = ag[2], *ag3 = ag[3];
    const uint16_t *bg0 = bg[0], *bg1 = bg[1], *bg2 = bg[2], *bg3 = bg[3];

    f32x16 c00, c01, c10, c11;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        c00[q] = 0.f;
        c01[q] = 0.f;
        c10[q] = 0.f;
        c11[q] = 0.f;
    }

    const int nk = p.K / BK;
    auto boff = [&](int kt) -> long long {
        const int k = kt * BK;
        const int seg = k / p.Kseg;
        return (long long)seg * p.sB_seg + (k - seg * p.Kseg);
    };
    const int br0 = MODE == GM_UP_SWIGLU ? wn * 32 : wn * 64;
    const int br1 = MODE == GM_UP_SWIGLU ? 64 + wn * 32 : wn * 64 + 32;
    const int arow = wm * 64;

    MOE_STAGE_DECL(s0_);
    MOE_STAGE_DECL(s1_);
    MOE_STAGE_LOAD(s0_, 0, boff(0));
    const int k1 = nk > 1 ? 1 : 0;
    MOE_STAGE_LOAD(s1_, k1 * BK, boff(k1));
    __syncthreads();  // the previous tile's epilogue may still read the staging area
    MOE_STAGE_STORE(s0_, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
        // even step: compute buffer 0, refill s0 with kt+2, publish s1 (kt+1) into buffer 1
        {
            const int kn = kt + 2 < nk ? kt + 2 : nk - 1;
            MOE_STAGE_LOAD(s0_, kn * BK, boff(kn));
            mma_tile(c00, c01, c10, c11, sA[0], sB[0], arow, br0, br1, lane);
            if (kt + 1 < nk) MOE_STAGE_STORE(s1_, 1);
            __syncthreads();
        }
        if (kt + 1 < nk) {
            const int kn = kt + 3 < nk ? kt + 3 : nk - 1;
            MOE_STAGE_LOAD(s1_, kn * BK, boff(kn));
            mma_tile(c00, c01, c10, c11, sA[1], sB[1], arow, br0, br1, lane);
            if (kt + 2 < nk) MOE_STAGE_STORE(s0_, 0);
            __syncthreads();
        }
    }

    // ---- epilogue: stage through LDS, then each row is covered by 16-byte vectors.
    // D[i][j] of a 32x32 block: column j = lane % 32, row i = 8 (q / 4) + 4 (lane / 32) + (q % 4).
    constexpr int OUTW = MODE == GM_UP_SWIGLU ? 64 : BN;  // output columns of the tile
    float* st = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int rl = wm * 64 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        if (MODE == GM_UP_SWIGLU) {
            st[rl * EPW + wn * 32 + (lane & 31)] = silu(c00[q]) * c01[q];
            st[(rl + 32) * EPW + wn * 32 + (lane & 31)] = silu(c10[q]) * c11[q];
        } else {
            st[rl * EPW + wn * 64 + (lane & 31)] = c00[q];
            st[rl * EPW + wn * 64 + 32 + (lane & 31)] = c01[q];
            st[(rl + 32) * EPW + wn * 64 + (lane & 31)] = c10[q];
            st[(rl + 32) * EPW + wn * 64 + 32 + (lane & 31)] = c11[q];
        }
    }
    __syncthreads();
    constexpr int TPR = OUTW / 8;    // threads per row
    constexpr int RPP = 256 / TPR;   // rows per pass
    const int cq = (tid % TPR) * 8;
    const int col0 = ti.nt * OUTW + cq;
    if (col0 >= p.N) return;
    uint16_t* C = (uint16_t*)p.C;
    const long long coff = p.offsets ? 0 : (long long)ti.g * p.sC_group;
    float bias8[8];
    if (MODE == GM_UP_RELU) {
#pragma unroll
        for (int e = 0; e < 8; ++e) bias8[e] = p.bias ? p.bias[(long long)ti.g * p.sbias_group + col0 + e] : 0.f;
    }
    for (int rl = tid / TPR; rl < ti.rows; rl += RPP) {
        const float4 v0 = *reinterpret_cast<const float4*>(&st[rl * EPW + cq]);
        const float4 v1 = *reinterpret_cast<const float4*>(&st[rl * EPW + cq + 4]);
        float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        const long long row = ti.row0 + rl;
        if (MODE == GM_UP_RELU) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = fmaxf(v[e] + bias8[e], 0.0f);
        }
        if (MODE == GM_DOWN_COMBINE) {
            // fixed order: residual + shared experts, then the routed rows k = 0 .. K_r-1
            if (p.resid) {
                const uint4 q = *reinterpret_cast<const uint4*>((const uint16_t*)p.resid + row * p.N + col0);
                float u8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                add8_bf16(u8, q);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = u8[e] + v[e];
            }
            const int32_t* prr = p.pair_row + row * p.K_r;
            const float* gr = p.topk_w + row * p.K_r;
            int k = 0;
            for (; k + 4 <= p.K_r; k += 4) {
                long long r4[4];
                float g4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const long long x = (long long)(uint32_t)prr[k + e];
                    r4[e] = x < p.R ? x : p.R - 1;
                    g4[e] = gr[k + e];
                }
                uint4 y4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    y4[e] = *reinterpret_cast<const uint4*>((const uint16_t*)p.y_perm + r4[e] * p.N + col0);
#pragma unroll
                for (int e = 0; e < 4; ++e) fma8_bf16(v, g4[e], y4[e]);
            }
            for (; k < p.K_r; ++k) {
                long long x = (long long)(uint32_t)prr[k];
                x = x < p.R ? x : p.R - 1;
                fma8_bf16(v, gr[k], *reinterpret_cast<const uint4*>((const uint16_t*)p.y_perm + x * p.N + col0));
            }
        }
        *reinterpret_cast<uint4*>(C + row * p.ldc + coff + col0) = pack8_bf16(v);
    }
}

__device__ __forceinline__ int total_tiles(const GemmParams& p, int NT) {
    if (p.offsets) return p.tiles[p.G] * NT;
    return p.G * ((p.M_dense + BM - 1) / BM) * NT;
}

template <int MODE>
__global__ __launch_bounds__(256, 2) void k_gemm_bf16(GemmParams p, int NT) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kSmemBytes];
    const int total = total_tiles(p, NT);
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
    const int beg = (int)((long long)total * xcd / 8);
    const int end = (int)((long long)total * (xcd + 1) / 8);
    for (int L = beg + loc; L < end; L += per_xcd) {
        TileInfo ti;
        decode_tile(p, NT, BM, L, ti);
        gemm_tile<MODE>(p, ti, smem);
    }
}

// ---------------------------------------------------------------- fp32 VALU path
// One thread per (row, output column).  Row r of the row space belongs to the group found by
// binary search in offsets (grouped) or to blockIdx.z (dense).
__device__ __forceinline__ int group_of_row(const int32_t* offsets, int G, int r) {
    int lo = 0, hi = G;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offsets[mid] <= r) lo = mid;
        else hi = mid;
    }
    return lo;
}

template <int MODE>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmParams p) {
    const int col = blockIdx.x * 64 + (threadIdx.x & 63);
    const int r = blockIdx.y * 4 + (threadIdx.x >> 6);
    if (col >= p.N) return;
    int g;
    long long rowC;
    if (p.offsets) {
        if (r >= p.offsets[p.G]) return;
        g = group_of_row(p.offsets, p.G, r);
        rowC = r;
    } else {
        if (r >= p.M_dense) return;
        g = blockIdx.z;
        rowC = r;
    }
    long long src = r;
    if (p.a_rows) src = min(max((long long)p.a_rows[r], 0LL), p.a_nrows - 1);
    const float* a = (const float*)p.A + src * p.lda;
    const float* Bg = (const float*)p.B + (size_t)g * p.sB_group;
    float* C = (float*)p.C + rowC * p.ldc + (p.offsets ? 0 : (long long)g * p.sC_group);
    if (MODE == GM_UP_SWIGLU) {
        const float* wg = Bg + (size_t)col * p.ldb;
        const float* wu = Bg + (size_t)(p.up_off + col) * p.ldb;
        float zg = 0.f, zu = 0.f;
        for (int k = 0; k < p.K; ++k) {
            zg = fmaf(a[k], wg[k], zg);
            zu = fmaf(a[k], wu[k], zu);
        }
        C[col] = zg / (1.0f + expf(-zg)) * zu;
    } else {
        float z = 0.f;
        for (int k = 0; k < p.K; ++k) {
            const int seg = k / p.Kseg;
            z = fmaf(a[k], Bg[(long long)seg * p.sB_seg + (size_t)col * p.ldb + (k - seg * p.Kseg)], z);
        }
        if (MODE == GM_UP_RELU) {
            if (p.bias) z += p.bias[(long long)g * p.sbias_group + col];
            z = fmaxf(z, 0.0f);
        }
        C[col] = z;
    }
}

hipError_t launch_gemm(int dtype, int mode, const GemmParams& p, hipStream_t s) {
    if (p.G == 0 || p.max_rows == 0 || p.N == 0) return hipSuccess;
    if (dtype == 0) {
        if (mode == GM_DOWN_COMBINE) return hipErrorInvalidValue;  // fp32 layers combine separately
        dim3 grid((p.N + 63) / 64, (p.max_rows + 3) / 4, p.offsets ? 1 : p.G);
        if (mode == GM_UP_SWIGLU) hipLaunchKernelGGL(k_gemm_f32<GM_UP_SWIGLU>, grid, dim3(256), 0, s, p);
        else if (mode == GM_UP_RELU) hipLaunchKernelGGL(k_gemm_f32<GM_UP_RELU>, grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL(k_gemm_f32<GM_DOWN>, grid, dim3(256), 0, s, p);
        return hipGetLastError();
    }
    const int NT = mode == GM_UP_SWIGLU ? (p.N + 63) / 64 : (p.N + BN - 1) / BN;
    if (mode == GM_DOWN_COMBINE && p.offsets) return hipErrorInvalidValue;  // dense (shared) groups only
    // persistent grid: two workgroups per CU (LDS and registers allow two), a multiple of 8
    long long mt;
    if (p.offsets) mt = (p.max_rows + BM - 1) / BM + p.G;  // upper bound of sum ceil(rows_g / BM)
    else mt = (long long)p.G * ((p.M_dense + BM - 1) / BM);
    long long nb = 2LL * device_cus();
    const long long need = (mt * NT + 7) / 8 * 8;
    nb = nb < need ? nb : need;
    nb = (nb + 7) / 8 * 8;
    if (mode == GM_UP_SWIGLU) hipLaunchKernelGGL(k_gemm_bf16<GM_UP_SWIGLU>, dim3((unsigned)nb), dim3(256), 0, s, p, NT);
    else if (mode == GM_UP_RELU) hipLaunchKernelGGL(k_gemm_bf16<GM_UP_RELU>, dim3((unsigned)nb), dim3(256), 0, s, p, NT);
    else if (mode == GM_DOWN) hipLaunchKernelGGL(k_gemm_bf16<GM_DOWN>, dim3((unsigned)nb), dim3(256), 0, s, p, NT);
    else hipLaunchKernelGGL(k_gemm_bf16<GM_DOWN_COMBINE>, dim3((unsigned)nb), dim3(256), 0, s, p, NT);
    return hipGetLastError();
}

}  // namespace moe
