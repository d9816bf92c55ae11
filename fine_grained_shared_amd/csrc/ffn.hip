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
constexpr int EPW = BN + 4;  // fp32 staging row of the LDS epilogue (floats)
constexpr int kSmemBytes = 2 * (BM + BN) * LDSW * 2;
static_assert(BM * EPW * 4 <= kSmemBytes, "epilogue staging must fit in the operand buffers");

template <int MODE>
__global__ __launch_bounds__(256, 2) void k_gemm_bf16(GemmParams p, int NT) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kSmemBytes];
    auto sA = reinterpret_cast<uint16_t(*)[BM][LDSW]>(smem);
    auto sB = reinterpret_cast<uint16_t(*)[BN][LDSW]>(smem + 2 * BM * LDSW * 2);

    const int L = xcd_remap(blockIdx.x, gridDim.x);
    TileInfo ti;
    if (!decode_tile(p, NT, BM, L, ti)) return;

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

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    const int nk = p.K / BK;
    // B offset of k-tile kt inside the (possibly segmented) reduction
#define MOE_BOFF(kt) ((long long)(((kt) * BK) / p.Kseg) * p.sB_seg + (((kt) * BK) % p.Kseg))
    uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
    {
        const long long bo = MOE_BOFF(0);
        ra0 = *reinterpret_cast<const uint4*>(ag[0]);
        ra1 = *reinterpret_cast<const uint4*>(ag[1]);
        ra2 = *reinterpret_cast<const uint4*>(ag[2]);
        ra3 = *reinterpret_cast<const uint4*>(ag[3]);
        rb0 = *reinterpret_cast<const uint4*>(bg[0] + bo);
        rb1 = *reinterpret_cast<const uint4*>(bg[1] + bo);
        rb2 = *reinterpret_cast<const uint4*>(bg[2] + bo);
        rb3 = *reinterpret_cast<const uint4*>(bg[3] + bo);
    }
    *reinterpret_cast<uint4*>(&sA[0][lr][kc]) = ra0;
    *reinterpret_cast<uint4*>(&sA[0][lr + 32][kc]) = ra1;
    *reinterpret_cast<uint4*>(&sA[0][lr + 64][kc]) = ra2;
    *reinterpret_cast<uint4*>(&sA[0][lr + 96][kc]) = ra3;
    *reinterpret_cast<uint4*>(&sB[0][lr][kc]) = rb0;
    *reinterpret_cast<uint4*>(&sB[0][lr + 32][kc]) = rb1;
    *reinterpret_cast<uint4*>(&sB[0][lr + 64][kc]) = rb2;
    *reinterpret_cast<uint4*>(&sB[0][lr + 96][kc]) = rb3;
    __syncthreads();
    const int br0 = MODE == GM_UP_SWIGLU ? wn * 32 : wn * 64;
    const int br1 = MODE == GM_UP_SWIGLU ? 64 + wn * 32 : wn * 64 + 32;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        // prefetch the next k-tile (the last iteration re-reads the current one: no branch,
        // so the staging registers stay registers)
        const int kn = kt + 1 < nk ? kt + 1 : kt;
        {
            const int k = kn * BK;
            const long long bo = MOE_BOFF(kn);
            ra0 = *reinterpret_cast<const uint4*>(ag[0] + k);
            ra1 = *reinterpret_cast<const uint4*>(ag[1] + k);
            ra2 = *reinterpret_cast<const uint4*>(ag[2] + k);
            ra3 = *reinterpret_cast<const uint4*>(ag[3] + k);
            rb0 = *reinterpret_cast<const uint4*>(bg[0] + bo);
            rb1 = *reinterpret_cast<const uint4*>(bg[1] + bo);
            rb2 = *reinterpret_cast<const uint4*>(bg[2] + bo);
            rb3 = *reinterpret_cast<const uint4*>(bg[3] + bo);
        }
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int ko = s * 16 + (lane >> 5) * 8;
            const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&sA[buf][wm * 64 + (lane & 31)][ko]);
            const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&sA[buf][wm * 64 + 32 + (lane & 31)][ko]);
            const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(&sB[buf][br0 + (lane & 31)][ko]);
            const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(&sB[buf][br1 + (lane & 31)][ko]);
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
        }
        const int nb = buf ^ 1;
        *reinterpret_cast<uint4*>(&sA[nb][lr][kc]) = ra0;
        *reinterpret_cast<uint4*>(&sA[nb][lr + 32][kc]) = ra1;
        *reinterpret_cast<uint4*>(&sA[nb][lr + 64][kc]) = ra2;
        *reinterpret_cast<uint4*>(&sA[nb][lr + 96][kc]) = ra3;
        *reinterpret_cast<uint4*>(&sB[nb][lr][kc]) = rb0;
        *reinterpret_cast<uint4*>(&sB[nb][lr + 32][kc]) = rb1;
        *reinterpret_cast<uint4*>(&sB[nb][lr + 64][kc]) = rb2;
        *reinterpret_cast<uint4*>(&sB[nb][lr + 96][kc]) = rb3;
        __syncthreads();
    }
#undef MOE_BOFF

    // epilogue.  D[i][j] of a 32x32 block: column j = lane % 32,
    // row i = 8 * (q / 4) + 4 * (lane / 32) + (q % 4) for accumulator element q.
    if (MODE == GM_DOWN || MODE == GM_DOWN_COMBINE) {
        // Stage the fp32 tile through LDS, then let 16 threads cover each row with 16-byte
        // vectors (coalesced stores; the combine reads whole 16-byte pieces of routed rows).
        float* st = reinterpret_cast<float*>(smem);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int rl = wm * 64 + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                    st[rl * EPW + wn * 64 + j * 32 + (lane & 31)] = acc[i][j][q];
                }
        __syncthreads();
        const int cq = (tid & 15) * 8;
        const int col0 = ti.nt * BN + cq;
        if (col0 >= p.N) return;
        uint16_t* C = (uint16_t*)p.C;
#pragma unroll 1
        for (int pr = 0; pr < BM / 16; ++pr) {
            const int rl = (tid >> 4) + 16 * pr;
            if (rl >= ti.rows) break;
            const float4 v0 = *reinterpret_cast<const float4*>(&st[rl * EPW + cq]);
            const float4 v1 = *reinterpret_cast<const float4*>(&st[rl * EPW + cq + 4]);
            float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            const long long row = ti.row0 + rl;
            if (MODE == GM_DOWN_COMBINE) {
                // fixed order: residual, shared experts, then k = 0 .. K_r-1
                if (p.resid) {
                    const uint4 q = *reinterpret_cast<const uint4*>((const uint16_t*)p.resid + row * p.N + col0);
                    const uint32_t wv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[2 * e] = __uint_as_float(wv[e] << 16) + v[2 * e];
                        v[2 * e + 1] = __uint_as_float(wv[e] & 0xFFFF0000u) + v[2 * e + 1];
                    }
                }
                for (int k = 0; k < p.K_r; ++k) {
                    long long pr_row = (long long)(uint32_t)p.pair_row[row * p.K_r + k];
                    pr_row = pr_row < p.R ? pr_row : p.R - 1;
                    const float g = p.topk_w[row * p.K_r + k];
                    const uint4 q = *reinterpret_cast<const uint4*>((const uint16_t*)p.y_perm + pr_row * p.N + col0);
                    const uint32_t wv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[2 * e] = fmaf(g, __uint_as_float(wv[e] << 16), v[2 * e]);
                        v[2 * e + 1] = fmaf(g, __uint_as_float(wv[e] & 0xFFFF0000u), v[2 * e + 1]);
                    }
                }
            }
            uint4 o;
            o.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
            o.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
            o.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
            o.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
            *reinterpret_cast<uint4*>(C + row * p.ldc + col0) = o;
        }
        return;
    }
    uint16_t* C = (uint16_t*)p.C;
    const long long coff = p.offsets ? 0 : (long long)ti.g * p.sC_group;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int rl = wm * 64 + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
            if (rl >= ti.rows) continue;
            uint16_t* crow = C + (long long)(ti.row0 + rl) * p.ldc + coff;
            if (MODE == GM_UP_SWIGLU) {
                const int col = ti.nt * 64 + wn * 32 + (lane & 31);
                crow[col] = f32_to_bf16(silu(acc[i][0][q]) * acc[i][1][q]);
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int col = ti.nt * BN + wn * 64 + j * 32 + (lane & 31);
                    if (col >= p.N) continue;
                    float v = acc[i][j][q];
                    if (MODE == GM_UP_RELU) {
                        if (p.bias) v += p.bias[(long long)ti.g * p.sbias_group + col];
                        v = fmaxf(v, 0.0f);
                    }
                    crow[col] = f32_to_bf16(v);
                }
            }
        }
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
    long long mt;
    if (p.offsets) mt = (p.max_rows + BM - 1) / BM + p.G;  // sum of ceil(rows_g / BM) <= this
    else mt = (long long)p.G * ((p.M_dense + BM - 1) / BM);
    long long nb = mt * NT;
    nb = (nb + 7) / 8 * 8;
    if (nb > 0x7FFFFFF8LL) return hipErrorInvalidValue;
    if (mode == GM_UP_SWIGLU) hipLaunchKernelGGL(k_gemm_bf16<GM_UP_SWIGLU>, dim3((unsigned)nb), dim3(256), 0, s, p, NT);
    else if (mode == GM_UP_RELU) hipLaunchKernelGGL(k_gemm_bf16<GM_UP_RELU>, dim3((unsigned)nb), dim3(256), 0, s, p, NT);
    else if (mode == GM_DOWN) hipLaunchKernelGGL(k_gemm_bf16<GM_DOWN>, dim3((unsigned)nb), dim3(256), 0, s, p, NT);
    else hipLaunchKernelGGL(k_gemm_bf16<GM_DOWN_COMBINE>, dim3((unsigned)nb), dim3(256), 0, s, p, NT);
    return hipGetLastError();
}

}  // namespace moe
