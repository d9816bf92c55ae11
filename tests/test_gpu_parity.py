"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, stage by stage and whole layer.

Small layers are compared on every token; they span several 128-row tiles, ragged tails in
both GEMM dimensions, empty and overfull expert groups.
"""
import numpy as np
import pytest

import oracle
import synth
from parity_util import (Case, check_close, check_routing, gpu_shape, layer_parity, say, to_dev,
                         to_f64)
from synth import (ACT_RELU_BIAS, ACT_SWIGLU, DT_BF16, DT_F32, GATE_SIGMOID_BIAS_NORM, GATE_SOFTMAX,
                   GATE_SOFTMAX_RENORM, Workload)

pytestmark = pytest.mark.gpu

# T=300 rows -> 3 m-tiles with a ragged tail; H=320 -> a ragged 128-column tile in the down GEMM;
# I=192 -> 3 SwiGLU column tiles.
RAGGED = Workload("ragged", "ragged bf16 SwiGLU sigmoid+bias layer", 300, 320, 16, 3, 2, 192,
                  GATE_SIGMOID_BIAS_NORM, ACT_SWIGLU, DT_BF16, bias_var=0.01)

VARIANTS = {
    "ragged": RAGGED,
    "relu_softmax_bf16": RAGGED.with_(name="relu_softmax_bf16", gating=GATE_SOFTMAX, act=ACT_RELU_BIAS, bias_var=0.0,
                                      I=256),
    "swiglu_f32": RAGGED.with_(name="swiglu_f32", dtype=DT_F32, T=130),
    "renorm_softmax": RAGGED.with_(name="renorm_softmax", gating=GATE_SOFTMAX_RENORM, bias_var=0.0),
    "all_experts": RAGGED.with_(name="all_experts", K_r=16, Ks=1),
    # 600 tokens: the shared down GEMM with the fused combine takes the 128 x 128 kernel, and K_r = 16
    # routed rows per token take its epilogue without the LDS copy of the pair rows (that holds 12)
    "all_experts_prefill": RAGGED.with_(name="all_experts_prefill", T=600, K_r=16, Ks=1),
    "no_shared": RAGGED.with_(name="no_shared", Ks=0, K_r=5),
    "group_limited": RAGGED.with_(name="group_limited", N_r=32, K_r=4, n_group=8, topk_group=2),
    "group_limited_softmax": RAGGED.with_(name="group_limited_softmax", N_r=32, K_r=4, n_group=4, topk_group=2,
                                          gating=GATE_SOFTMAX, bias_var=0.0),
    "mask_probe": RAGGED.with_(name="mask_probe", N_r=32, K_r=4, mask_top_r=2),
    "many_experts": RAGGED.with_(name="many_experts", T=200, N_r=600, K_r=12, Ks=1, I=64, H=256),
}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fine_grained_shared_amd as moe
    moe.load()
    return torch


def test_c0_tiny_fp32_layer_every_token(torch_cuda):
    case = Case(synth.WORKLOADS["c0"])
    stats, _ = layer_parity(case, label="c0")
    assert stats["fro_out"] <= 1e-5


def test_c0_coarse_layer_equals_its_fine_split(torch_cuda):
    """llm-infra-atlas 02, section 2.1 (Eq. 6-8, iso-parameter / iso-FLOP split): the tiny fp32 layer's
    geometry, a coarse N=4, M=256, top-1 ReLU layer with one shared expert of width 256, run on the GPU
    next to its m=4 split (16 routed experts of width 64, top-4; four shared experts of width 64).
    Each slice keeps its coarse expert's centroid, so the four slices of the chosen coarse expert tie and
    are all selected, each with a quarter of the coarse softmax weight; their down projections are
    scaled by m (a power of two, exact).  The shared expert is split into four of width 64 with
    weight 1 (the sum of the slices is the coarse FFN).  Both GPU outputs must agree within the fp32 bar
    and each must match the oracle."""
    import fine_grained_shared_amd as moe
    torch = torch_cuda
    T, H, N, M, m = 64, 128, 4, 256, 4
    wc = Workload("c0_coarse", "coarse N=4 M=256 top-1 ReLU layer", T, H, N, 1, 1, M, GATE_SOFTMAX, ACT_RELU_BIAS,
                  DT_F32)
    ci = synth.make_inputs(wc)
    ci["b1"] = synth.normal(8, (N, M), 0.2, DT_F32)
    ci["b1_sh"] = synth.normal(8, (1, M), 0.2, DT_F32, offset=N * M)
    iw = M // m
    fi = dict(ci)
    fi["centroids"] = np.repeat(ci["centroids"], m, axis=0)
    fi["w1"] = np.ascontiguousarray(ci["w1"].reshape(N * m, iw, H))
    fi["b1"] = np.ascontiguousarray(ci["b1"].reshape(N * m, iw))
    fi["w2"] = np.ascontiguousarray(
        (ci["w2"].reshape(N, H, m, iw).transpose(0, 2, 1, 3) * np.float32(m)).reshape(N * m, H, iw))
    fi["w1_sh"] = np.ascontiguousarray(ci["w1_sh"].reshape(m, iw, H))
    fi["b1_sh"] = np.ascontiguousarray(ci["b1_sh"].reshape(m, iw))
    fi["w2_sh"] = np.ascontiguousarray(ci["w2_sh"].reshape(H, m, iw).transpose(1, 0, 2))
    wf = wc.with_(name="c0_fine", N_r=N * m, K_r=m, Ks=m, I=iw)
    coarse, fine = Case(wc, ci), Case(wf, fi)
    out_c, idx_c, w_c = coarse.forward()
    out_f, idx_f, w_f = fine.forward()
    torch.cuda.synchronize()
    sel_c, sel_f = idx_c.cpu().numpy(), idx_f.cpu().numpy()
    assert np.array_equal(sel_f, sel_c * m + np.arange(m)), "the fine layer must take the coarse expert's slices"
    np.testing.assert_allclose(w_f.cpu().numpy(), np.repeat(w_c.cpu().numpy(), m, axis=1) / m, rtol=1e-6)
    got_c, got_f = to_f64(out_c), to_f64(out_f)
    rel = np.linalg.norm(got_f - got_c) / np.linalg.norm(got_c)
    rel_moe = np.linalg.norm(got_f - got_c) / np.linalg.norm(got_c - synth.as_float64(ci["u"], DT_F32))
    say("[c0 split] GPU coarse vs fine: rel Frobenius %.3e (MoE part %.3e)" % (rel, rel_moe))
    assert rel <= 1e-5 and rel_moe <= 1e-5
    for case, label in ((coarse, "c0 coarse"), (fine, "c0 fine")):
        stats, _ = layer_parity(case, label=label)
        assert stats["fro_out"] <= 1e-5


@pytest.mark.parametrize("name", list(VARIANTS))
def test_layer_variants_every_token(torch_cuda, name):
    case = Case(VARIANTS[name])
    layer_parity(case, label=name)


@pytest.mark.parametrize("name", ["c1a", "c1b", "c1b_iso", "c2"])
def test_layer_configs_every_token(torch_cuda, name):
    w = synth.WORKLOADS[name]
    case = Case(w)
    stats, (out, idx, wts) = layer_parity(case, label=name)
    # load histogram of the realised routing (c2: the 8 hot experts draw more tokens)
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=w.N_r)
    say("[parity] %s: load max/mean %.2f, empty %d" % (name, counts.max() / counts.mean(), (counts == 0).sum()))
    if name == "c2":
        assert counts[:8].mean() > counts[8:].mean()


# ---------------------------------------------------------------- stages (ragged layer)

@pytest.fixture(scope="module")
def ragged(torch_cuda):
    return Case(RAGGED)


def test_stage_route(ragged, torch_cuda):
    import fine_grained_shared_amd as moe
    torch = torch_cuda
    w, d = ragged.w, ragged.dev
    s = gpu_shape(w)
    idx = torch.empty((w.T, w.K_r), dtype=torch.int32, device="cuda")
    wts = torch.empty((w.T, w.K_r), dtype=torch.float32, device="cuda")
    moe.moe_route(s, d["u"], d["centroids"], d["bias"], idx, wts, moe.workspace(s))
    torch.cuda.synchronize()
    sel_o, g_o, gap = oracle.route(oracle.shape_of(w), ragged.inp["u"], ragged.inp["centroids"], ragged.inp["bias"])
    check_routing(idx.cpu().numpy(), wts.cpu().numpy().astype(np.float64), sel_o, g_o, gap, "route")
    # descending key order inside each token's list
    sc = 1.0 / (1.0 + np.exp(-(synth.as_float64(ragged.inp["u"], DT_BF16) @
                               synth.as_float64(ragged.inp["centroids"], DT_BF16).T)))
    key = sc + ragged.inp["bias"].astype(np.float64)
    kk = np.take_along_axis(key, idx.cpu().numpy().astype(np.int64), axis=1)
    assert np.all(np.diff(kk, axis=1) <= 1e-6)


def test_dispatch_gather_with_skipped_entries(torch_cuda):
    """Entries outside [0, N_r) are skipped by the dispatch: those pairs get no row, and the rows past
    the last segment keep whatever the caller's buffer held.  The x_perm gather clamps every row's
    token index into [0, T), so it reads only u; the kept pairs' rows are exact."""
    import fine_grained_shared_amd as moe
    torch = torch_cuda
    T, N, K, H = 40, 8, 3, 64
    rng = np.random.default_rng(11)
    idx_np = np.stack([rng.permutation(N)[:K] for _ in range(T)]).astype(np.int32)
    idx_np[3, 1] = -1
    idx_np[17, 0] = N
    idx_np[29, 2] = 1 << 30
    s = moe.make_shape(T, H, N, K, 0, 64, synth.GATE_SOFTMAX, synth.ACT_SWIGLU, synth.DT_BF16)
    ws = moe.workspace(s)
    u = torch.randn((T, H), generator=torch.Generator().manual_seed(4)).bfloat16().cuda()
    R = T * K
    offsets = torch.full((N + 1,), -7, dtype=torch.int32, device="cuda")
    row_token = torch.full((R,), -1000000, dtype=torch.int32, device="cuda")   # unwritten rows: far out of range
    pair_row = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    x_perm = torch.zeros((R, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_dispatch(s, torch.from_numpy(idx_np).cuda(), offsets, row_token, pair_row, u, x_perm, ws)
    torch.cuda.synchronize()
    off = offsets.cpu().numpy()
    kept = (idx_np >= 0) & (idx_np < N)
    assert off[N] == kept.sum() == R - 3
    # the kept pairs, ordered by expert, then by (token, slot)
    flat = idx_np.reshape(-1)
    order = np.argsort(np.where(kept.reshape(-1), flat, N), kind="stable")[:off[N]]
    rt = row_token.cpu().numpy()
    assert np.array_equal(rt[:off[N]], order // K)
    assert np.array_equal(off[:N], np.concatenate([[0], np.cumsum(np.bincount(flat[kept.reshape(-1)],
                                                                              minlength=N))[:-1]]))
    xp = x_perm.cpu()
    assert torch.equal(xp[:off[N]], u.cpu()[torch.from_numpy(rt[:off[N]]).long()])
    assert torch.equal(xp[off[N]:], u.cpu()[torch.zeros(R - off[N], dtype=torch.long)])   # clamped to token 0


def test_stage_dispatch_bit_exact(ragged, torch_cuda):
    import fine_grained_shared_amd as moe
    torch = torch_cuda
    w, d = ragged.w, ragged.dev
    s = gpu_shape(w)
    ws = moe.workspace(s)
    idx = torch.empty((w.T, w.K_r), dtype=torch.int32, device="cuda")
    wts = torch.empty((w.T, w.K_r), dtype=torch.float32, device="cuda")
    moe.moe_route(s, d["u"], d["centroids"], d["bias"], idx, wts, ws)
    R = w.T * w.K_r
    offsets = torch.full((w.N_r + 1,), -7, dtype=torch.int32, device="cuda")
    row_token = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    pair_row = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    x_perm = torch.empty((R, w.H), dtype=torch.bfloat16, device="cuda")
    moe.moe_dispatch(s, idx, offsets, row_token, pair_row, d["u"], x_perm, ws)
    torch.cuda.synchronize()
    o_ref, rt_ref, pr_ref = oracle.dispatch(idx.cpu().numpy(), w.N_r)
    assert np.array_equal(offsets.cpu().numpy(), o_ref)
    assert np.array_equal(row_token.cpu().numpy(), rt_ref)
    assert np.array_equal(pair_row.cpu().numpy(), pr_ref)
    assert torch.equal(x_perm, d["u"][row_token.long()])


@pytest.mark.parametrize("T,N,K", [(5000, 300, 6), (20000, 1024, 8), (10000, 64, 2),
                                   (200, 300, 6), (256, 1024, 8), (37, 16, 16), (1, 64, 2)])
def test_dispatch_bit_exact_many_chunks(T, N, K, torch_cuda):
    """Dispatch on skewed synthetic selections.  Many 256-token chunks: the scan runs one workgroup per
    64 experts (a partial last one at N = 300) with 16 chunk ranges per expert, some of them empty.
    One chunk (T <= 256, a decode step): the single-launch path.  Offsets, rows and pair positions must
    equal the oracle's nested loops exactly."""
    import fine_grained_shared_amd as moe
    torch = torch_cuda
    rng = np.random.default_rng(T + N + K)
    skew = np.linspace(0.0, 3.0, N)[rng.permutation(N)]          # a few experts far more popular
    keys = rng.random((T, N)) + skew[None, :]
    idx_np = np.argsort(-keys, axis=1)[:, :K].astype(np.int32)    # K distinct experts per token
    s = moe.make_shape(T, 64, N, K, 0, 64, synth.GATE_SOFTMAX, synth.ACT_SWIGLU, synth.DT_BF16)
    ws = moe.workspace(s)
    idx = torch.from_numpy(idx_np).cuda()
    R = T * K
    offsets = torch.full((N + 1,), -7, dtype=torch.int32, device="cuda")
    row_token = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    pair_row = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    moe.moe_dispatch(s, idx, offsets, row_token, pair_row, None, None, ws)
    torch.cuda.synchronize()
    o_ref, rt_ref, pr_ref = oracle.dispatch(idx_np, N)
    assert np.array_equal(offsets.cpu().numpy(), o_ref)
    assert np.array_equal(row_token.cpu().numpy(), rt_ref)
    assert np.array_equal(pair_row.cpu().numpy(), pr_ref)


@pytest.mark.parametrize("T", [300, 1100])
@pytest.mark.parametrize("gating", [GATE_SOFTMAX, GATE_SIGMOID_BIAS_NORM])
def test_exact_ties_go_to_the_lower_index(T, gating, torch_cuda):
    """Experts with identical centroids (and bias) tie exactly, on the GPU as in the oracle.  Pair
    (5, 70) sits in different lanes of the selection wave (its index bits decide), pair (9, 73) in one
    lane.  Tokens planted along one centroid of a pair must select [low, high] in that order with equal
    gate weights.  T = 300 takes the decode-size logits kernel, T = 1100 the tiled GEMM."""
    import fine_grained_shared_amd as moe
    torch = torch_cuda
    w = Workload("ties", "exact ties", T, 128, 128, 2, 0, 64, gating, ACT_SWIGLU, DT_BF16,
                 bias_var=0.01 if gating == GATE_SIGMOID_BIAS_NORM else 0.0)
    inp = synth.make_inputs(w, weights=False)
    cen = inp["centroids"].copy()
    u = inp["u"].copy()
    bias = None if inp["bias"] is None else inp["bias"].copy()
    plants = {}
    for lo, hi in ((5, 70), (9, 73)):
        cen[hi] = cen[lo]
        if bias is not None:   # sigmoid saturates: the pair's lead comes from an equal, larger bias
            bias[lo] = bias[hi] = 1.0
        toks = np.arange(lo, T, 17)
        # u_t = 16 e_lo (exact in bf16): the pair's logit 16 |e_lo|^2 dominates every other expert's
        u[toks] = synth.f32_to_bf16_bits(16.0 * synth.bf16_bits_to_f32(cen[lo]))
        plants[(lo, hi)] = toks
    s = gpu_shape(w)
    ws = moe.workspace(s)
    idx = torch.empty((T, 2), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, 2), dtype=torch.float32, device="cuda")
    moe.moe_route(s, to_dev(u), to_dev(cen), to_dev(bias), idx, wts, ws)
    torch.cuda.synchronize()
    got, g = idx.cpu().numpy(), wts.cpu().numpy()
    for (lo, hi), toks in plants.items():
        assert (got[toks] == [lo, hi]).all(), (lo, hi, got[toks][:4])
        assert (g[toks, 0] == g[toks, 1]).all()
    # the oracle agrees on the planted tokens (its keys tie exactly as well)
    sel, _, _ = oracle.route(oracle.shape_of(w), u, cen, bias)
    for (lo, hi), toks in plants.items():
        assert (sel[toks] == [lo, hi]).all()


def test_stage_expert_ffn_both_gather_modes(ragged, torch_cuda):
    import fine_grained_shared_amd as moe
    torch = torch_cuda
    w, d = ragged.w, ragged.dev
    s = gpu_shape(w)
    ws = moe.workspace(s)
    R = w.T * w.K_r
    idx = torch.empty((w.T, w.K_r), dtype=torch.int32, device="cuda")
    wts = torch.empty((w.T, w.K_r), dtype=torch.float32, device="cuda")
    moe.moe_route(s, d["u"], d["centroids"], d["bias"], idx, wts, ws)
    offsets = torch.empty((w.N_r + 1,), dtype=torch.int32, device="cuda")
    row_token = torch.empty((R,), dtype=torch.int32, device="cuda")
    pair_row = torch.empty((R,), dtype=torch.int32, device="cuda")
    x_perm = torch.empty((R, w.H), dtype=torch.bfloat16, device="cuda")
    moe.moe_dispatch(s, idx, offsets, row_token, pair_row, d["u"], x_perm, ws)
    y1 = torch.empty((R, w.H), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((R, w.H), dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_ffn(s, d["u"], row_token, offsets, d["w1"], None, d["w2"], y1, ws)
    moe.moe_expert_ffn(s, x_perm, None, offsets, d["w1"], None, d["w2"], y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    off = offsets.cpu().numpy()
    rt = row_token.cpu().numpy()
    uf = synth.as_float64(ragged.inp["u"], DT_BF16)
    ref = np.zeros((R, w.H))
    for e in range(w.N_r):
        for r in range(off[e], off[e + 1]):
            ref[r] = oracle.expert_ffn(w.H, w.I, w.act, w.dtype, ragged.inp["w1"][e], None, ragged.inp["w2"][e],
                                       uf[rt[r]])
    check_close(to_f64(y1), ref, DT_BF16, "expert_ffn")


def test_stage_shared_ffn(ragged, torch_cuda):
    import fine_grained_shared_amd as moe
    torch = torch_cuda
    w, d = ragged.w, ragged.dev
    s = gpu_shape(w)
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    moe.moe_shared_ffn(s, d["u"], d["w1_sh"], None, d["w2_sh"], y, moe.workspace(s))
    torch.cuda.synchronize()
    uf = synth.as_float64(ragged.inp["u"], DT_BF16)
    ref = np.zeros((w.T, w.H))
    for t in range(w.T):
        for j in range(w.Ks):
            ref[t] += oracle.expert_ffn(w.H, w.I, w.act, w.dtype, ragged.inp["w1_sh"][j], None,
                                        ragged.inp["w2_sh"][j], uf[t])
    check_close(to_f64(y), ref, DT_BF16, "shared_ffn")


@pytest.mark.parametrize("dtype", [DT_BF16, DT_F32])
def test_stage_combine(torch_cuda, dtype):
    import fine_grained_shared_amd as moe
    torch = torch_cuda
    T, H, K, N = 77, 192, 4, 9
    rng = np.random.default_rng(3)
    tdt = torch.bfloat16 if dtype == DT_BF16 else torch.float32
    resid = torch.randn((T, H), generator=torch.Generator().manual_seed(1)).to(tdt).cuda()
    ysh = torch.randn((T, H), generator=torch.Generator().manual_seed(2)).to(tdt).cuda()
    yp = torch.randn((T * K, H), generator=torch.Generator().manual_seed(3)).to(tdt).cuda()
    pr = torch.from_numpy(rng.permutation(T * K).astype(np.int32)).cuda()
    g = torch.from_numpy(rng.random((T, K)).astype(np.float32)).cuda()
    out = torch.empty((T, H), dtype=tdt, device="cuda")
    s = moe.make_shape(T, H, N, K, 1, 64, 0, 1, dtype)
    for use_res, use_sh in ((True, True), (False, True), (True, False)):
        moe.moe_combine(s, resid if use_res else None, ysh if use_sh else None, yp, pr, g, out)
        torch.cuda.synchronize()
        ref = np.zeros((T, H))
        mag = np.zeros((T, H))          # sum of |terms|: bounds the fp32 accumulation error
        if use_res:
            ref += to_f64(resid)
            mag += np.abs(to_f64(resid))
        if use_sh:
            ref += to_f64(ysh)
            mag += np.abs(to_f64(ysh))
        ypf = to_f64(yp)
        prn = pr.cpu().numpy().reshape(T, K)
        gn = g.cpu().numpy().astype(np.float64)
        for k in range(K):
            ref += gn[:, k:k + 1] * ypf[prn[:, k]]
            mag += np.abs(gn[:, k:k + 1] * ypf[prn[:, k]])
        got = to_f64(out)
        # fp32 accumulation of K+2 terms, then (bf16) one rounding of the result
        allow = (K + 2) * 2.0 ** -24 * mag + (2.0 ** -8 * np.abs(ref) if dtype == DT_BF16 else 0.0)
        assert np.all(np.abs(got - ref) <= allow)


# ---------------------------------------------------------------- invariants and edge cases

def test_token_permutation_and_batch_split_bit_exact(ragged, torch_cuda):
    torch = torch_cuda
    w = ragged.w
    out, idx, wts = ragged.forward()
    perm = torch.from_numpy(np.random.default_rng(5).permutation(w.T)).cuda()
    up = ragged.dev["u"][perm].contiguous()
    out_p, idx_p, _ = ragged.forward(u=up)
    assert torch.equal(out_p, out[perm]) and torch.equal(idx_p, idx[perm])
    h = 123
    out_a, _, _ = ragged.forward(shape=gpu_shape(w, T=h), u=ragged.dev["u"][:h].contiguous())
    out_b, _, _ = ragged.forward(shape=gpu_shape(w, T=w.T - h), u=ragged.dev["u"][h:].contiguous())
    assert torch.equal(torch.cat([out_a, out_b]), out)
    out2, idx2, wts2 = ragged.forward()
    assert torch.equal(out2, out) and torch.equal(idx2, idx) and torch.equal(wts2, wts)


def test_identity_when_no_experts(ragged, torch_cuda):
    torch = torch_cuda
    w = ragged.w.with_(K_r=0, Ks=0)
    out, _, _ = ragged.forward(shape=gpu_shape(w))
    assert torch.equal(out, ragged.dev["u"])
    # K_r = 0 with shared experts: out = u + shared sum
    w1 = ragged.w.with_(K_r=0)
    case = Case(w1, ragged.inp)
    layer_parity(case, label="kr0")


def test_overfull_and_empty_groups(torch_cuda):
    """A bias that forces every token onto experts 0..K_r-1: K_r groups of T rows, the rest empty."""
    w = RAGGED.with_(name="forced", T=260)
    inp = synth.make_inputs(w)
    inp["bias"] = np.zeros(w.N_r, dtype=np.float32)
    inp["bias"][: w.K_r] = 10.0
    case = Case(w, inp)
    _, (out, idx, wts) = layer_parity(case, label="forced")
    assert np.array_equal(np.sort(idx.cpu().numpy(), axis=1), np.tile(np.arange(w.K_r), (w.T, 1)))


@pytest.mark.parametrize("T", [0, 1, 2])
def test_tiny_token_counts(torch_cuda, T):
    torch = torch_cuda
    case = Case(RAGGED.with_(T=max(T, 1)))
    if T == 0:
        out, idx, wts = case.forward(shape=gpu_shape(case.w, T=0), u=case.dev["u"][:0])
        torch.cuda.synchronize()
        assert out.shape == (0, case.w.H)
        return
    case = case.with_tokens(T)
    layer_parity(case, label="T=%d" % T)


def test_error_paths(ragged, torch_cuda):
    import fine_grained_shared_amd as moe
    torch = torch_cuda
    w, d = ragged.w, ragged.dev
    s = gpu_shape(w)
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    small = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_forward(s, d["u"], d["centroids"], d["bias"], d["w1"], None, d["w2"], d["w1_sh"], None,
                              d["w2_sh"], 0, out, None, None, small)
    assert e.value.status == moe.MOE_ERR_WORKSPACE
    ws = moe.workspace(s)
    flat = torch.empty(w.T * w.H + 1, dtype=torch.bfloat16, device="cuda")
    mis = flat[1:].view(w.T, w.H)   # 2-byte misaligned
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_forward(s, mis, d["centroids"], d["bias"], d["w1"], None, d["w2"], d["w1_sh"], None,
                              d["w2_sh"], 0, out, None, None, ws)
    assert e.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as e:   # selection bias outside the sigmoid gating
        moe.moe_layer_forward(gpu_shape(w, gating=GATE_SOFTMAX), d["u"], d["centroids"], d["bias"], d["w1"], None,
                              d["w2"], d["w1_sh"], None, d["w2_sh"], 0, out, None, None, ws)
    assert e.value.status == moe.MOE_ERR_INVALID_ARG


def test_bias_update_bit_exact(ragged, torch_cuda):
    import fine_grained_shared_amd as moe
    torch = torch_cuda
    w, d = ragged.w, ragged.dev
    s = gpu_shape(w)
    ws = moe.workspace(s)
    R = w.T * w.K_r
    idx = torch.empty((w.T, w.K_r), dtype=torch.int32, device="cuda")
    wts = torch.empty((w.T, w.K_r), dtype=torch.float32, device="cuda")
    bias = d["bias"].clone()
    offsets = torch.empty((w.N_r + 1,), dtype=torch.int32, device="cuda")
    row_token = torch.empty((R,), dtype=torch.int32, device="cuda")
    pair_row = torch.empty((R,), dtype=torch.int32, device="cuda")
    counts = torch.empty((w.N_r,), dtype=torch.int32, device="cuda")
    b_host = ragged.inp["bias"].copy()
    for step in range(3):
        moe.moe_route(s, d["u"], d["centroids"], bias, idx, wts, ws)
        moe.moe_dispatch(s, idx, offsets, row_token, pair_row, None, None, ws)
        moe.moe_bias_update(s, offsets, 0.01, bias, counts)
        torch.cuda.synchronize()
        ref_counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=w.N_r)
        assert np.array_equal(counts.cpu().numpy(), ref_counts)
        b_host = oracle.bias_update(w.N_r, w.T, w.K_r, ref_counts, 0.01, b_host)
        assert np.array_equal(bias.cpu().numpy(), b_host)


def test_profile_api_counts_launches(ragged, torch_cuda):
    import fine_grained_shared_amd as moe
    torch = torch_cuda
    torch.cuda.synchronize()
    moe.moe_profile_enable(True)
    for _ in range(3):
        ragged.forward()
    torch.cuda.synchronize()
    moe.moe_profile_enable(False)
    n_up, ms_up = moe.moe_profile_query(moe.MOE_PROF_FFN_UP)
    n_rt, ms_rt = moe.moe_profile_query(moe.MOE_PROF_ROUTER)
    assert n_up == 3 and ms_up > 0.0          # one routed up launch per layer call
    assert n_rt == 6 and ms_rt > 0.0          # logits + selection per call
    with pytest.raises(moe.MoeError):
        moe.moe_profile_query(99)


def test_graph_capture_replays_match_eager(ragged, torch_cuda):
    """The layer only enqueues work (no host sync, no memset): it can be captured in a HIP graph.
    Replays, with eager work between them, must reproduce the eager output bit for bit."""
    import fine_grained_shared_amd as moe
    torch = torch_cuda
    w, d = ragged.w, ragged.dev
    s = gpu_shape(w)
    ws = moe.workspace(s)
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((w.T, w.K_r), dtype=torch.int32, device="cuda")
    wts = torch.empty((w.T, w.K_r), dtype=torch.float32, device="cuda")

    def run():
        moe.moe_layer_forward(s, d["u"], d["centroids"], d["bias"], d["w1"], None, d["w2"], d["w1_sh"], None,
                              d["w2_sh"], 0, out, idx, wts, ws)
    run()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(4):
        out.zero_()
        ragged.forward()          # eager work on other buffers between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d differs from eager" % i


def test_bf16_output_rounding_is_nearest_even(torch_cuda):
    """Outputs are rounded fp32 -> bf16 to nearest, ties to even: residual + shared sums that fall
    exactly halfway between two bf16 values (exact in fp32) must go to the even neighbour."""
    import fine_grained_shared_amd as moe
    torch = torch_cuda
    e7, e8, e15, e16 = 2.0 ** -7, 2.0 ** -8, 2.0 ** -15, 2.0 ** -16
    cases = [  # (residual, shared, expected bf16 value)
        (1 + e7, e8, 1 + 2 * e7),          # 1 + 3*2^-8: tie between odd 1+2^-7 and even 1+2^-6 -> up
        (1.0, e8, 1.0),                    # 1 + 2^-8: tie between even 1.0 and odd 1+2^-7 -> down
        (-(1 + e7), -e8, -(1 + 2 * e7)),   # negative tie -> away from the odd neighbour
        (1.0, e8 + e15, 1 + e7),           # just above the tie -> up
        (1 + e7, e8 - e16, 1 + e7),        # just below the tie -> down
        (3.0, 0.0, 3.0),
        (0.0, 0.0, 0.0),
    ]
    H = 64
    r = np.zeros((1, H), dtype=np.float32)
    s = np.zeros((1, H), dtype=np.float32)
    want = np.zeros((1, H), dtype=np.float32)
    for i, (a, b, c) in enumerate(cases):
        r[0, i], s[0, i], want[0, i] = a, b, c
    rt = torch.from_numpy(r).cuda().bfloat16()
    st = torch.from_numpy(s).cuda().bfloat16()
    assert torch.equal(rt.float().cpu(), torch.from_numpy(r)) and torch.equal(st.float().cpu(), torch.from_numpy(s))
    out = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")
    shape = moe.make_shape(1, H, 1, 0, 1, 64, 0, 1, moe.MOE_BF16)
    moe.moe_combine(shape, rt, st, None, None, None, out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.array_equal(got, want), (got[0, :len(cases)], want[0, :len(cases)])
