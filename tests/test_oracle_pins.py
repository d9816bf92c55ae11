"""Pins for the fp64 oracle: brute force, closed forms, library routines.

Each test checks the oracle against something other than itself, so that a
dropped term, a wrong sign or index or a transposed operand fails one of them.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle
import synth
from synth import (ACT_RELU_BIAS, ACT_SWIGLU, DT_BF16, DT_F32, GATE_SIGMOID_BIAS_NORM,
                   GATE_SOFTMAX, GATE_SOFTMAX_RENORM, Workload)

RNG = np.random.default_rng(1234)


def shape(**kw):
    d = dict(T=1, H=8, N_r=4, K_r=2, Ks=0, I=8, gating=GATE_SOFTMAX, act=ACT_SWIGLU, dtype=DT_F32,
             n_group=0, topk_group=0, mask_top_r=0)
    d.update(kw)
    return oracle.OrcShape(**d)


def diag_layer(c):
    """Inputs whose logits are exactly c: u = 1, centroid i = c_i on coordinate i."""
    n = len(c)
    u = np.ones((1, n), dtype=np.float32)
    e = np.zeros((n, n), dtype=np.float32)
    e[np.arange(n), np.arange(n)] = np.asarray(c, dtype=np.float32)
    return u, e


def brute_topk(key, K):
    """The unique K-subset S with key_i > key_j, or equal keys and i < j, for all i in S, j not in S."""
    n = len(key)
    found = []
    for S in itertools.combinations(range(n), K):
        out = [j for j in range(n) if j not in S]
        if all(key[i] > key[j] or (key[i] == key[j] and i < j) for i in S for j in out):
            found.append(S)
    assert len(found) == 1
    S = found[0]
    order = sorted(S, key=lambda i: (-key[i], i))
    rest = [j for j in range(n) if j not in S]
    gap = min(key[i] for i in S) - max(key[j] for j in rest) if S and rest else math.inf
    return order, gap


# ---------------------------------------------------------------- selection (Eq. 7, section 7.4)

@pytest.mark.parametrize("gating", [GATE_SOFTMAX, GATE_SIGMOID_BIAS_NORM])
def test_topk_matches_brute_force_with_ties(gating):
    for trial in range(150):
        n = int(RNG.integers(1, 10))
        K = int(RNG.integers(0, n + 1))
        c = RNG.integers(-3, 4, size=n) / 4.0          # coarse grid -> exact ties
        u, e = diag_layer(c)
        bias = None
        if gating == GATE_SIGMOID_BIAS_NORM and trial % 2:
            bias = (RNG.integers(-2, 3, size=n) / 8.0).astype(np.float32)
        s = shape(H=n, N_r=n, K_r=K, gating=gating)
        sel, g, gap, lo, sc = oracle.route(s, u, e, bias, want_scores=True)
        assert np.array_equal(lo[0], c)              # logits are exact here
        if gating == GATE_SOFTMAX:
            key = list(sps.softmax(c))
        else:
            key = list(sps.expit(c) + (bias if bias is not None else 0.0))
        order, bgap = brute_topk(key, K)
        assert list(sel[0]) == order
        if math.isinf(bgap):
            assert math.isinf(gap[0])
        else:
            assert abs(gap[0] - bgap) <= 1e-15


def test_exact_tie_goes_to_lower_index():
    u, e = diag_layer([0.5, 0.5, 0.5, 0.25, 0.5])
    sel, g, gap = oracle.route(shape(H=5, N_r=5, K_r=2), u, e)
    assert list(sel[0]) == [0, 1] and gap[0] == 0.0


# ---------------------------------------------------------------- scores (Eq. 8, V3 Eq. 12)

@pytest.mark.parametrize("dtype", [DT_F32, DT_BF16])
def test_logits_and_scores_match_library(dtype):
    T, H, N = 5, 96, 12
    u = synth.normal(1, (T, H), 1.0, dtype)
    e = synth.normal(2, (N, H), H ** -0.5, dtype)
    uf, ef = synth.as_float64(u, dtype), synth.as_float64(e, dtype)
    for gating in (GATE_SOFTMAX, GATE_SIGMOID_BIAS_NORM):
        s = shape(T=T, H=H, N_r=N, K_r=3, gating=gating, dtype=dtype)
        sel, g, gap, lo, sc = oracle.route(s, u, e, want_scores=True)
        ref_l = uf @ ef.T
        np.testing.assert_allclose(lo, ref_l, rtol=0, atol=1e-12)
        ref_s = sps.softmax(ref_l, axis=1) if gating == GATE_SOFTMAX else sps.expit(ref_l)
        np.testing.assert_allclose(sc, ref_s, rtol=1e-13, atol=1e-15)


def test_two_expert_softmax_is_logistic_of_difference():
    u, e = diag_layer([1.25, -0.5])
    sel, g, gap, lo, sc = oracle.route(shape(H=2, N_r=2, K_r=1), u, e, want_scores=True)
    assert abs(sc[0, 0] - 1.0 / (1.0 + math.exp(-(1.25 + 0.5)))) < 1e-15
    assert list(sel[0]) == [0] and abs(g[0, 0] - sc[0, 0]) < 1e-16


# ---------------------------------------------------------------- weights

def test_softmax_weights_unnormalised_and_bounded():
    T, H, N = 40, 64, 16
    u = synth.normal(1, (T, H), 1.0, DT_F32)
    e = synth.normal(2, (N, H), H ** -0.5, DT_F32)
    for K in range(0, N + 1):
        s = shape(T=T, H=H, N_r=N, K_r=K)
        sel, g, gap, lo, sc = oracle.route(s, u, e, want_scores=True)
        assert np.all(g.sum(axis=1) <= 1.0 + 1e-12)
        assert np.array_equal(g, np.take_along_axis(sc, sel.astype(np.int64), axis=1))
        if K == N:
            np.testing.assert_allclose(g.sum(axis=1), 1.0, atol=1e-12)


def test_sigmoid_weights_normalised_over_selected():
    T, H, N = 40, 64, 16
    u = synth.normal(1, (T, H), 1.0, DT_F32)
    e = synth.normal(2, (N, H), H ** -0.5, DT_F32)
    b = synth.normal(3, (N,), 0.1, DT_F32)
    for K in (1, 3, 8, 16):
        s = shape(T=T, H=H, N_r=N, K_r=K, gating=GATE_SIGMOID_BIAS_NORM)
        sel, g, gap, lo, sc = oracle.route(s, u, e, b, want_scores=True)
        np.testing.assert_allclose(g.sum(axis=1), 1.0, atol=1e-12)
        ss = sps.expit(lo)
        picked = np.take_along_axis(ss, sel.astype(np.int64), axis=1)
        np.testing.assert_allclose(g, picked / picked.sum(axis=1, keepdims=True), rtol=1e-13)


def test_masked_softmax_gate_is_softmax_over_selected_logits():
    T, H, N, K = 30, 64, 16, 4
    u = synth.normal(1, (T, H), 1.0, DT_F32)
    e = synth.normal(2, (N, H), H ** -0.5, DT_F32)
    s0 = shape(T=T, H=H, N_r=N, K_r=K, gating=GATE_SOFTMAX)
    s2 = shape(T=T, H=H, N_r=N, K_r=K, gating=GATE_SOFTMAX_RENORM)
    sel0, g0, _ = oracle.route(s0, u, e)
    sel2, g2, _, lo, _ = oracle.route(s2, u, e, want_scores=True)
    assert np.array_equal(sel0, sel2)                      # same selection as Eq. 7
    ref = sps.softmax(np.take_along_axis(lo, sel2.astype(np.int64), axis=1), axis=1)
    np.testing.assert_allclose(g2, ref, rtol=1e-13)
    np.testing.assert_allclose(g2.sum(axis=1), 1.0, atol=1e-12)
    # renormalising Eq. 7's weights over the selected set gives the same numbers
    np.testing.assert_allclose(g2, g0 / g0.sum(axis=1, keepdims=True), rtol=1e-12)


def test_bias_changes_selection_only():
    T, H, N, K = 50, 64, 16, 4
    u = synth.normal(1, (T, H), 1.0, DT_F32)
    e = synth.normal(2, (N, H), H ** -0.5, DT_F32)
    s = shape(T=T, H=H, N_r=N, K_r=K, gating=GATE_SIGMOID_BIAS_NORM)
    b = synth.normal(3, (N,), 0.1, DT_F32)
    sel1, g1, _ = oracle.route(s, u, e, b)
    sel2, g2, _ = oracle.route(s, u, e, (b + np.float32(0.25)).astype(np.float32))  # same ranking
    assert np.array_equal(sel1, sel2) and np.array_equal(g1, g2)
    # a bias large enough to force the set {3, 7, 11, 12}
    forced = np.zeros(N, dtype=np.float32)
    forced[[3, 7, 11, 12]] = 10.0
    sel3, g3, _, lo, sc = oracle.route(s, u, e, forced, want_scores=True)
    assert all(sorted(r) == [3, 7, 11, 12] for r in sel3.tolist())
    picked = np.take_along_axis(sc, sel3.astype(np.int64), axis=1)
    np.testing.assert_allclose(g3, picked / picked.sum(axis=1, keepdims=True), rtol=1e-13)
    # the bias is rejected outside the sigmoid gating
    with pytest.raises(ValueError):
        oracle.route(shape(T=T, H=H, N_r=N, K_r=K), u, e, b)


def test_sigmoid_zero_sum_guard():
    u = np.full((1, 1), 1000.0, dtype=np.float32)
    e = np.full((4, 1), -1.0, dtype=np.float32)            # l = -1000 -> sigmoid = 0 exactly
    b = np.array([0.3, 0.2, 0.1, 0.0], dtype=np.float32)
    sel, g, gap = oracle.route(shape(H=1, N_r=4, K_r=2, gating=GATE_SIGMOID_BIAS_NORM), u, e, b)
    assert list(sel[0]) == [0, 1] and np.array_equal(g[0], [0.5, 0.5])


# ---------------------------------------------------------------- group-limited routing, masking probe

def brute_group_limited(key, G, M, K):
    n = len(key)
    per = n // G
    gsum = [sum(key[g * per + j] for j in range(per)) for g in range(G)]
    groups, _ = brute_topk(gsum, M)
    cand = [i for i in range(n) if i // per in groups]
    sub = [key[i] for i in cand]
    order, _ = brute_topk(sub, K)
    return [cand[i] for i in order]


def test_group_limited_topk_brute_force():
    for trial in range(60):
        G = int(RNG.choice([2, 3, 4]))
        per = int(RNG.integers(1, 4))
        n = G * per
        M = int(RNG.integers(1, G + 1))
        K = int(RNG.integers(1, M * per + 1))
        c = RNG.integers(-4, 5, size=n) / 4.0
        u, e = diag_layer(c)
        gating = GATE_SOFTMAX if trial % 2 else GATE_SIGMOID_BIAS_NORM
        s = shape(H=n, N_r=n, K_r=K, gating=gating, n_group=G, topk_group=M)
        sel, g, gap = oracle.route(s, u, e)
        key = list(sps.softmax(c)) if gating == GATE_SOFTMAX else list(sps.expit(c))
        assert list(sel[0]) == brute_group_limited(key, G, M, K)
        if M == G:   # all groups kept: plain top-k
            sp = shape(H=n, N_r=n, K_r=K, gating=gating)
            assert np.array_equal(oracle.route(sp, u, e)[0], sel)


def test_masking_probe_reselects_from_the_rest():
    T, H, N, K = 30, 64, 16, 4
    u = synth.normal(1, (T, H), 1.0, DT_F32)
    e = synth.normal(2, (N, H), H ** -0.5, DT_F32)
    for r in (0, 1, 3):
        s = shape(T=T, H=H, N_r=N, K_r=K, mask_top_r=r)
        sel, g, gap, lo, sc = oracle.route(s, u, e, want_scores=True)
        wide, _, _ = oracle.route(shape(T=T, H=H, N_r=N, K_r=K + r), u, e)
        assert np.array_equal(sel, wide[:, r:])
        assert np.array_equal(g, np.take_along_axis(sc, sel.astype(np.int64), axis=1))


# ---------------------------------------------------------------- expert FFN (tomabc explainer; SwiGLU)

def test_relu_ffn_linear_regime_matches_numpy():
    H, I = 48, 32
    w1 = synth.normal(4, (I, H), H ** -0.5, DT_F32)
    w2 = synth.normal(5, (H, I), I ** -0.5, DT_F32)
    b1 = np.full(I, 50.0, dtype=np.float32)                # z > 0 everywhere -> ReLU is the identity
    x = synth.normal(1, (H,), 1.0, -1)
    y = oracle.expert_ffn(H, I, ACT_RELU_BIAS, DT_F32, w1, b1, w2, x)
    ref = w2.astype(np.float64) @ (w1.astype(np.float64) @ x + b1.astype(np.float64))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", [DT_F32, DT_BF16])
def test_ffn_matches_torch_fp64(dtype):
    H, I = 64, 40
    for act in (ACT_RELU_BIAS, ACT_SWIGLU):
        n1 = 2 * I if act == ACT_SWIGLU else I
        w1 = synth.normal(4, (n1, H), H ** -0.5, dtype)
        w2 = synth.normal(5, (H, I), I ** -0.5, dtype)
        b1 = synth.normal(8, (I,), 0.3, DT_F32) if act == ACT_RELU_BIAS else None
        x = synth.normal(1, (H,), 1.0, -1)
        y = oracle.expert_ffn(H, I, act, dtype, w1, b1, w2, x)
        W1 = torch.from_numpy(synth.as_float64(w1, dtype))
        W2 = torch.from_numpy(synth.as_float64(w2, dtype))
        X = torch.from_numpy(x)
        if act == ACT_SWIGLU:
            a = torch.nn.functional.silu(W1[:I] @ X) * (W1[I:] @ X)
        else:
            a = torch.relu(W1 @ X + torch.from_numpy(b1.astype(np.float64)))
        np.testing.assert_allclose(y, (W2 @ a).numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("act", [ACT_RELU_BIAS, ACT_SWIGLU])
def test_split_identity_ffn_level(act):
    """Splitting an FFN along I into m slices, all taken with weight 1, gives the coarse FFN."""
    H, M, m = 64, 256, 4
    n1 = 2 * M if act == ACT_SWIGLU else M
    w1 = synth.normal(4, (n1, H), H ** -0.5, DT_F32)
    w2 = synth.normal(5, (H, M), M ** -0.5, DT_F32)
    b1 = synth.normal(8, (M,), 0.5, DT_F32) if act == ACT_RELU_BIAS else None
    x = synth.normal(1, (H,), 1.0, -1)
    coarse = oracle.expert_ffn(H, M, act, DT_F32, w1, b1, w2, x)
    w = M // m
    fine = np.zeros(H)
    for q in range(m):
        cols = slice(q * w, (q + 1) * w)
        if act == ACT_SWIGLU:
            w1q = np.concatenate([w1[:M][cols], w1[M:][cols]])
        else:
            w1q = w1[cols]
        fine += oracle.expert_ffn(H, w, act, DT_F32, w1q, None if b1 is None else b1[cols],
                                  np.ascontiguousarray(w2[:, cols]), x)
    np.testing.assert_allclose(fine, coarse, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- layer-level identities (Eq. 6-11)

def tiny_inputs(T, H, N, K, Ks, I, act=ACT_RELU_BIAS, dtype=DT_F32, gating=GATE_SOFTMAX):
    w = Workload("t", "t", T, H, N, K, Ks, I, gating, act, dtype,
                 bias_var=0.01 if gating == GATE_SIGMOID_BIAS_NORM else 0.0)
    return w, synth.make_inputs(w)


def test_layer_split_identity_coarse_vs_fine():
    """Coarse N=4, M=256, top-1 layer == its m=4 split into 16 experts of width 64, top-4."""
    T, H, N, M, m = 64, 128, 4, 256, 4
    wc, ci = tiny_inputs(T, H, N, 1, 1, M)
    ci["b1"] = synth.normal(8, (N, M), 0.2, DT_F32)
    ci["b1_sh"] = synth.normal(8, (1, M), 0.2, DT_F32, offset=N * M)
    out_c, sel_c, g_c, _ = oracle.layer(oracle.shape_of(wc), ci)
    w = M // m
    fi = dict(ci)
    fi["centroids"] = np.repeat(ci["centroids"], m, axis=0)                    # each slice keeps the centroid
    fi["w1"] = ci["w1"].reshape(N * m, w, H)                                   # rows of W split along I
    fi["b1"] = ci["b1"].reshape(N * m, w)
    fi["w2"] = np.ascontiguousarray(
        (ci["w2"].reshape(N, H, m, w).transpose(0, 2, 1, 3) * np.float32(m)).reshape(N * m, H, w))
    fi["w1_sh"], fi["b1_sh"], fi["w2_sh"] = ci["w1_sh"], ci["b1_sh"], ci["w2_sh"]
    # the shared expert keeps width M, so the routed parts are compared with Ks = 0 on both sides
    sf0 = oracle.shape_of(wc, N_r=N * m, K_r=m, I=w, Ks=0)
    out_f, sel_f, g_f, _ = oracle.layer(sf0, fi)
    sc0 = oracle.shape_of(wc, Ks=0)
    out_c0, _, _, _ = oracle.layer(sc0, ci)
    assert np.array_equal(sel_f, sel_c * m + np.arange(m))                      # the top coarse expert's slices
    np.testing.assert_allclose(g_f, np.repeat(g_c, m, axis=1) / m, rtol=1e-13)
    np.testing.assert_allclose(out_f, out_c0, rtol=1e-12, atol=1e-12)
    # with the shared expert (same width M on both sides) the identity still holds
    sh = np.stack([oracle.expert_ffn(H, M, ACT_RELU_BIAS, DT_F32, ci["w1_sh"][0], ci["b1_sh"][0],
                                     ci["w2_sh"][0], synth.as_float64(ci["u"][t], DT_F32)) for t in range(T)])
    np.testing.assert_allclose(out_f + sh, out_c, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act,dtype", [(ACT_RELU_BIAS, DT_F32), (ACT_SWIGLU, DT_BF16)])
def test_kr_zero_is_shared_plus_residual(act, dtype):
    T, H, N, Ks, I = 6, 64, 8, 2, 32
    w, inp = tiny_inputs(T, H, N, 0, Ks, I, act=act, dtype=dtype)
    out, sel, g, gap = oracle.layer(oracle.shape_of(w), inp)
    uf = synth.as_float64(inp["u"], dtype)
    ref = uf.copy()
    for j in range(Ks):
        for t in range(T):
            ref[t] += oracle.expert_ffn(H, I, act, dtype, inp["w1_sh"][j], None if inp["b1_sh"] is None
                                        else inp["b1_sh"][j], inp["w2_sh"][j], uf[t])
    np.testing.assert_allclose(out, ref, rtol=1e-14, atol=1e-14)
    # no shared experts and no routed ones: the layer is the identity, exactly
    w0 = w.with_(Ks=0)
    out0, _, _, _ = oracle.layer(oracle.shape_of(w0), dict(inp, w1_sh=None, w2_sh=None, b1_sh=None))
    assert np.array_equal(out0, uf)


def test_shared_fold_identity():
    """Ks shared experts of width I == one shared expert of width Ks*I (weights concatenated along I)."""
    T, H, N, K, Ks, I = 8, 64, 8, 2, 2, 32
    w, inp = tiny_inputs(T, H, N, K, Ks, I, act=ACT_SWIGLU, dtype=DT_BF16)
    out2, sel2, g2, _ = oracle.layer(oracle.shape_of(w), inp)
    # one shared expert of width 2I; routed experts padded to width 2I with zero columns (exact no-ops)
    g1 = np.concatenate([inp["w1_sh"][j][:I] for j in range(Ks)])
    u1 = np.concatenate([inp["w1_sh"][j][I:] for j in range(Ks)])
    w1_sh = np.concatenate([g1, u1])[None]
    w2_sh = np.concatenate([inp["w2_sh"][j] for j in range(Ks)], axis=1)[None]
    zr = np.zeros((N, I, H), dtype=np.uint16)
    w1r = np.concatenate([inp["w1"][:, :I], zr, inp["w1"][:, I:], zr], axis=1)
    w2r = np.concatenate([inp["w2"], np.zeros((N, H, I), dtype=np.uint16)], axis=2)
    s1 = oracle.shape_of(w, Ks=1, I=Ks * I)
    out1, sel1, g1_, _ = oracle.layer(s1, dict(inp, w1_sh=np.ascontiguousarray(w1_sh),
                                               w2_sh=np.ascontiguousarray(w2_sh), w1=w1r, w2=w2r))
    assert np.array_equal(sel1, sel2)
    np.testing.assert_allclose(out1, out2, rtol=1e-13, atol=1e-13)


def test_forced_routing_equal_to_own_and_residual_flag():
    T, H, N, K, Ks, I = 10, 64, 16, 4, 1, 32
    w, inp = tiny_inputs(T, H, N, K, Ks, I, act=ACT_SWIGLU, dtype=DT_BF16, gating=GATE_SIGMOID_BIAS_NORM)
    s = oracle.shape_of(w)
    out, sel, g, gap = oracle.layer(s, inp)
    out2, sel2, g2, _ = oracle.layer(s, inp, forced_sel=sel)
    assert np.array_equal(out, out2) and np.array_equal(g, g2)
    moe, _, _, _ = oracle.layer(s, inp, residual=False)
    np.testing.assert_allclose(out - synth.as_float64(inp["u"], DT_BF16), moe, rtol=0, atol=1e-13)
    # subsets of tokens give the same rows (tokens are independent)
    sub = np.array([7, 2, 9])
    out3, sel3, _, _ = oracle.layer(s, inp, tokens=sub)
    assert np.array_equal(out3, out[sub]) and np.array_equal(sel3, sel[sub])


def test_empty_token_list():
    w, inp = tiny_inputs(4, 64, 8, 2, 1, 32)
    out, sel, g, gap = oracle.layer(oracle.shape_of(w), inp, tokens=np.zeros(0, dtype=np.int64))
    assert out.shape == (0, 64) and sel.shape == (0, 2)


def test_bad_arguments_rejected():
    w, inp = tiny_inputs(4, 64, 8, 2, 1, 32)
    with pytest.raises(ValueError):
        oracle.layer(oracle.shape_of(w, K_r=9), inp)
    with pytest.raises(ValueError):
        oracle.layer(oracle.shape_of(w), inp, tokens=np.array([4]))
    with pytest.raises(ValueError):
        oracle.route(oracle.shape_of(w, n_group=3, topk_group=1), inp["u"], inp["centroids"])


# ---------------------------------------------------------------- dispatch and the balance controller

def test_dispatch_matches_nested_loops():
    for trial in range(20):
        T, N = int(RNG.integers(0, 40)), int(RNG.integers(1, 12))
        K = int(RNG.integers(0, N + 1))
        sel = np.stack([RNG.permutation(N)[:K] for _ in range(T)]).astype(np.int32).reshape(T, K)
        offsets, row_token, pair_row = oracle.dispatch(sel, N)
        rows = []
        ref_off = [0]
        for ex in range(N):
            for t in range(T):
                for k in range(K):
                    if sel[t, k] == ex:
                        rows.append((t, k))
            ref_off.append(len(rows))
        assert list(offsets) == ref_off
        assert list(row_token) == [t for t, _ in rows]
        for p, (t, k) in enumerate(rows):
            assert pair_row[t * K + k] == p


def test_bias_update_closed_form():
    b = np.array([0.5, -0.25, 0.0, 1.0], dtype=np.float32)
    out = oracle.bias_update(4, 3, 2, [3, 1, 2, 0], 0.125, b)            # mean load 6/4 = 1.5
    assert np.array_equal(out, np.array([0.375, -0.125, -0.125, 1.125], dtype=np.float32))
    out = oracle.bias_update(2, 2, 1, [1, 1], 0.5, np.array([0.1, 0.2], dtype=np.float32))
    assert np.array_equal(out, np.array([0.1, 0.2], dtype=np.float32))   # at the mean: unchanged
