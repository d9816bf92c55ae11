"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path, compare with the oracle."""
import sys

import numpy as np

import oracle
import synth

# Tolerances (from the layer's stated parity bar): routing sets bit-exact outside near ties
# (oracle key gap < 1e-6), gate weights within 1e-6, bf16 outputs within 5e-3 relative
# Frobenius and 2e-2 * rms(ref) max-abs, fp32 outputs within 1e-5 relative Frobenius.
NEAR_TIE = 1e-6
W_TOL = 1e-6
BF16_FRO, BF16_MAX = 5e-3, 2e-2
F32_FRO = 1e-5


# one line per compared output (label, relative Frobenius, max abs / rms, near ties), printed at the
# end of the session by tests/conftest.py
RESULTS = []


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(arr):
    import torch
    if arr is None:
        return None
    a = np.ascontiguousarray(arr)
    t = torch.from_numpy(a)
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def to_f64(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def gpu_shape(w, T=None, **over):
    import fine_grained_shared_amd as moe
    d = dict(T=w.T if T is None else T, H=w.H, N_r=w.N_r, K_r=w.K_r, Ks=w.Ks, I=w.I, gating=w.gating, act=w.act,
             dtype=w.dtype, n_group=w.n_group, topk_group=w.topk_group, mask_top_r=w.mask_top_r)
    d.update(over)
    return moe.MoeShape(**d)


class Case:
    """A workload's seeded inputs on host and device."""

    def __init__(self, w, inputs=None):
        self.w = w
        self.inp = inputs if inputs is not None else synth.make_inputs(w)
        self.dev = {k: to_dev(v) for k, v in self.inp.items()}

    def with_tokens(self, T):
        """The same layer on the first T tokens (the decode slice of a prefill workload)."""
        w = self.w.with_(T=T)
        c = Case.__new__(Case)
        c.w = w
        c.inp = dict(self.inp)
        c.inp["u"] = np.ascontiguousarray(self.inp["u"][:T])
        c.dev = dict(self.dev)
        c.dev["u"] = self.dev["u"][:T].contiguous()
        return c

    def forward(self, flags=0, shape=None, u=None, bias="default"):
        import fine_grained_shared_amd as moe
        s = shape if shape is not None else gpu_shape(self.w)
        d = self.dev
        b = d["bias"] if bias == "default" else bias
        flags |= getattr(self, "extra_flags", 0)   # e.g. MOE_FLAG_PACKED_WEIGHTS for packed routed banks
        return moe.layer_forward(s, d["u"] if u is None else u, d["centroids"], b, d["w1"], d["b1"], d["w2"],
                                 d["w1_sh"], d["b1_sh"], d["w2_sh"], flags=flags)


def check_routing(sel_gpu, w_gpu, sel_orc, g_orc, gap, label=""):
    """Index sets equal outside near ties; weights aligned by expert within W_TOL. Returns #near ties."""
    near = gap < NEAR_TIE
    far = ~near
    sg = np.sort(sel_gpu, axis=1)
    so = np.sort(sel_orc, axis=1)
    bad = np.nonzero(far & ~np.all(sg == so, axis=1))[0]
    assert bad.size == 0, "%s: %d tokens routed differently (first %d: gpu %s oracle %s gap %g)" % (
        label, bad.size, bad[0], sel_gpu[bad[0]], sel_orc[bad[0]], gap[bad[0]])
    same = np.all(sg == so, axis=1)
    og = np.argsort(sel_gpu, axis=1, kind="stable")
    oo = np.argsort(sel_orc, axis=1, kind="stable")
    wg = np.take_along_axis(w_gpu, og, axis=1)[same]
    wo = np.take_along_axis(g_orc, oo, axis=1)[same]
    if wg.size:
        err = np.abs(wg - wo).max()
        assert err <= W_TOL, "%s: gate weight error %g > %g" % (label, err, W_TOL)
    return int(near.sum())


def check_close(got, ref, dtype, label="", output_rounding=False):
    """Relative Frobenius and max-abs checks.  output_rounding: the compared tensor is itself a
    bf16 output of a different quantity than the bar was set for (the MoE-only part); each
    element may then also differ by its own bf16 rounding, at most 2^-8 |ref|."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % label
    den = np.linalg.norm(ref)
    fro = np.linalg.norm(got - ref) / max(den, 1e-300)
    if dtype == synth.DT_F32:
        RESULTS.append({"label": label, "n": int(ref.shape[0]) if ref.ndim else 0, "fro": fro, "max_over_rms": None})
        assert fro <= F32_FRO, "%s: rel Frobenius %g > %g" % (label, fro, F32_FRO)
    else:
        rms = den / np.sqrt(max(ref.size, 1))
        err = np.abs(got - ref)
        allow = BF16_MAX * rms + (2.0 ** -8 * np.abs(ref) if output_rounding else 0.0)
        excess = (err - allow).max() if ref.size else -1.0
        mx = err.max() if ref.size else 0.0
        say("[check] %s: rel Frobenius %.3e, max abs %.3e = %.4f rms" % (label, fro, mx, mx / max(rms, 1e-300)))
        RESULTS.append({"label": label, "n": int(ref.shape[0]) if ref.ndim else 0, "fro": fro,
                        "max_over_rms": mx / max(rms, 1e-300)})
        assert fro <= BF16_FRO, "%s: rel Frobenius %g > %g" % (label, fro, BF16_FRO)
        assert excess <= 0.0, "%s: max abs %g beyond %g * rms %g%s" % (
            label, mx, BF16_MAX, rms, " + 2^-8 |ref|" if output_rounding else "")
    return fro


def sample_tokens(T, n, seed=7):
    """n distinct token ids: both ends, a stride through the middle and a seeded random set."""
    if T <= n:
        return np.arange(T, dtype=np.int64)
    rng = np.random.default_rng(seed)
    s = set([0, T - 1])
    s.update(np.linspace(0, T - 1, n // 2).astype(np.int64).tolist())
    while len(s) < n:
        s.add(int(rng.integers(0, T)))
    return np.array(sorted(s), dtype=np.int64)


def cover_routed_tiles(sel, N_r, tokens, tile=128):
    """tokens, extended so that every m-tile of `tile` rows of every routed expert segment (the rows
    of the grouped GEMMs, ordered by expert, then by (token, slot)) holds a row of a listed token.
    Returns (sorted token ids, number of m-tiles, number added)."""
    offsets, row_token, _ = oracle.dispatch(sel, N_r)
    have = np.zeros(sel.shape[0], dtype=bool)
    have[np.asarray(tokens, dtype=np.int64)] = True
    n_tiles = added = 0
    for e in range(N_r):
        for r0 in range(int(offsets[e]), int(offsets[e + 1]), tile):
            rows = row_token[r0:min(r0 + tile, int(offsets[e + 1]))]
            n_tiles += 1
            if not have[rows].any():
                have[rows[0]] = True
                added += 1
    return np.nonzero(have)[0].astype(np.int64), n_tiles, added


def strided_tokens(T, stride):
    """Every stride-th token (0, stride, ...) and the last one."""
    return np.unique(np.concatenate([np.arange(0, T, stride), [T - 1]])).astype(np.int64)


def layer_parity(case, tokens=None, route_all=True, label="", cover_tiles=False):
    """Run the layer on the GPU and compare with the oracle. Returns a dict of stats.

    tokens: the token ids whose outputs are compared (None = all).  cover_tiles: extend them so that
    every 128-row m-tile of every routed expert segment holds a compared row.  The MoE-only part
    (run with MOE_FLAG_NO_RESIDUAL) is compared with the oracle's output minus u, formed in fp64."""
    import torch
    import fine_grained_shared_amd as moe
    w = case.w
    say("[parity] %s: GPU layer forward T=%d" % (label or w.name, w.T))
    out, idx, wts = case.forward()
    moe_part, idx2, _ = case.forward(flags=moe.MOE_FLAG_NO_RESIDUAL)
    torch.cuda.synchronize()
    sel_gpu = idx.cpu().numpy()
    w_gpu = wts.cpu().numpy().astype(np.float64)
    assert np.array_equal(sel_gpu, idx2.cpu().numpy())
    s = oracle.shape_of(w)
    stats = {}
    if w.K_r > 0:
        rt = None if route_all else tokens
        say("[parity] %s: oracle routing on %s tokens" % (label or w.name, "all" if rt is None else len(rt)))
        sel_o, g_o, gap = oracle.route(s, case.inp["u"], case.inp["centroids"], case.inp["bias"], tokens=rt)
        rows = slice(None) if rt is None else rt
        stats["near_ties"] = check_routing(sel_gpu[rows], w_gpu[rows], sel_o, g_o, gap, label)
    tok = np.arange(w.T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    if cover_tiles and w.K_r > 0 and tokens is not None:
        tok, n_tiles, added = cover_routed_tiles(sel_gpu, w.N_r, tok)
        stats["routed_m_tiles"], stats["tokens_added_for_tiles"] = n_tiles, added
    stats["tokens_checked"] = int(len(tok))
    say("[parity] %s: oracle layer on %d tokens" % (label or w.name, len(tok)))
    forced = sel_gpu[tok] if w.K_r > 0 else None
    ref, _, _, _ = oracle.layer(s, case.inp, tokens=tok, forced_sel=forced)
    ref_moe = ref - synth.as_float64(case.inp["u"][tok], w.dtype)
    stats["fro_out"] = check_close(to_f64(out)[tok], ref, w.dtype, label + " out")
    stats["fro_moe"] = check_close(to_f64(moe_part)[tok], ref_moe, w.dtype, label + " moe part",
                                   output_rounding=True)
    say("[parity] %s: ok %s" % (label or w.name, stats))
    for r in RESULTS[-2:]:
        r["near_ties"] = stats.get("near_ties")
    return stats, (out, idx, wts)
