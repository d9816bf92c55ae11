"""fp64 CPU oracle for the DeepSeekMoE layer forward pass.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``fine_grained_shared_amd``) and never imports it;
the only module both sides use is ``synth`` (seeded inputs, no layer maths).

Routing, expert FFNs and the layer sum are plain C (``oracle.c``); the dispatch
definition below is a stable sort by expert id (numpy's stable argsort as the
library step).

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against brute force, closed forms and library routines; the numeric values of
random bf16 layers beyond those identities are "parity unpinned" (no page
prints a worked numeric example).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None


class OrcShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "H", "N_r", "K_r", "Ks", "I", "gating", "act", "dtype",
                 "n_group", "topk_group", "mask_top_r")]


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc: -O2, OpenMP, no FMA contraction, no fast-math."""
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-shared", "-fPIC", "-o", tmp, src, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        sp = ctypes.POINTER(OrcShape)
        lib.orc_route.restype = ctypes.c_int
        lib.orc_route.argtypes = [sp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp]
        lib.orc_expert_ffn.restype = ctypes.c_int
        lib.orc_expert_ffn.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
        lib.orc_layer.restype = ctypes.c_int
        lib.orc_layer.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, i32, vp, vp, vp, vp]
        lib.orc_bias_update.restype = ctypes.c_int
        lib.orc_bias_update.argtypes = [i32, i64, i32, vp, ctypes.c_float, vp, vp]
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the oracle runs with (OMP_NUM_THREADS, else all cores)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.strip().isdigit():
        return int(env)
    return os.cpu_count() or 1


def shape_of(w, T: Optional[int] = None, **over) -> OrcShape:
    d = dict(T=w.T if T is None else T, H=w.H, N_r=w.N_r, K_r=w.K_r, Ks=w.Ks, I=w.I, gating=w.gating,
             act=w.act, dtype=w.dtype, n_group=w.n_group, topk_group=w.topk_group, mask_top_r=w.mask_top_r)
    d.update(over)
    return OrcShape(**d)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dt=None):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dt) if dt is not None else np.ascontiguousarray(a)


def _tokens(s: OrcShape, tokens) -> np.ndarray:
    if tokens is None:
        return np.arange(s.T, dtype=np.int64)
    return np.ascontiguousarray(tokens, dtype=np.int64)


def route(s: OrcShape, u, centroids, bias=None, tokens=None, want_scores: bool = False):
    """Routing of the listed tokens: (sel [n,K_r] int32, g [n,K_r] f64, gap [n] f64[, logits, scores])."""
    tok = _tokens(s, tokens)
    n = tok.size
    sel = np.zeros((n, s.K_r), dtype=np.int32)
    g = np.zeros((n, s.K_r), dtype=np.float64)
    gap = np.zeros(n, dtype=np.float64)
    lo = np.zeros((n, s.N_r), dtype=np.float64) if want_scores else None
    sc = np.zeros((n, s.N_r), dtype=np.float64) if want_scores else None
    u, centroids, bias = _c(u), _c(centroids), _c(bias, np.float32)
    rc = _load().orc_route(ctypes.byref(s), _ptr(u), _ptr(centroids), _ptr(bias), _ptr(tok), n,
                           _ptr(sel), _ptr(g), _ptr(gap), _ptr(lo), _ptr(sc))
    if rc != 0:
        raise ValueError("orc_route rejected its arguments")
    return (sel, g, gap, lo, sc) if want_scores else (sel, g, gap)


def expert_ffn(H: int, I: int, act: int, dtype: int, w1, b1, w2, x) -> np.ndarray:
    """One expert on one fp64 vector: ReLU(Wx+b)->V or SwiGLU; weights [out, in]."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.zeros(H, dtype=np.float64)
    w1, w2, b1 = _c(w1), _c(w2), _c(b1, np.float32)
    rc = _load().orc_expert_ffn(H, I, act, dtype, _ptr(w1), _ptr(b1), _ptr(w2), _ptr(x), _ptr(y))
    if rc != 0:
        raise ValueError("orc_expert_ffn rejected its arguments")
    return y


def layer(s: OrcShape, inp: dict, tokens=None, forced_sel=None, residual: bool = True):
    """Layer output for the listed tokens: (out [n,H] f64, sel, g, gap)."""
    tok = _tokens(s, tokens)
    n = tok.size
    out = np.zeros((n, s.H), dtype=np.float64)
    sel = np.zeros((n, s.K_r), dtype=np.int32)
    g = np.zeros((n, s.K_r), dtype=np.float64)
    gap = np.zeros(n, dtype=np.float64)
    fs = _c(forced_sel, np.int32)
    a = {k: _c(v) for k, v in inp.items() if k not in ("bias", "b1", "b1_sh")}
    bias, b1, b1_sh = _c(inp.get("bias"), np.float32), _c(inp.get("b1"), np.float32), _c(inp.get("b1_sh"), np.float32)
    rc = _load().orc_layer(ctypes.byref(s), _ptr(a["u"]), _ptr(a.get("centroids")), _ptr(bias),
                           _ptr(a.get("w1")), _ptr(b1), _ptr(a.get("w2")),
                           _ptr(a.get("w1_sh")), _ptr(b1_sh), _ptr(a.get("w2_sh")),
                           _ptr(tok), n, _ptr(fs), 1 if residual else 0,
                           _ptr(out), _ptr(sel), _ptr(g), _ptr(gap))
    if rc != 0:
        raise ValueError("orc_layer rejected its arguments")
    return out, sel, g, gap


def dispatch(sel: np.ndarray, N_r: int):
    """Contiguous per-expert segments, ordered by (token, slot) inside each segment.

    Returns offsets [N_r+1], row_token [T*K_r] (token of each permuted row) and
    pair_row [T*K_r] (permuted row of pair (t, k), flat t*K_r + k).
    """
    sel = np.ascontiguousarray(sel, dtype=np.int64)
    T, K = sel.shape
    flat = sel.reshape(-1)
    order = np.argsort(flat, kind="stable")          # pairs ordered by expert, then by (t, k)
    counts = np.bincount(flat, minlength=N_r)
    offsets = np.zeros(N_r + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    row_token = (order // max(K, 1)).astype(np.int32)
    pair_row = np.empty(T * K, dtype=np.int32)
    pair_row[order] = np.arange(T * K, dtype=np.int32)
    return offsets, row_token, pair_row


def bias_update(N_r: int, T: int, K_r: int, counts, gamma: float, bias) -> np.ndarray:
    """One step of the aux-loss-free balance controller; returns the new fp32 bias."""
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    b = np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty_like(b)
    rc = _load().orc_bias_update(N_r, T, K_r, _ptr(counts), gamma, _ptr(b), _ptr(out))
    if rc != 0:
        raise ValueError("orc_bias_update rejected its arguments")
    return out
