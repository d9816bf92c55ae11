"""Seeded synthetic inputs for the DeepSeekMoE layer (workload table + generator).

This package draws the random tensors and names the workloads; it contains none
of the layer's arithmetic.  The fp64 oracle (``oracle/``) and the HIP library
(``fine_grained_shared_amd``) both take their inputs from here, bit for bit.

Recipe (x in ``N(0, x)`` is a variance):

======================  ============================  ======
tensor                  distribution                  stream
======================  ============================  ======
u   [T, H]              N(0, 1)                       1
centroids [N_r, H]      N(0, 1/H) (x row scale)       2
bias [N_r] (sigmoid)    N(0, 0.01)                    3
routed W1 [N_r, n1, H]  N(0, 1/H)                     4
routed W2 [N_r, H, I]   N(0, 1/I)                     5
shared W1 [Ks, n1, H]   N(0, 1/H)                     6
shared W2 [Ks, H, I]    N(0, 1/I)                     7
ReLU bias b1            zeros                         (8)
Zipf rank permutation   seeded Fisher-Yates           9
======================  ============================  ======

n1 = 2I for SwiGLU (gate rows [0, I), then up rows [I, 2I)) and I for ReLU.
Every workload uses seed 0, so a decode workload's tokens are exactly the
first T tokens of the matching prefill workload.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

STREAM_U, STREAM_CENTROIDS, STREAM_BIAS = 1, 2, 3
STREAM_W1, STREAM_W2, STREAM_W1_SH, STREAM_W2_SH = 4, 5, 6, 7
STREAM_RELU_B, STREAM_ZIPF_PERM = 8, 9

GATE_SOFTMAX, GATE_SIGMOID_BIAS_NORM, GATE_SOFTMAX_RENORM = 0, 1, 2
ACT_RELU_BIAS, ACT_SWIGLU = 0, 1
DT_F32, DT_BF16 = 0, 1


def build(force: bool = False) -> str:
    """Compile ``libsynth.so`` with gcc (OpenMP, no fast-math, no FMA contraction)."""
    src = os.path.join(_HERE, "gen.c")
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
        u64, i64, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        lib.synth_word.restype = u64
        lib.synth_word.argtypes = [u64, u64, u64]
        lib.synth_normal.restype = dbl
        lib.synth_normal.argtypes = [u64, u64, u64]
        lib.synth_fill_f64.argtypes = [u64, u64, u64, i64, dbl, vp]
        lib.synth_fill_f32.argtypes = [u64, u64, u64, i64, dbl, vp, i64, vp]
        lib.synth_fill_bf16.argtypes = [u64, u64, u64, i64, dbl, vp, i64, vp]
        lib.synth_f32_to_bf16.argtypes = [vp, i64, vp]
        lib.synth_permutation.argtypes = [u64, u64, i64, vp]
        lib.synth_splitmix64.argtypes = [u64, i64, vp]
        _lib = lib
    return _lib


def word(stream: int, idx: int, seed: int = 0) -> int:
    return int(_load().synth_word(seed, stream, idx))


def normal_scalar(stream: int, idx: int, seed: int = 0) -> float:
    return float(_load().synth_normal(seed, stream, idx))


def normal(stream: int, shape, sigma: float, dtype: int, seed: int = 0, offset: int = 0,
           row_scale: Optional[np.ndarray] = None, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Draw ``sigma * N(0,1)`` for the elements ``offset ..`` of ``stream``.

    dtype DT_F32 -> float32 array; DT_BF16 -> uint16 array of bf16 bits; -1 -> float64.
    ``row_scale`` multiplies row r (the last axis is the row) of the flat tensor.
    """
    lib = _load()
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    npdt = {DT_F32: np.float32, DT_BF16: np.uint16, -1: np.float64}[dtype]
    if out is None:
        out = np.empty(shape, dtype=npdt)
    assert out.dtype == npdt and out.flags.c_contiguous and out.size == n
    rs_ptr, row_len, rs = None, 1, None
    if row_scale is not None:
        rs = np.ascontiguousarray(row_scale, dtype=np.float64)
        row_len = shape[-1]
        assert rs.size * row_len == n
        rs_ptr = rs.ctypes.data
    if n == 0:
        return out
    if dtype == -1:
        assert row_scale is None
        lib.synth_fill_f64(seed, stream, offset, n, sigma, out.ctypes.data)
    elif dtype == DT_F32:
        lib.synth_fill_f32(seed, stream, offset, n, sigma, rs_ptr, row_len, out.ctypes.data)
    else:
        lib.synth_fill_bf16(seed, stream, offset, n, sigma, rs_ptr, row_len, out.ctypes.data)
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest even) and return the uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    if x.size:
        _load().synth_f32_to_bf16(x.ctypes.data, x.size, out.ctypes.data)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def splitmix64(state: int, n: int) -> list:
    out = np.zeros(n, dtype=np.uint64)
    _load().synth_splitmix64(state, n, out.ctypes.data)
    return [int(v) for v in out]


def permutation(stream: int, n: int, seed: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().synth_permutation(seed, stream, n, out.ctypes.data)
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    """One layer configuration: shapes, gating, activation and input recipe."""
    name: str
    desc: str
    T: int
    H: int
    N_r: int
    K_r: int
    Ks: int
    I: int
    gating: int
    act: int
    dtype: int
    centroid_scale: str = "none"   # "none" | "hot8x1.5" | "zipf1.1"
    bias_var: float = 0.0          # variance of b_i (sigmoid gating only)
    n_group: int = 0               # group-limited routing: groups (0 = off)
    topk_group: int = 0
    mask_top_r: int = 0            # masking probe

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def n1(self) -> int:
        return 2 * self.I if self.act == ACT_SWIGLU else self.I


WORKLOADS = {
    "c0": Workload("c0", "tiny fp32 layer: T=64 H=128, 16 routed (m=4 split of N=4, M=256) top-4 + 1 shared, "
                   "I=64, ReLU(xW+b)V, softmax", 64, 128, 16, 4, 1, 64,
                   GATE_SOFTMAX, ACT_RELU_BIAS, DT_F32),
    "c1a": Workload("c1a", "2B-style bf16 layer: T=4096 H=2048, 64 routed top-8, no shared, I=1024, SwiGLU, softmax",
                    4096, 2048, 64, 8, 0, 1024, GATE_SOFTMAX, ACT_SWIGLU, DT_BF16),
    "c1b": Workload("c1b", "2B-style bf16 layer: T=4096 H=2048, 64 routed top-7 + 1 shared, I=1024, SwiGLU, softmax",
                    4096, 2048, 64, 7, 1, 1024, GATE_SOFTMAX, ACT_SWIGLU, DT_BF16),
    "c1b_iso": Workload("c1b_iso", "2B-style bf16 layer, iso-parameter split: T=4096 H=2048, 63 routed top-7 + 1 "
                        "shared, I=1024, SwiGLU, softmax", 4096, 2048, 63, 7, 1, 1024,
                        GATE_SOFTMAX, ACT_SWIGLU, DT_BF16),
    "c2": Workload("c2", "16B-style bf16 layer: T=8192 H=2048, 64 routed top-6 + 2 shared, I=1408, SwiGLU, softmax, "
                   "centroids 0-7 x1.5", 8192, 2048, 64, 6, 2, 1408, GATE_SOFTMAX, ACT_SWIGLU, DT_BF16,
                   centroid_scale="hot8x1.5"),
    "c3p": Workload("c3p", "V3-style bf16 layer, prefill: T=16384 H=7168, 256 routed top-8 + 1 shared, I=2048, "
                    "SwiGLU, sigmoid + selection bias", 16384, 7168, 256, 8, 1, 2048,
                    GATE_SIGMOID_BIAS_NORM, ACT_SWIGLU, DT_BF16, bias_var=0.01),
    "c3d": Workload("c3d", "V3-style bf16 layer, decode: T=128 H=7168, 256 routed top-8 + 1 shared, I=2048, "
                    "SwiGLU, sigmoid + selection bias", 128, 7168, 256, 8, 1, 2048,
                    GATE_SIGMOID_BIAS_NORM, ACT_SWIGLU, DT_BF16, bias_var=0.01),
    "c4p": Workload("c4p", "high-sparsity bf16 layer, prefill: T=32768 H=2048, 512 routed top-10 + 1 shared, I=512, "
                    "SwiGLU, sigmoid + selection bias, Zipf(1.1) centroid norms", 32768, 2048, 512, 10, 1, 512,
                    GATE_SIGMOID_BIAS_NORM, ACT_SWIGLU, DT_BF16, centroid_scale="zipf1.1", bias_var=0.01),
    "c4d": Workload("c4d", "high-sparsity bf16 layer, decode: T=64 H=2048, 512 routed top-10 + 1 shared, I=512, "
                    "SwiGLU, sigmoid + selection bias, Zipf(1.1) centroid norms", 64, 2048, 512, 10, 1, 512,
                    GATE_SIGMOID_BIAS_NORM, ACT_SWIGLU, DT_BF16, centroid_scale="zipf1.1", bias_var=0.01),
}


def centroid_row_scale(w: Workload, seed: int = 0) -> Optional[np.ndarray]:
    """Per-expert centroid scale factors of the input recipe."""
    if w.centroid_scale == "none":
        return None
    if w.centroid_scale == "hot8x1.5":
        s = np.ones(w.N_r, dtype=np.float64)
        s[:8] = 1.5
        return s
    if w.centroid_scale == "zipf1.1":
        rank = permutation(STREAM_ZIPF_PERM, w.N_r, seed).astype(np.float64) + 1.0
        f = rank ** -1.1
        return f / np.sqrt(np.mean(f * f))
    raise ValueError(w.centroid_scale)


def make_inputs(w: Workload, seed: int = 0, weights: bool = True) -> dict:
    """All layer inputs as numpy arrays (bf16 tensors as uint16 bits)."""
    dt = w.dtype
    d = {}
    d["u"] = normal(STREAM_U, (w.T, w.H), 1.0, dt, seed)
    d["centroids"] = normal(STREAM_CENTROIDS, (w.N_r, w.H), (1.0 / w.H) ** 0.5, dt, seed,
                            row_scale=centroid_row_scale(w, seed))
    d["bias"] = (normal(STREAM_BIAS, (w.N_r,), w.bias_var ** 0.5, DT_F32, seed)
                 if w.gating == GATE_SIGMOID_BIAS_NORM and w.bias_var > 0 else None)
    if weights:
        d["w1"] = normal(STREAM_W1, (w.N_r, w.n1, w.H), (1.0 / w.H) ** 0.5, dt, seed)
        d["w2"] = normal(STREAM_W2, (w.N_r, w.H, w.I), (1.0 / w.I) ** 0.5, dt, seed)
        d["w1_sh"] = normal(STREAM_W1_SH, (w.Ks, w.n1, w.H), (1.0 / w.H) ** 0.5, dt, seed) if w.Ks else None
        d["w2_sh"] = normal(STREAM_W2_SH, (w.Ks, w.H, w.I), (1.0 / w.I) ** 0.5, dt, seed) if w.Ks else None
        if w.act == ACT_RELU_BIAS:
            d["b1"] = np.zeros((w.N_r, w.I), dtype=np.float32)
            d["b1_sh"] = np.zeros((w.Ks, w.I), dtype=np.float32) if w.Ks else None
        else:
            d["b1"] = None
            d["b1_sh"] = None
    return d


def as_float64(a: Optional[np.ndarray], dtype: int) -> Optional[np.ndarray]:
    """Widen stored input bits to float64 exactly."""
    if a is None:
        return None
    if dtype == DT_BF16 and a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)
