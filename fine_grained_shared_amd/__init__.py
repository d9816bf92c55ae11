"""Python binding of libmoe: the MI355X (gfx950) DeepSeekMoE layer forward pass.

Thin ctypes marshalling over the C ABI in ``include/moe.h`` - every step of the
layer runs in the library's HIP kernels.  PyTorch supplies device memory and
the current stream only.  The functions keep the C names and argument order;
tensors are passed for pointers (``None`` for NULL) and the stream defaults to
torch's current stream.

There is no fallback: if ``libmoe.so`` is missing or cannot be loaded, every
call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_SCRATCH = 0, -1, -2, -3, -4, -5
MOE_GATE_SOFTMAX, MOE_GATE_SIGMOID_BIAS_NORM, MOE_GATE_SOFTMAX_RENORM = 0, 1, 2
MOE_ACT_RELU_BIAS, MOE_ACT_SWIGLU = 0, 1
MOE_F32, MOE_BF16 = 0, 1
MOE_FLAG_NO_RESIDUAL = 1
MOE_FLAG_PACKED_WEIGHTS = 2
MOE_FLAG_PACKED_SHARED_UP = 4
(MOE_PROF_ROUTER, MOE_PROF_DISPATCH, MOE_PROF_FFN_UP, MOE_PROF_FFN_DOWN, MOE_PROF_SHARED_UP,
 MOE_PROF_SHARED_DOWN, MOE_PROF_COMBINE, MOE_PROF_OTHER) = range(8)
PROF_NAMES = ["router", "dispatch", "ffn_up", "ffn_down", "shared_up", "shared_down", "combine", "other"]

# every entry point of include/moe.h
EXPORTS = ("moe_workspace_size", "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_pack_weights",
           "moe_expert_ffn_packed", "moe_shared_ffn", "moe_combine", "moe_layer_forward",
           "moe_layer_forward_noalloc", "moe_noalloc_scratch_bytes", "moe_bias_update",
           "moe_status_string", "moe_last_hip_error", "moe_profile_enable", "moe_profile_query")


class MoeShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "H", "N_r", "K_r", "Ks", "I", "gating", "act", "dtype",
                 "n_group", "topk_group", "mask_top_r")]

    def __repr__(self):
        return "MoeShape(%s)" % ", ".join("%s=%d" % (n, getattr(self, n)) for n, _ in self._fields_)


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (%d)%s" % (what, status_string(status), status,
                                                   " hipError %d" % last_hip_error() if status == MOE_ERR_HIP else ""))


_lib = None


def load() -> ctypes.CDLL:
    """Load libmoe.so (raises if it is not built: no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libmoe.so is not built (%s); run __graft_entry__.build() or "
                           "python fine_grained_shared_amd/build.py" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    sp = ctypes.POINTER(MoeShape)
    sz = ctypes.c_size_t
    sig = {
        "moe_workspace_size": [sp, ctypes.POINTER(ctypes.c_size_t)],
        "moe_route": [sp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_dispatch": [sp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_expert_ffn": [sp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_pack_weights": [vp, vp, i32, i32, i32, vp],
        "moe_expert_ffn_packed": [sp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_shared_ffn": [sp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_combine": [sp, vp, vp, vp, vp, vp, vp, vp],
        "moe_layer_forward": [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp],
        "moe_layer_forward_noalloc": [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp],
        "moe_noalloc_scratch_bytes": [],
        "moe_bias_update": [sp, vp, f32, vp, vp, vp],
        "moe_status_string": [ctypes.c_int],
        "moe_last_hip_error": [],
        "moe_profile_enable": [i32],
        "moe_profile_query": [i32, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = {"moe_status_string": ctypes.c_char_p,
                      "moe_noalloc_scratch_bytes": ctypes.c_size_t}.get(name, ctypes.c_int)
    _lib = lib
    return lib


def make_shape(T, H, N_r, K_r, Ks, I, gating, act, dtype, n_group=0, topk_group=0, mask_top_r=0) -> MoeShape:
    return MoeShape(T, H, N_r, K_r, Ks, I, gating, act, dtype, n_group, topk_group, mask_top_r)


def status_string(status: int) -> str:
    return load().moe_status_string(status).decode()


def last_hip_error() -> int:
    return load().moe_last_hip_error()


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor must be in device memory")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, what: str):
    if rc != MOE_OK:
        raise MoeError(rc, what)


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def moe_workspace_size(shape: MoeShape) -> int:
    n = ctypes.c_size_t(0)
    _check(load().moe_workspace_size(ctypes.byref(shape), ctypes.byref(n)), "moe_workspace_size")
    return n.value


def moe_route(shape, u, centroids, bias, topk_idx, topk_w, ws, stream=None):
    _check(load().moe_route(ctypes.byref(shape), _ptr(u), _ptr(centroids), _ptr(bias), _ptr(topk_idx),
                            _ptr(topk_w), _ptr(ws), _nbytes(ws), _stream(stream)), "moe_route")


def moe_dispatch(shape, topk_idx, offsets, row_token, pair_row, u, x_perm, ws, stream=None):
    _check(load().moe_dispatch(ctypes.byref(shape), _ptr(topk_idx), _ptr(offsets), _ptr(row_token),
                               _ptr(pair_row), _ptr(u), _ptr(x_perm), _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_dispatch")


def moe_expert_ffn(shape, x, row_token, offsets, w1, b1, w2, y, ws, stream=None):
    _check(load().moe_expert_ffn(ctypes.byref(shape), _ptr(x), _ptr(row_token), _ptr(offsets), _ptr(w1),
                                 _ptr(b1), _ptr(w2), _ptr(y), _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_expert_ffn")


def moe_pack_weights(w, packed, G, N, K, stream=None):
    _check(load().moe_pack_weights(_ptr(w), _ptr(packed), int(G), int(N), int(K), _stream(stream)),
           "moe_pack_weights")


def moe_expert_ffn_packed(shape, x, row_token, offsets, w1, b1, w2, y, ws, stream=None):
    _check(load().moe_expert_ffn_packed(ctypes.byref(shape), _ptr(x), _ptr(row_token), _ptr(offsets), _ptr(w1),
                                        _ptr(b1), _ptr(w2), _ptr(y), _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_expert_ffn_packed")


def moe_shared_ffn(shape, x, w1_sh, b1_sh, w2_sh, y, ws, stream=None):
    _check(load().moe_shared_ffn(ctypes.byref(shape), _ptr(x), _ptr(w1_sh), _ptr(b1_sh), _ptr(w2_sh), _ptr(y),
                                 _ptr(ws), _nbytes(ws), _stream(stream)), "moe_shared_ffn")


def moe_combine(shape, residual, y_shared, y_perm, pair_row, topk_w, out, stream=None):
    _check(load().moe_combine(ctypes.byref(shape), _ptr(residual), _ptr(y_shared), _ptr(y_perm), _ptr(pair_row),
                              _ptr(topk_w), _ptr(out), _stream(stream)), "moe_combine")


def moe_layer_forward(shape, u, centroids, bias, w1, b1, w2, w1_sh, b1_sh, w2_sh, flags, out,
                      topk_idx_out, topk_w_out, ws, stream=None):
    _check(load().moe_layer_forward(ctypes.byref(shape), _ptr(u), _ptr(centroids), _ptr(bias), _ptr(w1), _ptr(b1),
                                    _ptr(w2), _ptr(w1_sh), _ptr(b1_sh), _ptr(w2_sh), flags, _ptr(out),
                                    _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(ws), _nbytes(ws), _stream(stream)),
           "moe_layer_forward")


def moe_layer_forward_noalloc(shape, u, centroids, bias, w1, b1, w2, w1_sh, b1_sh, w2_sh, flags, out,
                              topk_idx_out, topk_w_out, stream=None):
    _check(load().moe_layer_forward_noalloc(ctypes.byref(shape), _ptr(u), _ptr(centroids), _ptr(bias), _ptr(w1),
                                            _ptr(b1), _ptr(w2), _ptr(w1_sh), _ptr(b1_sh), _ptr(w2_sh), flags,
                                            _ptr(out), _ptr(topk_idx_out), _ptr(topk_w_out), _stream(stream)),
           "moe_layer_forward_noalloc")


def moe_noalloc_scratch_bytes() -> int:
    return load().moe_noalloc_scratch_bytes()


def moe_bias_update(shape, offsets, gamma, bias, counts, stream=None):
    _check(load().moe_bias_update(ctypes.byref(shape), _ptr(offsets), float(gamma), _ptr(bias), _ptr(counts),
                                  _stream(stream)), "moe_bias_update")


def moe_profile_enable(on: bool):
    _check(load().moe_profile_enable(1 if on else 0), "moe_profile_enable")


def moe_profile_query(kernel: int):
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    _check(load().moe_profile_query(kernel, ctypes.byref(n), ctypes.byref(ms)), "moe_profile_query")
    return n.value, ms.value


# ---------------------------------------------------------------- conveniences (allocation via torch)

def torch_dtype(shape: MoeShape):
    import torch
    return torch.float32 if shape.dtype == MOE_F32 else torch.bfloat16


def workspace(shape: MoeShape, device="cuda"):
    import torch
    n = moe_workspace_size(shape)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def pack_weights(w, stream=None):
    """Return a new tensor holding the [G, N, K] bf16 bank w in the packed order of moe_pack_weights."""
    import torch
    G, N, K = w.shape
    out = torch.empty_like(w, memory_format=torch.contiguous_format)
    moe_pack_weights(w, out, G, N, K, stream)
    return out


def layer_forward(shape, u, centroids, bias, w1, b1, w2, w1_sh=None, b1_sh=None, w2_sh=None, flags=0,
                  ws=None, stream=None):
    """Allocate the outputs and run moe_layer_forward; returns (out, topk_idx, topk_w)."""
    import torch
    dev = u.device
    out = torch.empty((shape.T, shape.H), dtype=torch_dtype(shape), device=dev)
    idx = torch.empty((shape.T, shape.K_r), dtype=torch.int32, device=dev)
    w = torch.empty((shape.T, shape.K_r), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(shape, dev)
    moe_layer_forward(shape, u, centroids, bias, w1, b1, w2, w1_sh, b1_sh, w2_sh, flags, out, idx, w, ws, stream)
    return out, idx, w
