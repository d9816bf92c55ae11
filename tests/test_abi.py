"""Host-side checks of the C ABI library (no GPU work): symbols, status strings, argument checks."""
import re
import os

import pytest

import fine_grained_shared_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_binding_exports():
    assert declared() == sorted(moe.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = moe.load()
    for name in declared():
        assert hasattr(lib, name), name


def test_status_strings():
    assert moe.status_string(0) == "ok"
    assert "workspace" in moe.status_string(moe.MOE_ERR_WORKSPACE)
    assert moe.status_string(12345) == "unknown status"


@pytest.mark.parametrize("bad", [
    dict(K_r=17), dict(H=100), dict(I=96 + 1), dict(T=-1), dict(gating=3), dict(dtype=2),
    dict(n_group=3, topk_group=1), dict(n_group=4, topk_group=5), dict(n_group=4, topk_group=1, K_r=5),
    dict(mask_top_r=13), dict(n_group=4, topk_group=2, mask_top_r=1),
])
def test_invalid_shapes_rejected_on_host(bad):
    d = dict(T=16, H=128, N_r=16, K_r=4, Ks=1, I=64, gating=0, act=1, dtype=1)
    d.update(bad)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_workspace_size(moe.make_shape(**d))
    assert e.value.status == moe.MOE_ERR_INVALID_ARG


def test_unsupported_shapes():
    with pytest.raises(moe.MoeError) as e:
        moe.moe_workspace_size(moe.make_shape(16, 128, 2048, 4, 1, 64, 0, 1, 1))
    assert e.value.status == moe.MOE_ERR_UNSUPPORTED


def test_workspace_size_grows_with_tokens():
    a = moe.moe_workspace_size(moe.make_shape(128, 7168, 256, 8, 1, 2048, 1, 1, 1))
    b = moe.moe_workspace_size(moe.make_shape(16384, 7168, 256, 8, 1, 2048, 1, 1, 1))
    assert 0 < a < b
    # the permuted rows dominate: T*K_r rows of H and of I, bf16
    assert b >= 16384 * 8 * (7168 + 2048) * 2


def test_calls_rejected_before_any_launch():
    s = moe.make_shape(16, 128, 16, 4, 1, 64, 0, 1, 1)
    lib = moe.load()
    import ctypes
    # NULL required pointers -> invalid argument, returned by the host checks
    assert lib.moe_route(ctypes.byref(s), None, None, None, None, None, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_forward(ctypes.byref(s), None, None, None, None, None, None, None, None, None, 0, None,
                                 None, None, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    # unknown flag bits
    assert lib.moe_layer_forward(ctypes.byref(s), None, None, None, None, None, None, None, None, None, 8, None,
                                 None, None, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    # empty token batch: nothing to do
    s0 = moe.make_shape(0, 128, 16, 4, 1, 64, 0, 1, 1)
    assert lib.moe_layer_forward(ctypes.byref(s0), None, None, None, None, None, None, None, None, None, 0, None,
                                 None, None, None, 0, None) == moe.MOE_OK
    assert lib.moe_profile_query(99, ctypes.byref(ctypes.c_int64()), ctypes.byref(ctypes.c_double())) == \
        moe.MOE_ERR_INVALID_ARG


def test_packed_weight_calls_rejected_before_any_launch():
    """moe_pack_weights / moe_expert_ffn_packed / MOE_FLAG_PACKED_* argument checks (host only:
    the pointers are never dereferenced because every case is rejected before a launch)."""
    import ctypes
    lib = moe.load()
    A, B = 1 << 20, 1 << 30   # 16-byte aligned stand-ins, far apart
    assert lib.moe_pack_weights(A, B, 2, 48, 128, None) == moe.MOE_ERR_INVALID_ARG    # N % 32
    assert lib.moe_pack_weights(A, B, 2, 64, 96, None) == moe.MOE_ERR_INVALID_ARG     # K % 64
    assert lib.moe_pack_weights(A, B, -1, 64, 64, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_pack_weights(A, A + 4096, 1, 64, 64, None) == moe.MOE_ERR_INVALID_ARG  # overlap
    assert lib.moe_pack_weights(A + 8, B, 1, 64, 64, None) == moe.MOE_ERR_INVALID_ARG     # alignment
    assert lib.moe_pack_weights(None, B, 1, 64, 64, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_pack_weights(A, B, 1, 32768, 65536, None) == moe.MOE_ERR_UNSUPPORTED   # 4 GiB matrix
    assert lib.moe_pack_weights(None, None, 0, 64, 64, None) == moe.MOE_OK               # nothing to pack
    # fp32 layers have no packed form
    s32 = moe.make_shape(16, 128, 16, 4, 1, 64, 0, 1, moe.MOE_F32)
    assert lib.moe_expert_ffn_packed(ctypes.byref(s32), A, None, A, A, None, A, A, A, 1 << 30, None) == \
        moe.MOE_ERR_INVALID_ARG
    for flag in (moe.MOE_FLAG_PACKED_WEIGHTS, moe.MOE_FLAG_PACKED_SHARED_UP):
        assert lib.moe_layer_forward(ctypes.byref(s32), None, None, None, None, None, None, None, None, None,
                                     flag, None, None, None, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    s16 = moe.make_shape(16, 128, 16, 4, 1, 64, 0, 1, moe.MOE_BF16)
    assert lib.moe_layer_forward(ctypes.byref(s16), None, None, None, None, None, None, None, None, None,
                                 8, None, None, None, None, 0, None) == moe.MOE_ERR_INVALID_ARG   # unknown flag
    # bf16 with too large an expert matrix for 32-bit offsets
    sbig = moe.make_shape(16, 65536, 16, 4, 0, 16384, 0, 1, moe.MOE_BF16)
    assert lib.moe_layer_forward(ctypes.byref(sbig), None, None, None, None, None, None, None, None, None,
                                 moe.MOE_FLAG_PACKED_WEIGHTS, None, None, None, None, 0, None) == \
        moe.MOE_ERR_UNSUPPORTED


def test_no_kernel_uses_scratch_memory():
    """Every HIP kernel keeps its working set in registers/LDS (hipcc resource report): at most a
    few spilled registers, no arrays in scratch memory."""
    import subprocess
    from fine_grained_shared_amd import build as hb
    for src in hb.SOURCES:
        out = subprocess.run([os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")] + hb.FLAGS +
                             ["-c", os.path.join(hb.CSRC, src), "-o", os.devnull,
                              "-Rpass-analysis=kernel-resource-usage"],
                             capture_output=True, text=True)
        assert out.returncode == 0, out.stderr[-2000:]
        names = re.findall(r"Function Name: (\S+)", out.stderr)
        scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", out.stderr)]
        spills = [int(x) for x in re.findall(r"VGPRs Spill: (\d+)", out.stderr)]
        assert len(names) == len(scratch) == len(spills)
        assert names or src == "api.hip"   # the C-ABI file holds host code only
        # scratch may only hold a few spilled registers, never arrays placed in memory
        bad = [(n, sz, sp) for n, sz, sp in zip(names, scratch, spills) if sz > 4 * sp + 16 or sp > 16]
        assert not bad, "kernels using scratch: %s" % bad
