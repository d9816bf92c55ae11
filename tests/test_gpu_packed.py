"""GPU: routed expert weights stored in fragment order (moe_pack_weights).

The packing kernel is checked against the layout written out on the host.  The packed layer and the
packed expert FFN are checked against the unpacked ones bit for bit: every GEMM kernel accumulates an
output in one fixed order, so the storage order of the weights cannot change a result.  One packed
layer is also compared with the oracle.  The shapes cover the packed kernels (the 128 x 512 tile, the
128 x 256 tile of reductions up to 512 and the 32-row decode tile, grouped for the routed experts and
dense for the shared up bank), odd k-step counts, ragged column tiles and empty expert groups.
"""
import gc

import numpy as np
import pytest

import synth
from parity_util import Case, gpu_shape, layer_parity, say, to_dev
from synth import ACT_RELU_BIAS, DT_BF16, GATE_SIGMOID_BIAS_NORM, GATE_SOFTMAX, ACT_SWIGLU, Workload

pytestmark = pytest.mark.gpu

# T=600 x top-3 over 16 experts: ~112 rows per expert (the 128 x 512 tile) with ragged m-tiles;
# H=320 and I=192: 5 and 3 k-steps of 64 (odd counts), I=192 a ragged SwiGLU column tile.
RAGGED = Workload("packed_ragged", "ragged bf16 SwiGLU sigmoid+bias layer", 600, 320, 16, 3, 2, 192,
                  GATE_SIGMOID_BIAS_NORM, ACT_SWIGLU, DT_BF16, bias_var=0.01)

VARIANTS = {
    "ragged": RAGGED,
    # reductions longer than 8 k-steps (H=576: 9, I=640: 10) take the 128 x 512 tile; ragged column tiles
    "ragged_wide": RAGGED.with_(name="packed_ragged_wide", H=576, I=640),
    "ragged_decode": RAGGED.with_(name="packed_ragged_decode", T=40),
    "relu": RAGGED.with_(name="packed_relu", gating=GATE_SOFTMAX, act=ACT_RELU_BIAS, bias_var=0.0, I=256),
    "relu_decode": RAGGED.with_(name="packed_relu_decode", gating=GATE_SOFTMAX, act=ACT_RELU_BIAS, bias_var=0.0,
                                I=256, T=24),
    "many_experts": RAGGED.with_(name="packed_many_experts", T=200, N_r=600, K_r=12, Ks=1, I=64, H=256),
    "no_shared": RAGGED.with_(name="packed_no_shared", Ks=0, K_r=5),
    # 500 dense rows x I=2048: 16 x 16 = 256 of the 32-row shared tiles, so the dense GEMMs take the
    # four-wave decode tile (fewer would take the one-wave one)
    "dense_four_wave": RAGGED.with_(name="packed_dense_four_wave", T=500, H=256, I=2048, K_r=2, Ks=1),
}


def pack_host(w: np.ndarray) -> np.ndarray:
    """The documented packed order: per matrix, block nb * (K/16) + kc of 64 pieces of 8 elements,
    piece l = row 32 nb + l % 32, columns 16 kc + 8 (l // 32) .. + 7."""
    G, N, K = w.shape
    x = w.reshape(G, N // 32, 32, K // 16, 2, 8)        # g, nb, r, kc, half, e
    return np.ascontiguousarray(x.transpose(0, 1, 3, 4, 2, 5)).reshape(G, N, K)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fine_grained_shared_amd as moe
    moe.load()
    return torch


def packed_case(case, routed=True, shared=True):
    """The same case with the routed banks and / or the shared up bank packed on the GPU (and the flags
    set for its forward)."""
    import fine_grained_shared_amd as moe
    c = Case.__new__(Case)
    c.w, c.inp = case.w, case.inp
    c.dev = dict(case.dev)
    c.extra_flags = 0
    if routed:
        c.dev["w1"] = moe.pack_weights(case.dev["w1"])
        c.dev["w2"] = moe.pack_weights(case.dev["w2"])
        c.extra_flags |= moe.MOE_FLAG_PACKED_WEIGHTS
    if shared and case.w.Ks > 0:
        c.dev["w1_sh"] = moe.pack_weights(case.dev["w1_sh"])
        c.extra_flags |= moe.MOE_FLAG_PACKED_SHARED_UP
    return c


def assert_same_layer(case, pcase, label):
    import torch
    import fine_grained_shared_amd as moe
    for flags in (0, moe.MOE_FLAG_NO_RESIDUAL):
        out, idx, wts = case.forward(flags=flags)
        pout, pidx, pwts = pcase.forward(flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(idx, pidx) and torch.equal(wts, pwts), label
        same = torch.equal(out.view(torch.int16), pout.view(torch.int16))
        if not same:
            d = (out.float() - pout.float()).abs()
            raise AssertionError("%s flags=%d: packed output differs in %d elements (max %g)" % (
                label, flags, int((d > 0).sum()), float(d.max())))
    say("[packed] %s: bit-identical to the unpacked layer" % label)


def test_pack_layout(torch_cuda):
    import fine_grained_shared_amd as moe
    torch = torch_cuda
    for (G, N, K) in [(3, 96, 192), (2, 32, 64), (1, 4096, 448)]:
        w = synth.normal(synth.STREAM_W1, (G, N, K), 1.0, DT_BF16, seed=G * 1000 + N)
        got = moe.pack_weights(to_dev(w))
        torch.cuda.synchronize()
        ref = pack_host(w)
        assert np.array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), ref), (G, N, K)


@pytest.mark.parametrize("name", list(VARIANTS))
def test_packed_layer_bit_identical(torch_cuda, name):
    case = Case(VARIANTS[name])
    assert_same_layer(case, packed_case(case), name)


@pytest.mark.parametrize("name", ["ragged", "ragged_decode", "relu"])
def test_packed_shared_up_only_bit_identical(torch_cuda, name):
    """Only the shared up bank packed: the dense packed GEMM (two shared experts side by side, 600 rows
    on the 128-row tiles, 40 rows on the 32-row decode tiles) next to [out, in] routed banks."""
    case = Case(VARIANTS[name])
    assert_same_layer(case, packed_case(case, routed=False), name + "_shared_only")


def test_packed_layer_against_oracle(torch_cuda):
    case = packed_case(Case(RAGGED))
    layer_parity(case, label="packed_ragged")


def test_packed_expert_ffn_bit_identical(torch_cuda):
    """moe_expert_ffn_packed against moe_expert_ffn, from x_perm and with the fused row gather."""
    import fine_grained_shared_amd as moe
    torch = torch_cuda
    case = Case(RAGGED.with_(name="packed_stage", T=700))
    w, d = case.w, case.dev
    s = gpu_shape(w)
    ws = moe.workspace(s)
    R = w.T * w.K_r
    idx = torch.empty((w.T, w.K_r), dtype=torch.int32, device="cuda")
    gw = torch.empty((w.T, w.K_r), dtype=torch.float32, device="cuda")
    moe.moe_route(s, d["u"], d["centroids"], d["bias"], idx, gw, ws)
    offsets = torch.empty(w.N_r + 1, dtype=torch.int32, device="cuda")
    row_token = torch.empty(R, dtype=torch.int32, device="cuda")
    pair_row = torch.empty(R, dtype=torch.int32, device="cuda")
    x_perm = torch.empty((R, w.H), dtype=torch.bfloat16, device="cuda")
    moe.moe_dispatch(s, idx, offsets, row_token, pair_row, d["u"], x_perm, ws)
    p1, p2 = moe.pack_weights(d["w1"]), moe.pack_weights(d["w2"])
    for x, rt in ((x_perm, None), (d["u"], row_token)):
        y = torch.empty((R, w.H), dtype=torch.bfloat16, device="cuda")
        yp = torch.full((R, w.H), float("nan"), dtype=torch.bfloat16, device="cuda")
        moe.moe_expert_ffn(s, x, rt, offsets, d["w1"], d["b1"], d["w2"], y, ws)
        moe.moe_expert_ffn_packed(s, x, rt, offsets, p1, d["b1"], p2, yp, ws)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), yp.view(torch.int16)), "gather" if rt is not None else "x_perm"


@pytest.mark.parametrize("name", ["c2", "c4p"])
def test_packed_workloads_bit_identical(torch_cuda, name):
    """Ragged SwiGLU column tiles (I=1408) and 512 experts with Zipf loads (empty groups)."""
    import torch
    case = Case(synth.WORKLOADS[name])
    assert_same_layer(case, packed_case(case), name)
    case.dev.clear()
    gc.collect()
    torch.cuda.empty_cache()


def test_packed_v3_bit_identical(torch_cuda):
    """The V3-style layer at its full size: prefill T=16384 and the decode slice T=128."""
    torch = torch_cuda
    say("[packed] generating the V3-style weights")
    case = Case(synth.WORKLOADS["c3p"])
    pcase = packed_case(case)
    assert_same_layer(case, pcase, "c3p")
    dec = case.with_tokens(128)
    pdec = Case.__new__(Case)
    pdec.w, pdec.inp = dec.w, dec.inp
    pdec.dev = dict(pcase.dev)
    pdec.dev["u"] = dec.dev["u"]
    pdec.extra_flags = pcase.extra_flags
    assert_same_layer(dec, pdec, "c3d")
    for c in (case, pcase, dec, pdec):
        c.dev.clear()
    gc.collect()
    torch.cuda.empty_cache()
