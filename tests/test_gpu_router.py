"""GPU: the router's logits are summed in one canonical order by two different kernels - the tiled
MFMA GEMM for batches of 1024 tokens or more (expert counts a multiple of 64) and a wave-per-block
kernel for smaller batches - so a token's routing must not depend on the batch it arrives in: topk_idx
and topk_w must be identical bit for bit whether a token is routed in a batch of 3000 or of a few
hundred.  The cases cover every gating mode, group-limited routing, the masking probe, H with two
reduction groups (H >= 4096) and with one, expert counts from 48 to 640 (the GEMM's 128- and 512-wide
column tiles), ragged token tiles, and exact ties; each is also checked against the oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from parity_util import check_routing, gpu_shape, say, to_dev
from synth import ACT_SWIGLU, DT_BF16, GATE_SIGMOID_BIAS_NORM, GATE_SOFTMAX, GATE_SOFTMAX_RENORM, Workload

pytestmark = pytest.mark.gpu


def W(name, H, N, K, gating, T=3013, **kw):
    return Workload(name, name, T, H, N, K, 0, 64, gating, ACT_SWIGLU, DT_BF16,
                    bias_var=0.01 if gating == GATE_SIGMOID_BIAS_NORM else 0.0, **kw)


# T is chosen so that the one-batch call takes the tiled GEMM: at least 256 of its 128 x 128 output tiles
# (ceil(T / 128) x ceil(N / 128) x reduction groups); the batches of 500 take the small-batch kernel.
CASES = {
    "sigmoid_bias_h2048_n512": W("sigmoid_bias_h2048_n512", 2048, 512, 10, GATE_SIGMOID_BIAS_NORM, T=8200),
    "softmax_h128_n128": W("softmax_h128_n128", 128, 128, 2, GATE_SOFTMAX, T=32800),
    "renorm_h576_n64": W("renorm_h576_n64", 576, 64, 8, GATE_SOFTMAX_RENORM, T=32800),
    "group_limited_h256_n256": W("group_limited_h256_n256", 256, 256, 8, GATE_SIGMOID_BIAS_NORM, T=16400,
                                 n_group=8, topk_group=4),
    "mask_probe_h320_n320": W("mask_probe_h320_n320", 320, 320, 4, GATE_SOFTMAX, T=11100, mask_top_r=2),
    "sigmoid_h192_n640": W("sigmoid_h192_n640", 192, 640, 12, GATE_SIGMOID_BIAS_NORM, T=6600),
    "softmax_h256_n48": W("softmax_h256_n48", 256, 48, 6, GATE_SOFTMAX),   # small-batch kernel only
    "sigmoid_h4096_n256": W("sigmoid_h4096_n256", 4096, 256, 8, GATE_SIGMOID_BIAS_NORM, T=8200),   # two groups
}


def gemm_path(w):
    groups = 2 if w.H >= 4096 and w.H % 128 == 0 else 1
    return w.T >= 1024 and w.N_r % 64 == 0 and -(-w.T // 128) * -(-w.N_r // 128) * groups >= 256


def route(torch, moe, w, u, cen, bias, T=None):
    T = w.T if T is None else T
    s = gpu_shape(w, T=T)
    idx = torch.empty((T, w.K_r), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, w.K_r), dtype=torch.float32, device="cuda")
    moe.moe_route(s, u, cen, bias, idx, wts, moe.workspace(s))
    return idx, wts


@pytest.mark.parametrize("name", list(CASES))
def test_routing_does_not_depend_on_the_batch(name):
    import torch
    import fine_grained_shared_amd as moe
    assert torch.cuda.is_available()
    w = CASES[name]
    assert gemm_path(w) == (name != "softmax_h256_n48")
    inp = synth.make_inputs(w, weights=False)
    u, cen, bias = to_dev(inp["u"]), to_dev(inp["centroids"]), to_dev(inp["bias"])
    idx, wts = route(torch, moe, w, u, cen, bias)               # one batch (tiled GEMM logits)
    parts = []
    for t0 in range(0, w.T, 500):                               # batches of <= 500 (the small-batch kernel)
        n = min(500, w.T - t0)
        parts.append(route(torch, moe, w, u[t0:t0 + n].contiguous(), cen, bias, T=n))
    torch.cuda.synchronize()
    idx_b = torch.cat([p[0] for p in parts])
    wts_b = torch.cat([p[1] for p in parts])
    assert torch.equal(idx, idx_b), "selection depends on the batch"
    assert torch.equal(wts.view(torch.int32), wts_b.view(torch.int32)), "gate weights depend on the batch"
    # and against the oracle on a strided sample (every token of the last, ragged tile included)
    tok = np.unique(np.concatenate([np.arange(0, w.T, 17), np.arange(w.T - 40, w.T)])).astype(np.int64)
    sel_o, g_o, gap = oracle.route(oracle.shape_of(w), inp["u"], inp["centroids"], inp["bias"], tokens=tok)
    ties = check_routing(idx.cpu().numpy()[tok], wts.cpu().numpy().astype(np.float64)[tok], sel_o, g_o, gap, name)
    say("[router] %s: T=%d in one batch == in batches of 500, bit for bit; oracle on %d tokens, %d near ties" % (
        name, w.T, len(tok), ties))


@pytest.mark.parametrize("T", [200, 32800])
def test_exact_ties_go_to_the_lower_index_on_both_logit_kernels(T):
    """Duplicated centroids tie exactly on both logit kernels: the lower index comes first."""
    import torch
    import fine_grained_shared_amd as moe
    w = W("ties", 128, 128, 2, GATE_SOFTMAX, T=T)
    inp = synth.make_inputs(w, weights=False)
    cen, u = inp["centroids"].copy(), inp["u"].copy()
    cen[70] = cen[5]
    toks = np.arange(5, w.T, 17)
    u[toks] = synth.f32_to_bf16_bits(16.0 * synth.bf16_bits_to_f32(cen[5]))
    idx, wts = route(torch, moe, w, to_dev(u), to_dev(cen), None)
    torch.cuda.synchronize()
    got, g = idx.cpu().numpy(), wts.cpu().numpy()
    assert (got[toks] == [5, 70]).all() and (g[toks, 0] == g[toks, 1]).all()
