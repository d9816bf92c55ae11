"""GPU parity when the activations span more than 2 GiB: T=152000 tokens of H=7168 bf16
(2.18 GB), 8 routed experts top-2 + 1 shared, I=256, sigmoid + selection bias.

The projections that read the activations (routed and shared up) cannot use 32-bit buffer
offsets there and run on the 128 x 512 kernel with 64-bit addressing and direct-to-LDS loads;
the down projections (the shared one with the fused combine) read the 156 MB / 78 MB hidden
activations and stay on the buffer-load kernel.  Routing is checked on every token; the layer
output on every 16th token, extended so that every 128-row m-tile of the routed segments holds a
checked row.  With the routed banks and the shared gate/up bank packed (fragment order), the routed
and the shared up projections take the packed kernel's 64-bit-address variants (grouped and dense);
the output must be bit-identical to the unpacked layer's.
"""
import gc

import numpy as np
import pytest

import synth
from parity_util import Case, layer_parity, say, strided_tokens

pytestmark = pytest.mark.gpu


def test_activations_beyond_2gib():
    import torch
    assert torch.cuda.is_available()
    w = synth.Workload("big_u", "T=152000 H=7168 bf16 activations (2.18 GB), 8 routed top-2 + 1 shared, I=256",
                       152000, 7168, 8, 2, 1, 256, synth.GATE_SIGMOID_BIAS_NORM, synth.ACT_SWIGLU, synth.DT_BF16,
                       bias_var=0.01)
    assert w.T * w.H * 2 > 2 ** 31
    say("[large] generating %.2f GB of activations" % (w.T * w.H * 2 / 1e9))
    case = Case(w)
    try:
        _, (out, idx, _) = layer_parity(case, tokens=strided_tokens(w.T, 16), route_all=True, label="big_u",
                                        cover_tiles=True)
        import fine_grained_shared_amd as moe
        pcase = Case.__new__(Case)
        pcase.w, pcase.inp = case.w, case.inp
        pcase.dev = dict(case.dev)
        pcase.dev["w1"] = moe.pack_weights(case.dev["w1"])
        pcase.dev["w2"] = moe.pack_weights(case.dev["w2"])
        pcase.dev["w1_sh"] = moe.pack_weights(case.dev["w1_sh"])
        pcase.extra_flags = moe.MOE_FLAG_PACKED_WEIGHTS | moe.MOE_FLAG_PACKED_SHARED_UP
        pout, pidx, _ = pcase.forward()
        torch.cuda.synchronize()
        assert torch.equal(idx, pidx)
        assert torch.equal(out.view(torch.int16), pout.view(torch.int16)), "packed layer differs"
        say("[large] packed routed banks and shared up bank: bit-identical")
        pcase.dev.clear()
    finally:
        case.dev.clear()
        case.inp.clear()
        gc.collect()
        torch.cuda.empty_cache()
