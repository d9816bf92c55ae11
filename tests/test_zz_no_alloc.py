"""moe_layer_forward_noalloc (scratch in the library's static device array) against moe_layer_forward
(scratch in a caller workspace): the same kernels, so the outputs and the routing must be identical bit
for bit.  Two calls in a row, the second with fewer tokens (the array keeps the first call's contents),
in bf16 (packed and [out, in] banks) and fp32; a shape beyond the array is refused before any launch."""
import numpy as np
import pytest

import synth
from parity_util import Case, gpu_shape, say
from synth import ACT_RELU_BIAS, ACT_SWIGLU, DT_BF16, DT_F32, GATE_SIGMOID_BIAS_NORM, GATE_SOFTMAX, Workload

pytestmark = pytest.mark.gpu

LAYERS = {
    # ~150 rows per expert: the prefill kernels; the second call (T=90) takes the decode-shaped ones
    "bf16": Workload("noalloc_bf16", "bf16 SwiGLU sigmoid+bias layer", 600, 512, 16, 4, 1, 256,
                     GATE_SIGMOID_BIAS_NORM, ACT_SWIGLU, DT_BF16, bias_var=0.01),
    "f32": Workload("noalloc_f32", "fp32 ReLU softmax layer", 130, 128, 16, 4, 1, 64, GATE_SOFTMAX, ACT_RELU_BIAS,
                    DT_F32),
}


def run_both(case, T, flags, d):
    import torch
    import fine_grained_shared_amd as moe
    s = gpu_shape(case.w, T=T)
    u = d["u"][:T].contiguous()
    tdt = moe.torch_dtype(s)
    outs = []
    for noalloc in (False, True):
        out = torch.full((T, case.w.H), 7.0, dtype=tdt, device="cuda")
        idx = torch.full((T, case.w.K_r), -1, dtype=torch.int32, device="cuda")
        wts = torch.full((T, case.w.K_r), -1.0, dtype=torch.float32, device="cuda")
        if noalloc:
            moe.moe_layer_forward_noalloc(s, u, d["centroids"], d["bias"], d["w1"], d["b1"], d["w2"], d["w1_sh"],
                                          d["b1_sh"], d["w2_sh"], flags, out, idx, wts)
        else:
            moe.moe_layer_forward(s, u, d["centroids"], d["bias"], d["w1"], d["b1"], d["w2"], d["w1_sh"], d["b1_sh"],
                                  d["w2_sh"], flags, out, idx, wts, moe.workspace(s))
        outs.append((out, idx, wts))
    torch.cuda.synchronize()
    (o0, i0, w0), (o1, i1, w1) = outs
    assert torch.equal(i0, i1) and torch.equal(w0.view(torch.int32), w1.view(torch.int32))
    bits = torch.int16 if tdt == torch.bfloat16 else torch.int32
    assert torch.equal(o0.view(bits), o1.view(bits)), "noalloc output differs (T=%d)" % T
    return o1


@pytest.mark.parametrize("name,packed", [("bf16", False), ("bf16", True), ("f32", False)])
def test_noalloc_matches_workspace_entry_point(name, packed):
    import torch
    import fine_grained_shared_amd as moe
    assert torch.cuda.is_available()
    case = Case(LAYERS[name])
    d = dict(case.dev)
    flags = 0
    if packed:
        for k in ("w1", "w2", "w1_sh"):
            d[k] = moe.pack_weights(d[k])
        flags = moe.MOE_FLAG_PACKED_WEIGHTS | moe.MOE_FLAG_PACKED_SHARED_UP
    T0 = case.w.T
    for T in (T0, 90 if name == "bf16" else 37):
        assert moe.moe_workspace_size(gpu_shape(case.w, T=T)) <= moe.moe_noalloc_scratch_bytes()
        run_both(case, T, flags, d)
        say("[noalloc] %s packed=%s T=%d: bit-identical to moe_layer_forward" % (name, packed, T))


def test_noalloc_refuses_shapes_beyond_its_scratch():
    import torch
    import fine_grained_shared_amd as moe
    s = moe.make_shape(16384, 7168, 256, 8, 1, 2048, synth.GATE_SIGMOID_BIAS_NORM, synth.ACT_SWIGLU, synth.DT_BF16)
    assert moe.moe_workspace_size(s) > moe.moe_noalloc_scratch_bytes()
    out = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_forward_noalloc(s, out, out, None, out, None, out, out, None, out, 0, out, None, None)
    assert e.value.status == moe.MOE_ERR_SCRATCH
