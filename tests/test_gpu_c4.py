"""GPU parity at the high-sparsity shape (H=2048, 1 shared + 512 routed, top-10, I=512, Zipf(1.1)
centroid norms, sigmoid+bias): prefill T=32768 (routing on every token, outputs on every 8th token,
extended so that every 128-row m-tile of every routed expert segment holds a checked row) and the T=64
decode slice (every token)."""
import gc

import numpy as np
import pytest

import synth
from parity_util import Case, layer_parity, say, strided_tokens

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def c4():
    import torch
    assert torch.cuda.is_available()
    case = Case(synth.WORKLOADS["c4p"])
    yield case
    case.dev.clear()
    case.inp.clear()
    gc.collect()
    torch.cuda.empty_cache()


def test_c4_prefill_skewed_loads(c4):
    w = c4.w
    stats, (out, idx, wts) = layer_parity(c4, tokens=strided_tokens(w.T, 8), route_all=True, label="c4p",
                                          cover_tiles=True)
    say("[c4] checked %d tokens over %d routed m-tiles (%d added)" % (
        stats["tokens_checked"], stats["routed_m_tiles"], stats["tokens_added_for_tiles"]))
    c = np.bincount(idx.cpu().numpy().reshape(-1), minlength=w.N_r)
    nz = c[c > 0]
    say("[c4] near ties %d, empty %d, max/mean %.1f, max/min nonzero %.1f" % (
        stats["near_ties"], (c == 0).sum(), c.max() / c.mean(), nz.max() / nz.min()))
    assert c.max() / c.mean() > 20.0   # loads span more than 20x: overfull and empty groups
    PREFILL["idx"], PREFILL["wts"] = idx[:64].clone(), wts[:64].clone()


PREFILL = {}


def test_c4_decode(c4):
    case = c4.with_tokens(64)
    case.w = case.w.with_(name="c4d")
    _, (out, idx, wts) = layer_parity(case, route_all=True, label="c4d")
    if PREFILL:   # the same routing as in the prefill batch, bit for bit (one canonical logit order)
        import torch
        assert torch.equal(idx, PREFILL["idx"])
        assert torch.equal(wts.view(torch.int32), PREFILL["wts"].view(torch.int32))
