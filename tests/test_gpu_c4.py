"""GPU parity at the high-sparsity shape (H=2048, 1 shared + 512 routed, top-10, I=512, Zipf(1.1)
centroid norms, sigmoid+bias): prefill T=32768 and the T=64 decode slice."""
import gc

import numpy as np
import pytest

import synth
from parity_util import Case, layer_parity, sample_tokens, say

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
    stats, (out, idx, wts) = layer_parity(c4, tokens=sample_tokens(w.T, 96), route_all=True, label="c4p")
    c = np.bincount(idx.cpu().numpy().reshape(-1), minlength=w.N_r)
    nz = c[c > 0]
    say("[c4] near ties %d, empty %d, max/mean %.1f, max/min nonzero %.1f" % (
        stats["near_ties"], (c == 0).sum(), c.max() / c.mean(), nz.max() / nz.min()))
    assert c.max() / c.mean() > 20.0   # loads span more than 20x: overfull and empty groups


def test_c4_decode(c4):
    case = c4.with_tokens(64)
    case.w = case.w.with_(name="c4d")
    layer_parity(case, route_all=True, label="c4d")
