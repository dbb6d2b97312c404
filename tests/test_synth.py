"""Seeded input generators: shapes, reproducibility and the workload
structure (load skew, outlier channels).  No GPU."""
import numpy as np
import pytest
import torch

import synth


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_routing_structure(name):
    wl = synth.WORKLOADS[name]
    ids, w = synth.routing(wl)
    assert ids.dtype == np.int32 and ids.shape == (wl.M,)
    assert w.dtype == np.float32 and w.shape == (wl.M,)
    assert ((ids >= 0) & (ids < wl.E)).all()
    per_tok = ids.reshape(wl.T, wl.k)
    assert all(len(set(r)) == wl.k for r in per_tok.tolist())
    assert np.allclose(w.reshape(wl.T, wl.k).sum(1), 1.0, atol=1e-6)
    ids2, w2 = synth.routing(wl)
    assert np.array_equal(ids, ids2) and np.array_equal(w, w2)
    st = synth.load_stats(ids, wl.E)
    if wl.bias == "zipf":
        assert st["zero"] > 0 and st["over_1000"] > 0
        assert abs(st["slope"] + synth.ZIPF_S) < 0.05
    if wl.bias == "gauss":
        assert st["zero"] > 0        # decode: many experts without rows


def test_tokens_outliers():
    wl = synth.WORKLOADS["decode-30b"]
    x = synth.tokens(wl)
    assert x.dtype == torch.bfloat16 and x.shape == (wl.T, wl.K_in)
    x2 = synth.tokens(wl, T=4096)
    big = (x2.float().abs().amax(0) > 12).sum().item()
    assert big == round(0.01 * wl.K_in)
    assert torch.equal(synth.tokens(wl), x)
    assert (synth.tokens(synth.WORKLOADS["tiny"]).float().abs().amax() < 8)


def test_dense_expert():
    wl = synth.WORKLOADS["tiny"]
    a = synth.dense_expert(wl, 0, 3)
    assert a.shape == (128, 256) and a.dtype == torch.float32
    assert torch.equal(a, synth.dense_expert(wl, 0, 3))
    assert not torch.equal(a, synth.dense_expert(wl, 0, 4))
    assert abs(a.std().item() - 0.02) < 0.002
