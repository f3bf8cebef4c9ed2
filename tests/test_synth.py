"""The synthetic input recipe: workload shapes, the distributions of the
draws, determinism and the bf16 rounding of the inputs.

The article's models and datasets are not available; these seeded inputs
stand in for them with the workload shapes and settings (batch 256 / 512,
16-token intervals, 4 drafts, fp32 state).  Distribution checks use exact
anchors where the transform fixes one: the median of dt = softplus(z - 2)
with z ~ N(0, 1) is softplus(-2), and its 99th percentile is
softplus(z_0.99 - 2).
"""
import math

import numpy as np
import pytest
import torch

import synth


def test_workload_shapes():
    w = synth.WORKLOADS
    assert (w["tiny"].batch, w["tiny"].layers, w["tiny"].heads, w["tiny"].groups, w["tiny"].steps,
            w["tiny"].in_dtype) == (4, 1, 8, 1, 64, "f32")
    assert (w["4b"].batch, w["4b"].layers, w["4b"].heads, w["4b"].groups, w["4b"].steps,
            w["4b"].in_dtype) == (256, 4, 96, 8, 512, "bf16")
    assert (w["120b"].batch, w["120b"].layers, w["120b"].heads, w["120b"].groups, w["120b"].steps) == \
        (256, 8, 128, 8, 256)
    assert (w["spec"].batch, w["spec"].layers, w["spec"].heads, w["spec"].drafts, w["spec"].rounds,
            w["spec"].max_draft) == (512, 4, 128, 4, 200, 5)
    assert (w["split"].batch, w["split"].layers, w["split"].heads, w["split"].groups) == (256, 4, 96, 8)
    for v in w.values():
        assert (v.head_dim, v.d_state, v.interval) == (64, 128, 16)


def _sample():
    w = synth.WORKLOADS["4b"]
    x, Bm, Cm, dt = synth.token_inputs(w, 0, 4, batch=32)
    return w, x.float(), Bm.float(), Cm.float(), dt.float()


def test_gaussian_inputs():
    _, x, Bm, Cm, _ = _sample()
    for t in (x, Bm, Cm):
        v = t.double().flatten()
        n = v.numel()
        assert abs(float(v.mean())) < 5 / math.sqrt(n)
        assert abs(float(v.std()) - 1.0) < 0.01
        # a quarter of N(0,1) lies beyond +-1.15035
        frac = float((v.abs() > 1.1503494).double().mean())
        assert abs(frac - 0.25) < 0.01


def test_dt_is_softplus_of_shifted_gaussian():
    # ~98k draws: the 99th percentile's standard error is ~0.007
    dt = synth.token_inputs(synth.WORKLOADS["4b"], 0, 16, batch=64)[3].float()
    v = dt.double().flatten().numpy()
    assert (v > 0).all()
    sp = lambda z: math.log1p(math.exp(z))
    assert abs(np.median(v) - sp(-2.0)) < 0.004                 # 0.1269
    assert abs(np.quantile(v, 0.99) - sp(2.3263479 - 2.0)) < 0.03   # 0.870
    assert abs(v.mean() - 0.183) < 0.005


def test_decay_and_skip_parameters():
    w = synth.WORKLOADS["120b"]
    As, Ds = zip(*(synth.layer_params(w, l) for l in range(64)))
    A, D = torch.cat(As).double(), torch.cat(Ds).double()
    assert (A <= -1.0).all() and (A > -16.0).all()
    u = torch.log(-A) / math.log(16.0)          # U[0, 1)
    assert abs(float(u.mean()) - 0.5) < 0.03 and abs(float(u.var()) - 1 / 12) < 0.01
    assert abs(float(D.mean())) < 0.1 and abs(float(D.std()) - 1.0) < 0.06


def test_initial_state_scale():
    S = synth.init_state(synth.WORKLOADS["tiny"], 0).double()
    assert abs(float(S.std()) - 0.1) < 0.002 and abs(float(S.mean())) < 0.002


def test_accepted_lengths():
    w = synth.WORKLOADS["spec"]
    nk = synth.n_keep(w, 64)
    assert nk.shape == (64, w.batch) and nk.dtype == torch.int32
    assert int(nk.min()) == 1 and int(nk.max()) == w.drafts + 1
    counts = torch.bincount(nk.flatten().long(), minlength=w.drafts + 2)[1:].double()
    assert (counts / counts.sum() - 1 / (w.drafts + 1)).abs().max() < 0.02


def test_deterministic_and_distinct_streams():
    w = synth.WORKLOADS["tiny"]
    a = synth.token_inputs(w, 0, 3)
    b = synth.token_inputs(w, 0, 3)
    c = synth.token_inputs(w, 0, 3, stream=1)
    d = synth.token_inputs(w, 1, 3)
    for ta, tb, tc, td in zip(a, b, c, d):
        assert torch.equal(ta, tb)
        assert not torch.equal(ta, tc) and not torch.equal(ta, td)
    assert torch.equal(synth.init_state(w, 0), synth.init_state(w, 0))
    assert not torch.equal(synth.init_state(w, 0), synth.init_state(w, 1))


@pytest.mark.parametrize("name", ["4b", "tiny"])
def test_bf16_inputs_are_one_rounding_of_the_fp32_draw(name):
    w = synth.WORKLOADS[name]
    lo = synth.token_inputs(w, 0, 2, batch=3)
    hi = synth.token_inputs(synth.dataclasses.replace(w, in_dtype="f32"), 0, 2, batch=3)
    for tl, th in zip(lo, hi):
        assert th.dtype == torch.float32
        assert torch.equal(tl, th.to(tl.dtype))    # identity for fp32 workloads, one RNE cast for bf16
