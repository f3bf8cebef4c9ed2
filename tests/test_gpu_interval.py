"""GPU parity of the decode step across interval lengths (the checkpoint is
rewritten every L tokens; article section 2 fixes L = 16, other lengths
trade the per-interval write against buffer reads of about L/2 entries).

L = 1 reduces replay to the conventional recurrence (every step commits);
L up to 64 exercises the long-interval kernels (B entries staged in LDS on
commit steps).  Both step kernels: 3 slots run the per-head row-split
kernel, 300 slots the head-tile kernel (oracle on sampled slots).  Bar:
2e-5 relative per element for every output and every checkpoint.
"""
import dataclasses

import pytest
import torch

import oracle
import synth
from helpers import assert_close, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rs():
    need_gpu()
    import state_space_recurrence_amd as rs
    rs.lib()
    return rs


@pytest.mark.parametrize("batch", [3, 300])
@pytest.mark.parametrize("L", [1, 4, 8, 24, 32, 64])
def test_interval_length(rs, L, batch):
    w = dataclasses.replace(synth.WORKLOADS["tiny"], interval=L)
    steps = 2 * L + 3
    A, D = synth.layer_params(w, 3)
    S0 = synth.init_state(w, 3, batch=batch)
    x, Bm, Cm, dt = synth.token_inputs(w, 3, steps, batch=batch, stream=11)
    ls = rs.LayerState(batch, w.heads, w.groups, A, D, interval=L, in_dtype=x.dtype)
    rs.load_checkpoint(ls, S0.cuda())
    sl = [0, batch // 2, batch - 1]
    ys, cks = [], []
    for t in range(steps):
        ys.append(rs.step(ls, x[t].cuda(), Bm[t].cuda(), Cm[t].cuda(), dt[t].cuda()).cpu()[sl])
        if (t + 1) % L == 0:
            cks.append(ls.ckpt.cpu()[sl].clone())
    torch.cuda.synchronize()
    rs.check_device_errors(ls)
    y_ref, ck_ref = oracle.decode_run(S0[sl], x[:, sl], Bm[:, sl], Cm[:, sl], dt[:, sl], A, D, w.groups, L)
    for t in range(steps):
        assert_close(ys[t], y_ref[t], f"y step {t} (L={L})")
    assert len(cks) == len(ck_ref) == steps // L
    for i, (c, r) in enumerate(zip(cks, ck_ref)):
        assert_close(c, r, f"checkpoint after interval {i} (L={L})")
    assert ls.pos.cpu().tolist() == [3 % L] * batch
    assert ls.intv.cpu().tolist() == [steps // L] * batch


def test_long_interval_bf16_head_layout(rs):
    """4B-class heads (H=96, G=8, bf16 inputs) at L=32: workgroups of 4
    heads, commit with B staged in LDS."""
    w = dataclasses.replace(synth.WORKLOADS["4b"], interval=32)
    batch, steps = 6, 2 * 32 + 5
    A, D = synth.layer_params(w, 0)
    S0 = synth.init_state(w, 0, batch=batch)
    x, Bm, Cm, dt = synth.token_inputs(w, 0, steps, batch=batch, stream=12)
    ls = rs.LayerState(batch, w.heads, w.groups, A, D, interval=32, in_dtype=x.dtype)
    rs.load_checkpoint(ls, S0.cuda())
    ys = [rs.step(ls, x[t].cuda(), Bm[t].cuda(), Cm[t].cuda(), dt[t].cuda()).cpu() for t in range(steps)]
    y_ref, ck_ref = oracle.decode_run(S0, x, Bm, Cm, dt, A, D, w.groups, 32)
    for t in range(steps):
        assert_close(ys[t], y_ref[t], f"y step {t}")
    rs.commit(ls)   # flush the 5-token tail
    S_end, _ = oracle.recurrent(S0, x, Bm, Cm, dt, A, D, w.groups)
    assert_close(ls.ckpt.cpu(), S_end, "flushed state")


@pytest.mark.parametrize("L", [32, 64])
def test_long_interval_bf16_head_tile(rs, L):
    """The head-tile step instances the interval sweep times (bf16 inputs,
    4B-class heads): 24 slots x 24 workgroups of 4 heads = 576 workgroups,
    above the row-split threshold, so replay_step_kernel<bf16, 32/64> runs.
    Every output of three slots and their checkpoint after every interval
    against the oracle."""
    w = dataclasses.replace(synth.WORKLOADS["4b"], interval=L)
    batch, steps = 24, 2 * L + 5
    A, D = synth.layer_params(w, 2)
    S0 = synth.init_state(w, 2, batch=batch)
    x, Bm, Cm, dt = synth.token_inputs(w, 2, steps, batch=batch, stream=13)
    ls = rs.LayerState(batch, w.heads, w.groups, A, D, interval=L, in_dtype=x.dtype)
    rs.load_checkpoint(ls, S0.cuda())
    sl = [0, 11, batch - 1]
    xs, Bs, Cs, ds = (t.cuda() for t in (x, Bm, Cm, dt))
    ys, cks = [], []
    for t in range(steps):
        ys.append(rs.step(ls, xs[t], Bs[t], Cs[t], ds[t])[sl].cpu())
        if (t + 1) % L == 0:
            cks.append(ls.ckpt[sl].cpu())
    rs.check_device_errors(ls)
    y_ref, ck_ref = oracle.decode_run(S0[sl], x[:, sl], Bm[:, sl], Cm[:, sl], dt[:, sl], A, D, w.groups, L)
    for t in range(steps):
        assert_close(ys[t], y_ref[t], f"y step {t} (L={L}, head tile)")
    assert len(cks) == len(ck_ref) == 2
    for i, (c, r) in enumerate(zip(cks, ck_ref)):
        assert_close(c, r, f"checkpoint after interval {i} (L={L}, head tile)")
    assert ls.pos.cpu().tolist() == [5] * batch
