"""GPU parity of the standard decode path: replay step with fused interval
commit, standalone commit and checkpoint load, against the fp64 oracle.

Article ("NVIDIA ReplaySSM: hybrid model SSM decoding with a state buffer"),
section 1: outputs replayed from the interval checkpoint plus the input buffer
match the conventional recurrence within floating-point error; the
checkpoint is written once per interval.  Bar: |dy| <= 2e-5 * max(1, |y|) per
element at every step, and the same for the checkpoint after each commit.
"""
import numpy as np
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


def _run_decode(rs, w, layer, steps, batch=None, heads=None, groups=None):
    if heads is not None:
        import dataclasses
        w = dataclasses.replace(w, heads=heads, groups=groups)
    A, D = synth.layer_params(w, layer)
    S0 = synth.init_state(w, layer, batch=batch)
    x, Bm, Cm, dt = synth.token_inputs(w, layer, steps, batch=batch)
    b = S0.shape[0]
    ls = rs.LayerState(b, w.heads, w.groups, A, D, interval=w.interval,
                       in_dtype=x.dtype, device="cuda")
    rs.load_checkpoint(ls, S0.cuda())
    xs, Bs, Cs, ds = (t.cuda() for t in (x, Bm, Cm, dt))
    ys, cks = [], []
    for t in range(steps):
        ys.append(rs.step(ls, xs[t], Bs[t], Cs[t], ds[t]).cpu())
        if (t + 1) % w.interval == 0:
            cks.append(ls.ckpt.cpu().clone())
    torch.cuda.synchronize()
    rs.check_device_errors(ls)
    y_ref, ck_ref = oracle.decode_run(S0, x, Bm, Cm, dt, A, D, w.groups, w.interval)
    return ls, torch.stack(ys), y_ref, cks, ck_ref


def test_tiny_replay_matches_oracle(rs):
    """fp32 inputs, B=4, H=8, G=1, L=16, 64 steps (4 fused commits)."""
    w = synth.WORKLOADS["tiny"]
    ls, y, y_ref, cks, ck_ref = _run_decode(rs, w, 0, w.steps)
    assert len(cks) == 4
    for t in range(w.steps):
        assert_close(y[t], y_ref[t], f"y step {t}")
    for i, (c, r) in enumerate(zip(cks, ck_ref)):
        assert_close(c, r, f"checkpoint after interval {i}")
    assert ls.pos.cpu().tolist() == [0] * 4
    assert ls.intv.cpu().tolist() == [4] * 4
    assert ls.work.cpu().tolist() == [0] * 5


def test_4b_shape_replay_bf16(rs):
    """bf16 inputs on the 4B-class head layout (H=96, G=8) at a small batch,
    3 intervals + a ragged tail of 5 tokens."""
    w = synth.WORKLOADS["4b"]
    steps = 3 * w.interval + 5
    ls, y, y_ref, cks, ck_ref = _run_decode(rs, w, 1, steps, batch=6)
    for t in range(steps):
        assert_close(y[t], y_ref[t], f"y step {t}")
    for i, (c, r) in enumerate(zip(cks, ck_ref)):
        assert_close(c, r, f"checkpoint after interval {i}")
    assert ls.pos.cpu().tolist() == [5] * 6


@pytest.mark.parametrize("heads,groups", [(6, 3), (3, 3), (10, 1), (16, 2)])
def test_head_group_layouts(rs, heads, groups):
    """Workgroups of 4, 2 and 1 heads (heads per group 2, 1, 10, 8)."""
    w = synth.WORKLOADS["tiny"]
    ls, y, y_ref, cks, ck_ref = _run_decode(rs, w, 2, 20, batch=3, heads=heads, groups=groups)
    for t in range(20):
        assert_close(y[t], y_ref[t], f"y step {t}")
    assert_close(cks[0], ck_ref[0], "checkpoint")


def test_flush_commit_and_empty_commit(rs):
    """replayssm_commit folds a partial buffer into the checkpoint (the state
    after the buffered tokens) and is the identity on an empty buffer."""
    w = synth.WORKLOADS["tiny"]
    A, D = synth.layer_params(w, 0)
    S0 = synth.init_state(w, 0)
    x, Bm, Cm, dt = synth.token_inputs(w, 0, 40, stream=7)
    ls = rs.LayerState(w.batch, w.heads, w.groups, A, D, in_dtype=x.dtype)
    rs.load_checkpoint(ls, S0.cuda())
    xs, Bs, Cs, ds = (t.cuda() for t in (x, Bm, Cm, dt))
    for t in range(7):
        rs.step(ls, xs[t], Bs[t], Cs[t], ds[t])
    rs.commit(ls)
    S7, _ = oracle.recurrent(S0, x[:7], Bm[:7], Cm[:7], dt[:7], A, D, w.groups)
    assert_close(ls.ckpt.cpu(), S7, "flushed checkpoint")
    assert ls.pos.cpu().tolist() == [0] * w.batch
    assert ls.intv.cpu().tolist() == [1] * w.batch
    before = ls.ckpt.clone()
    rs.commit(ls)   # empty buffer: nothing changes
    assert torch.equal(ls.ckpt, before)
    assert ls.intv.cpu().tolist() == [1] * w.batch
    # continue decoding after an early commit: outputs still follow the recurrence
    ys = [rs.step(ls, xs[t], Bs[t], Cs[t], ds[t]).cpu() for t in range(7, 40)]
    _, y_ref = oracle.recurrent(S0, x, Bm, Cm, dt, A, D, w.groups)
    for i, t in enumerate(range(7, 40)):
        assert_close(ys[i], y_ref[t], f"y step {t} after early commit")


def test_snapshot_restore_and_determinism(rs):
    w = synth.WORKLOADS["tiny"]
    A, D = synth.layer_params(w, 0)
    S0 = synth.init_state(w, 0).cuda()
    x, Bm, Cm, dt = (t.cuda() for t in synth.token_inputs(w, 0, 30, stream=3))
    ls = rs.LayerState(w.batch, w.heads, w.groups, A, D, in_dtype=x.dtype)
    rs.load_checkpoint(ls, S0)
    for t in range(9):
        rs.step(ls, x[t], Bm[t], Cm[t], dt[t])
    snap = ls.snapshot()
    ya = [rs.step(ls, x[t], Bm[t], Cm[t], dt[t]).clone() for t in range(9, 30)]
    cka = ls.ckpt.clone()
    ls.restore(snap)
    yb = [rs.step(ls, x[t], Bm[t], Cm[t], dt[t]).clone() for t in range(9, 30)]
    for a, b in zip(ya, yb):
        assert torch.equal(a, b)
    assert torch.equal(cka, ls.ckpt)


def test_empty_batch_is_noop(rs):
    w = synth.WORKLOADS["tiny"]
    A, D = synth.layer_params(w, 0)
    ls = rs.LayerState(0, w.heads, w.groups, A, D, in_dtype=torch.float32)
    e = torch.empty(0, w.heads, 64, device="cuda")
    Bm = torch.empty(0, w.groups, 128, device="cuda")
    dt = torch.empty(0, w.heads, device="cuda")
    y = rs.step(ls, e, Bm, Bm, dt)
    rs.commit(ls)
    torch.cuda.synchronize()
    assert y.shape == (0, w.heads, 64)


def test_position_out_of_range_is_flagged(rs):
    """A corrupted position is clamped and reported, never used to index out
    of the buffer."""
    w = synth.WORKLOADS["tiny"]
    A, D = synth.layer_params(w, 0)
    x, Bm, Cm, dt = (t.cuda() for t in synth.token_inputs(w, 0, 1))
    ls = rs.LayerState(w.batch, w.heads, w.groups, A, D, in_dtype=x.dtype)
    ls.pos.fill_(99)
    rs.step(ls, x[0], Bm[0], Cm[0], dt[0])
    with pytest.raises(rs.ReplaySSMError, match="device"):
        rs.check_device_errors(ls)
    rs.check_device_errors(ls)   # sticky flag was cleared by the read


def test_row_split_and_tile_kernels_agree_bitwise(rs):
    """Small batches run the per-head row-split step kernel, large ones the
    head-tile kernel; both do the same per-row arithmetic, so the slots they
    share give bit-identical outputs and checkpoints (and match the oracle)."""
    w = synth.WORKLOADS["tiny"]
    big, small, steps = 300, 3, 2 * w.interval + 3     # 600 vs 6 workgroups
    A, D = synth.layer_params(w, 0)
    S0 = synth.init_state(w, 0, batch=big)
    x, Bm, Cm, dt = synth.token_inputs(w, 0, steps, batch=big)
    outs = {}
    for b in (big, small):
        ls = rs.LayerState(b, w.heads, w.groups, A, D, in_dtype=x.dtype)
        rs.load_checkpoint(ls, S0[:b].contiguous().cuda())
        ys = [rs.step(ls, x[t, :b].contiguous().cuda(), Bm[t, :b].contiguous().cuda(),
                      Cm[t, :b].contiguous().cuda(), dt[t, :b].contiguous().cuda()).cpu() for t in range(steps)]
        outs[b] = (torch.stack(ys), ls.ckpt.cpu())
    assert torch.equal(outs[big][0][:, :small], outs[small][0])
    assert torch.equal(outs[big][1][:small], outs[small][1])
    sl = [0, 151, big - 1]
    y_ref, cks = oracle.decode_run(S0[sl], x[:, sl], Bm[:, sl], Cm[:, sl], dt[:, sl], A, D, w.groups, w.interval)
    for t in range(steps):
        assert_close(outs[big][0][t, sl], y_ref[t], f"y step {t} (head-tile kernel)")
    assert_close(outs[big][1][sl], cks[-1], "checkpoint (head-tile kernel)")


def test_step_inside_hip_graph(rs):
    """One interval of steps captured in a HIP graph and replayed three
    times, with eager work and syncs between replays: every replay matches
    eager execution of the same sequence bit for bit."""
    w = synth.WORKLOADS["tiny"]
    A, D = synth.layer_params(w, 0)
    S0 = synth.init_state(w, 0).cuda()
    x, Bm, Cm, dt = (t.cuda() for t in synth.token_inputs(w, 0, w.interval, stream=9))
    L = w.interval
    # eager reference: the same L inputs three times
    ref = rs.LayerState(w.batch, w.heads, w.groups, A, D, in_dtype=x.dtype)
    rs.load_checkpoint(ref, S0)
    eager = [[rs.step(ref, x[t], Bm[t], Cm[t], dt[t]).clone() for t in range(L)] for _ in range(3)]
    # graph
    ls = rs.LayerState(w.batch, w.heads, w.groups, A, D, in_dtype=x.dtype)
    rs.load_checkpoint(ls, S0)
    ys = [torch.empty(w.batch, w.heads, 64, device="cuda") for _ in range(L)]
    snap = ls.snapshot()
    g = torch.cuda.CUDAGraph()
    s2 = torch.cuda.Stream()
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s2):
        with torch.cuda.graph(g, stream=s2):
            for t in range(L):
                rs.step(ls, x[t], Bm[t], Cm[t], dt[t], y=ys[t])
    torch.cuda.current_stream().wait_stream(s2)
    torch.cuda.synchronize()
    ls.restore(snap)           # capture does not execute; start from the loaded state
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        for t in range(L):
            assert torch.equal(ys[t], eager[r][t]), (r, t)
        _ = (ls.ckpt * 1.0).sum().item()   # unrelated eager work between replays
    assert torch.equal(ls.ckpt, ref.ckpt)
    assert ls.pos.cpu().tolist() == ref.pos.cpu().tolist()
