"""GPU parity of the speculative path: verify (outputs of T draft positions,
no state written) and accept (position update, commit once the count reaches
the interval), against the fp64 oracle; plus the method's invariants.

Article ("NVIDIA ReplaySSM: hybrid model SSM decoding with a state buffer"),
section 3: draft inputs are buffered, only positions through the last
accepted token are valid, rejected tokens need no state restore, and
verification creates no intermediate states.
"""
import dataclasses

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


def _spec_setup(rs, w, batch, rounds, layer=0, stream=0):
    T = w.drafts + 1
    A, D = synth.layer_params(w, layer)
    S0 = synth.init_state(w, layer, batch=batch)
    x, Bm, Cm, dt = synth.token_inputs(w, layer, rounds, batch=batch, tokens=T, stream=stream)
    nk = synth.n_keep(w, rounds, batch=batch, stream=stream)
    ls = rs.LayerState(batch, w.heads, w.groups, A, D, interval=w.interval, max_draft=T,
                       in_dtype=x.dtype)
    rs.load_checkpoint(ls, S0.cuda())
    return T, A, D, S0, x, Bm, Cm, dt, nk, ls


def _bt(t):
    """[T, batch, ...] (oracle layout) <-> [batch, T, ...] (call layout)."""
    return t.transpose(0, 1).contiguous()


def test_spec_rounds_match_oracle(rs):
    """120B-class head layout (H=128, G=8) with 4 drafts at a small batch,
    24 rounds (several commits per slot at varying interval lengths)."""
    w = synth.WORKLOADS["spec"]
    batch, R = 5, 24
    T, A, D, S0, x, Bm, Cm, dt, nk, ls = _spec_setup(rs, w, batch, R)
    ref = oracle.spec_run(S0, x, Bm, Cm, dt, A, D, nk.numpy(), w.groups, w.interval)
    nkd = nk.cuda()
    for r in range(R):
        y = rs.verify(ls, _bt(x[r]).cuda(), _bt(Bm[r]).cuda(), _bt(Cm[r]).cuda(), _bt(dt[r]).cuda())
        rs.accept(ls, nkd[r].contiguous(), T)
        assert_close(_bt(y.cpu()), ref["y"][r], f"verify outputs, round {r}")
        pos = ls.pos.cpu().numpy()
        assert np.array_equal(pos, ref["pos"][r]), (r, pos, ref["pos"][r])
        ck = ls.ckpt.cpu()
        for b in np.nonzero(ref["commit"][r])[0]:
            assert_close(ck[b], ref["state"][r][b], f"checkpoint slot {b} after round {r}")
    rs.check_device_errors(ls)
    # flush and compare every slot with the oracle's final state
    rs.commit(ls)
    assert_close(ls.ckpt.cpu(), ref["state"][-1], "flushed final state")


def test_verify_equals_sequential_steps(rs):
    """verify(T) gives the outputs T single-token steps would give."""
    w = dataclasses.replace(synth.WORKLOADS["spec"], heads=16, groups=2)
    batch = 4
    T, A, D, S0, x, Bm, Cm, dt, nk, ls = _spec_setup(rs, w, batch, 3)
    y_spec = []
    for r in range(3):  # pos grows by T each round (all accepted)
        y_spec.append(_bt(rs.verify(ls, _bt(x[r]).cuda(), _bt(Bm[r]).cuda(), _bt(Cm[r]).cuda(),
                                    _bt(dt[r]).cuda()).cpu()))
        rs.accept(ls, torch.full((batch,), T, dtype=torch.int32, device="cuda"), T)
    ls2 = rs.LayerState(batch, w.heads, w.groups, A, D, interval=w.interval, max_draft=T,
                        in_dtype=x.dtype)
    rs.load_checkpoint(ls2, S0.cuda())
    y_step = []
    for r in range(3):
        for t in range(T):
            y_step.append(rs.step(ls2, x[r, t].cuda(), Bm[r, t].cuda(), Cm[r, t].cuda(),
                                  dt[r, t].cuda()).cpu())
    y_spec = torch.cat(y_spec)
    for i in range(3 * T):
        assert_close(y_spec[i], y_step[i].numpy(), f"position {i}")


def test_rejected_drafts_leave_no_trace(rs):
    """Bit-exact: rejected draft contents (random vs NaN / huge) change
    neither later outputs nor checkpoint bytes."""
    w = dataclasses.replace(synth.WORKLOADS["spec"], heads=16, groups=2)
    batch, R = 6, 12
    runs = []
    for poison in (False, True):
        T, A, D, S0, x, Bm, Cm, dt, nk, ls = _spec_setup(rs, w, batch, R, stream=5)
        if poison:
            x, Bm, dt = x.clone(), Bm.clone(), dt.clone()
            for r in range(R):
                for b in range(batch):
                    k = int(nk[r, b])
                    x[r, k:, b] = float("nan")
                    Bm[r, k:, b] = 1e30
                    dt[r, k:, b] = 5.0
        nkd = nk.cuda()
        ys, cks = [], []
        for r in range(R):
            y = rs.verify(ls, _bt(x[r]).cuda(), _bt(Bm[r]).cuda(), _bt(Cm[r]).cuda(), _bt(dt[r]).cuda())
            rs.accept(ls, nkd[r].contiguous(), T)
            ys.append(y.cpu())
            cks.append(ls.ckpt.cpu().clone())
        runs.append((ys, cks, nk))
    (ya, ca, nk), (yb, cb, _) = runs
    for r in range(R):
        for b in range(batch):
            k = int(nk[r, b])
            assert torch.equal(ya[r][b, :k], yb[r][b, :k]), (r, b)
        assert torch.equal(ca[r], cb[r]), r


def test_verify_causality(rs):
    """Output of draft t is bit-identical when drafts after t change."""
    w = dataclasses.replace(synth.WORKLOADS["spec"], heads=8, groups=1)
    batch = 3
    T, A, D, S0, x, Bm, Cm, dt, nk, ls = _spec_setup(rs, w, batch, 1)
    snap = ls.snapshot()
    y1 = rs.verify(ls, _bt(x[0]).cuda(), _bt(Bm[0]).cuda(), _bt(Cm[0]).cuda(), _bt(dt[0]).cuda()).cpu()
    ls.restore(snap)
    x2, B2, C2, d2 = x.clone(), Bm.clone(), Cm.clone(), dt.clone()
    x2[0, 2:] = 7.0
    B2[0, 2:] = -3.0
    C2[0, 2:] = 0.5
    d2[0, 2:] = 0.9
    y2 = rs.verify(ls, _bt(x2[0]).cuda(), _bt(B2[0]).cuda(), _bt(C2[0]).cuda(), _bt(d2[0]).cuda()).cpu()
    assert torch.equal(y1[:, :2], y2[:, :2])
    assert not torch.equal(y1[:, 2:], y2[:, 2:])


def test_verify_writes_no_state(rs):
    w = dataclasses.replace(synth.WORKLOADS["spec"], heads=8, groups=1)
    T, A, D, S0, x, Bm, Cm, dt, nk, ls = _spec_setup(rs, w, 3, 1)
    before = ls.ckpt.clone()
    pos = ls.pos.clone()
    rs.verify(ls, _bt(x[0]).cuda(), _bt(Bm[0]).cuda(), _bt(Cm[0]).cuda(), _bt(dt[0]).cuda())
    torch.cuda.synchronize()
    assert torch.equal(before, ls.ckpt)
    assert torch.equal(pos, ls.pos)


def test_accept_zero_keeps_everything(rs):
    """n_keep = 0 drops the whole round (the sampled token too)."""
    w = dataclasses.replace(synth.WORKLOADS["spec"], heads=8, groups=1)
    batch = 3
    T, A, D, S0, x, Bm, Cm, dt, nk, ls = _spec_setup(rs, w, batch, 2)
    rs.verify(ls, _bt(x[0]).cuda(), _bt(Bm[0]).cuda(), _bt(Cm[0]).cuda(), _bt(dt[0]).cuda())
    rs.accept(ls, torch.zeros(batch, dtype=torch.int32, device="cuda"), T)
    assert ls.pos.cpu().tolist() == [0] * batch
    y = rs.verify(ls, _bt(x[1]).cuda(), _bt(Bm[1]).cuda(), _bt(Cm[1]).cuda(), _bt(dt[1]).cuda()).cpu()
    _, yref = oracle.recurrent(S0, x[1], Bm[1], Cm[1], dt[1], A, D, w.groups)
    assert_close(_bt(y), yref, "outputs after a fully rejected round")


def test_n_keep_out_of_range_is_flagged(rs):
    w = dataclasses.replace(synth.WORKLOADS["spec"], heads=8, groups=1)
    batch = 2
    T, A, D, S0, x, Bm, Cm, dt, nk, ls = _spec_setup(rs, w, batch, 1)
    rs.verify(ls, _bt(x[0]).cuda(), _bt(Bm[0]).cuda(), _bt(Cm[0]).cuda(), _bt(dt[0]).cuda())
    rs.accept(ls, torch.tensor([9, -1], dtype=torch.int32, device="cuda"), T)
    with pytest.raises(rs.ReplaySSMError, match="device"):
        rs.check_device_errors(ls)
    assert ls.pos.cpu().tolist() == [T, 0]


@pytest.mark.parametrize("deferred", [False, True])
def test_spec_rounds_inside_hip_graph(rs, deferred):
    """Four speculative rounds (verify + accept, eager or deferred) captured
    in one HIP graph and replayed three times, with eager work and syncs
    between replays: every replay reproduces eager execution bit for bit
    (outputs, checkpoint, positions).  The path records no memset nodes."""
    w = dataclasses.replace(synth.WORKLOADS["spec"], heads=16, groups=2)
    T, R, batch = w.drafts + 1, 4, 5
    A, D = synth.layer_params(w, 1)
    S0 = synth.init_state(w, 1, batch=batch).cuda()
    x, Bm, Cm, dt = synth.token_inputs(w, 1, R, batch=batch, tokens=T, stream=41)
    nk = synth.n_keep(w, R, batch=batch, stream=41).cuda()
    ins = [tuple(_bt(t[r]).cuda() for t in (x, Bm, Cm, dt)) for r in range(R)]
    acc = rs.accept_deferred if deferred else rs.accept
    kw = dict(interval=w.interval, max_draft=T, in_dtype=x.dtype, deferred_commit=deferred)

    def rounds(ls, ys):
        for r in range(R):
            rs.verify(ls, *ins[r], y=ys[r])
            acc(ls, nk[r].contiguous(), T)

    ref = rs.LayerState(batch, w.heads, w.groups, A, D, **kw)
    rs.load_checkpoint(ref, S0)
    eager = []
    for _ in range(3):
        ys = [torch.empty(batch, T, w.heads, 64, device="cuda") for _ in range(R)]
        rounds(ref, ys)
        eager.append(([y.clone() for y in ys], ref.ckpt.clone(), ref.pos.clone()))
    ls = rs.LayerState(batch, w.heads, w.groups, A, D, **kw)
    rs.load_checkpoint(ls, S0)
    ys = [torch.empty(batch, T, w.heads, 64, device="cuda") for _ in range(R)]
    snap = ls.snapshot()
    g = torch.cuda.CUDAGraph()
    s2 = torch.cuda.Stream()
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s2):
        with torch.cuda.graph(g, stream=s2):
            rounds(ls, ys)
    torch.cuda.current_stream().wait_stream(s2)
    torch.cuda.synchronize()
    ls.restore(snap)
    ls.work.zero_()
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        for r in range(R):
            assert torch.equal(ys[r], eager[i][0][r]), (i, r)
        assert torch.equal(ls.ckpt, eager[i][1]) and torch.equal(ls.pos, eager[i][2]), i
        _ = (ls.ckpt * 2.0).sum().item()   # unrelated eager work between replays
    rs.check_device_errors(ls)
