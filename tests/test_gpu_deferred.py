"""GPU parity of the deferred commit on the speculative path.

replayssm_accept_deferred only advances positions; a slot whose accepted
count reaches the interval keeps its entries (up to L + Tmax - 1) until the
next verify, step or flush on it folds them into the checkpoint inside the
pass that reads the checkpoint anyway.  Article ("NVIDIA ReplaySSM: hybrid
model SSM decoding with a state buffer"), section 3: positions through the
last accepted token stay valid and the checkpoint is written once per
interval.  The fold does the per-element arithmetic of the eager commit, so
outputs, checkpoints and positions are bit-identical to the eager accept;
outputs also match the fp64 oracle at 2e-5.
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


def _bt(t):
    """[T, batch, ...] (oracle layout) <-> [batch, T, ...] (call layout)."""
    return t.transpose(0, 1).contiguous()


def _pair(rs, w, batch, T, S0, A, D, dtype):
    """An eager layer and one that declares deferred commits."""
    out = []
    for deferred in (False, True):
        ls = rs.LayerState(batch, w.heads, w.groups, A, D, interval=w.interval, max_draft=T, in_dtype=dtype,
                           deferred_commit=deferred)
        rs.load_checkpoint(ls, S0.cuda())
        out.append(ls)
    return out


def _rounds(rs, le, ld, x, Bm, Cm, dt, nk, T, R, ref=None, check=None):
    """R verify rounds on both states: eager accept on le, deferred on ld."""
    nkd = nk.cuda()
    folded = 0
    for r in range(R):
        args = (_bt(x[r]).cuda(), _bt(Bm[r]).cuda(), _bt(Cm[r]).cuda(), _bt(dt[r]).cuda())
        ye = rs.verify(le, *args)
        held = (ld.pos >= ld.interval).sum().item()
        yd = rs.verify(ld, *args)
        folded += held
        assert torch.equal(ye, yd), f"round {r}: deferred outputs differ from eager"
        assert torch.equal(le.pos, ld.pos) and torch.equal(le.intv, ld.intv), r
        assert torch.equal(le.ckpt, ld.ckpt), f"round {r}: checkpoints differ after the fold"
        if ref is not None:
            assert_close(_bt(ye.cpu()), ref["y"][r], f"verify outputs, round {r}")
        rs.accept(le, nk[r].contiguous().cuda(), T)
        rs.accept_deferred(ld, nkd[r].contiguous(), T)
    return folded


def test_deferred_verify_bit_identical_to_eager(rs):
    """120B-class heads (H=128, G=8), 4 drafts, 24 rounds at a small batch:
    many slots fold inside a verify at varying counts L..L+4."""
    w = synth.WORKLOADS["spec"]
    batch, R, T = 5, 24, w.drafts + 1
    A, D = synth.layer_params(w, 0)
    S0 = synth.init_state(w, 0, batch=batch)
    x, Bm, Cm, dt = synth.token_inputs(w, 0, R, batch=batch, tokens=T)
    nk = synth.n_keep(w, R, batch=batch)
    ref = oracle.spec_run(S0, x, Bm, Cm, dt, A, D, nk.numpy(), w.groups, w.interval)
    le, ld = _pair(rs, w, batch, T, S0, A, D, x.dtype)
    folded = _rounds(rs, le, ld, x, Bm, Cm, dt, nk, T, R, ref=ref)
    assert folded >= batch          # every slot folded at least once inside a verify
    assert (ld.pos.cpu() >= 0).all()
    rs.check_device_errors(le)
    rs.check_device_errors(ld)
    # flush: slots still holding >= L entries fold inside the commit call
    rs.commit(le)
    rs.commit(ld)
    assert torch.equal(le.ckpt, ld.ckpt)
    assert_close(ld.ckpt.cpu(), ref["state"][-1], "flushed final state")


def test_step_after_deferred_accept(rs):
    """A single-token step on slots left at pos >= L replays all pos + 1
    tokens and commits them in the same pass.  Inputs are generated for 300
    slots; the full batch runs the head-tile step kernel and its first 4
    slots (run alone) the per-head row-split kernel, which agree bit for
    bit; both match the oracle at 2e-5, outputs and checkpoints."""
    w = dataclasses.replace(synth.WORKLOADS["tiny"], drafts=2)
    big, small, T, R = 300, 4, 3, 6
    A, D = synth.layer_params(w, 1)
    S0 = synth.init_state(w, 1, batch=big)
    x, Bm, Cm, dt = synth.token_inputs(w, 1, R, batch=big, tokens=T, stream=5)
    nk = torch.full((R, big), T, dtype=torch.int32)
    nk[:, 1::2] = torch.randint(0, T + 1, (R, big // 2), generator=torch.Generator().manual_seed(3),
                                dtype=torch.int32)
    xs, Bs, Cs, ds = synth.token_inputs(w, 1, 2, batch=big, stream=6)
    res = {}
    for b in (big, small):
        ls = rs.LayerState(b, w.heads, w.groups, A, D, interval=w.interval, max_draft=T, in_dtype=x.dtype,
                           deferred_commit=True)
        rs.load_checkpoint(ls, S0[:b].contiguous().cuda())
        for r in range(R):
            rs.verify(ls, _bt(x[r, :, :b]).cuda(), _bt(Bm[r, :, :b]).cuda(), _bt(Cm[r, :, :b]).cuda(),
                      _bt(dt[r, :, :b]).cuda())
            rs.accept_deferred(ls, nk[r, :b].contiguous().cuda(), T)
        pos = ls.pos.cpu()
        assert (pos >= w.interval).any() and (pos < w.interval).any(), pos
        assert int(pos.max()) <= w.interval + T - 1
        ys = [rs.step(ls, xs[t, :b].contiguous().cuda(), Bs[t, :b].contiguous().cuda(),
                      Cs[t, :b].contiguous().cuda(), ds[t, :b].contiguous().cuda()).cpu() for t in range(2)]
        rs.check_device_errors(ls)
        folded = pos >= w.interval
        after = ls.pos.cpu()
        assert (after[folded] == 1).all()       # committed at the first step, then one token
        res[b] = (torch.stack(ys), ls.ckpt.cpu(), pos)
    assert torch.equal(res[big][0][:, :small], res[small][0])
    assert torch.equal(res[big][1][:small], res[small][1])
    # oracle: the kept tokens of every round, then the two steps
    pos = res[big][2]
    sl = [0, 1, 2, 3, big - 2, big - 1]
    assert any(pos[b] >= w.interval for b in sl) and any(pos[b] < w.interval for b in sl)
    S = np.asarray(oracle._f64(S0[sl]))
    for r in range(R):
        for i, b in enumerate(sl):
            k = int(nk[r, b])
            if k:
                Sb, _ = oracle.recurrent(S[i:i + 1], x[r, :k, b:b + 1], Bm[r, :k, b:b + 1],
                                         Cm[r, :k, b:b + 1], dt[r, :k, b:b + 1], A, D, w.groups)
                S[i] = np.asarray(Sb)[0]
    S1, y_ref = oracle.recurrent(S, xs[:1, sl], Bs[:1, sl], Cs[:1, sl], ds[:1, sl], A, D, w.groups)
    _, y_ref2 = oracle.recurrent(S1, xs[1:, sl], Bs[1:, sl], Cs[1:, sl], ds[1:, sl], A, D, w.groups)
    assert_close(res[big][0][0, sl], y_ref[0], "step output on the deferred slots")
    assert_close(res[big][0][1, sl], y_ref2[0], "next step")
    for i, b in enumerate(sl):
        if pos[b] >= w.interval:   # committed by the first step: checkpoint = state after it
            assert_close(res[big][1][b], np.asarray(S1)[i], f"checkpoint of slot {b} after the fold")


def test_second_deferred_accept_without_verify_is_flagged(rs):
    """An accept must follow a verify: a deferred accept on a slot already at
    pos >= L is clamped and reported, never indexes past the buffer."""
    w = dataclasses.replace(synth.WORKLOADS["tiny"], drafts=2)
    T = 3
    A, D = synth.layer_params(w, 0)
    ls = rs.LayerState(w.batch, w.heads, w.groups, A, D, interval=w.interval, max_draft=T,
                       in_dtype=torch.float32, deferred_commit=True)
    ls.pos.fill_(w.interval)
    rs.accept_deferred(ls, torch.ones(w.batch, dtype=torch.int32, device="cuda"), T)
    with pytest.raises(rs.ReplaySSMError, match="device"):
        rs.check_device_errors(ls)
    assert (ls.pos.cpu() <= w.interval).all()


def test_deferred_accept_needs_the_declaration(rs):
    """A layer that did not declare deferred commits refuses the call on the
    host (its steps and verifies never look for pos >= L)."""
    w = dataclasses.replace(synth.WORKLOADS["tiny"], drafts=2)
    A, D = synth.layer_params(w, 0)
    ls = rs.LayerState(w.batch, w.heads, w.groups, A, D, interval=w.interval, max_draft=3,
                       in_dtype=torch.float32)
    with pytest.raises(rs.ReplaySSMError, match="deferred_commit"):
        rs.accept_deferred(ls, torch.ones(w.batch, dtype=torch.int32, device="cuda"), 3)
