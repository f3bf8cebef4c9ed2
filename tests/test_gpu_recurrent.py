"""GPU parity of the conventional (recurrent) baseline kernels against the
fp64 oracle, and replay-vs-recurrent agreement on the GPU.

Article ("NVIDIA ReplaySSM: hybrid model SSM decoding with a state buffer"):
section 1 (the conventional scheme reads and writes the whole state every
token), section 3 (conventional speculative decoding keeps a state copy per
draft token so it can roll back).
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


@pytest.mark.parametrize("name,batch,steps", [("tiny", None, 40), ("4b", 5, 24)])
def test_recurrent_step_matches_oracle(rs, name, batch, steps):
    w = synth.WORKLOADS[name]
    A, D = synth.layer_params(w, 0)
    S0 = synth.init_state(w, 0, batch=batch)
    x, Bm, Cm, dt = synth.token_inputs(w, 0, steps, batch=batch)
    state = S0.cuda()
    Ad, Dd = A.cuda(), D.cuda()
    ys = []
    for t in range(steps):
        ys.append(rs.recurrent_step(state, x[t].cuda(), Bm[t].cuda(), Cm[t].cuda(), dt[t].cuda(),
                                    Ad, Dd, groups=w.groups).cpu())
    S_ref, y_ref = oracle.recurrent(S0, x, Bm, Cm, dt, A, D, w.groups)
    for t in range(steps):
        assert_close(ys[t], y_ref[t], f"y step {t}")
    assert_close(state.cpu(), S_ref, "final state")


def test_replay_equals_recurrent_on_gpu(rs):
    """Both GPU paths agree within the same bar (replay = recurrence)."""
    w = synth.WORKLOADS["4b"]
    batch, steps = 4, 35
    A, D = synth.layer_params(w, 2)
    S0 = synth.init_state(w, 2, batch=batch).cuda()
    x, Bm, Cm, dt = (t.cuda() for t in synth.token_inputs(w, 2, steps, batch=batch))
    ls = rs.LayerState(batch, w.heads, w.groups, A, D, in_dtype=x.dtype)
    rs.load_checkpoint(ls, S0)
    state = S0.clone()
    Ad, Dd = A.cuda(), D.cuda()
    for t in range(steps):
        yr = rs.step(ls, x[t], Bm[t], Cm[t], dt[t])
        yc = rs.recurrent_step(state, x[t], Bm[t], Cm[t], dt[t], Ad, Dd, groups=w.groups)
        assert_close(yr.cpu(), yc.double().cpu().numpy(), f"step {t}")


def test_recurrent_spec_copies_match_oracle(rs):
    """Conventional speculative verify writes one state copy per draft; the
    accepted copy becomes the next round's state."""
    w = dataclasses.replace(synth.WORKLOADS["spec"], heads=16, groups=2)
    batch, R = 4, 6
    T = w.drafts + 1
    A, D = synth.layer_params(w, 0)
    S0 = synth.init_state(w, 0, batch=batch)
    x, Bm, Cm, dt = synth.token_inputs(w, 0, R, batch=batch, tokens=T)
    nk = synth.n_keep(w, R, batch=batch)
    nk[2, 1] = 0   # one fully rejected round
    pool = torch.zeros(batch, T + 1, w.heads, 64, 128, device="cuda")
    pool[:, 0] = S0.cuda()
    sel = torch.zeros(batch, dtype=torch.int32, device="cuda")
    Ad, Dd = A.cuda(), D.cuda()
    ref = oracle.spec_run(S0, x, Bm, Cm, dt, A, D, nk.numpy(), w.groups, 10 ** 9)
    bt = lambda t: t.transpose(0, 1).contiguous().cuda()
    for r in range(R):
        y = rs.recurrent_verify(pool, sel, bt(x[r]), bt(Bm[r]), bt(Cm[r]), bt(dt[r]), Ad, Dd,
                                groups=w.groups)
        rs.recurrent_accept(T + 1, sel, nk[r].cuda(), T, heads=w.heads, groups=w.groups)
        assert_close(y.transpose(0, 1).cpu(), ref["y"][r], f"round {r}")
        cur = pool[torch.arange(batch), sel.long()].cpu()
        assert_close(cur, ref["state"][r], f"state after round {r}")
