"""replayssm_step_noalloc (the step for callers that cannot allocate): the
per-slot arrival counters come from library scratch instead of the caller's
workspace, the kernels are the same, so outputs, checkpoints, buffers and
positions must equal replayssm_step's bit for bit.  Two calls in a row on
the 4B-class layout (batch 256, fp32 checkpoint, with a fused commit), the
second with a smaller input (batch 5 through a slot map on a 7-slot state,
split-bf16 state), each against the existing entry point on an identical
copy of the state.  Called through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from helpers import need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rs():
    need_gpu()
    import state_space_recurrence_amd as rs
    rs.lib()
    return rs


def _pair(rs, w, batch, fmt, layer):
    A, D = synth.layer_params(w, layer)
    S0 = synth.init_state(w, layer, batch=batch).cuda()
    states = []
    for _ in range(2):
        ls = rs.LayerState(batch, w.heads, w.groups, A, D, interval=w.interval, in_dtype=torch.bfloat16,
                           state_format=fmt, seed=7, layer_id=layer)
        rs.load_checkpoint(ls, S0)
        states.append(ls)
    return states


def _run(rs, L, ls, fn, ins, rows, slots):
    x, Bm, Cm, dt = ins
    ys = []
    d, st, n = rs._ctx(ls, slots)
    for t in range(x.shape[0]):
        y = torch.full((n, ls.heads, 64), float("nan"), device="cuda")
        rc = fn(ctypes.byref(d), ctypes.byref(st), x[t].data_ptr(), Bm[t].data_ptr(), Cm[t].data_ptr(),
                dt[t].data_ptr(), y.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == 0, L.replayssm_last_error().decode()
        ys.append(y)
    torch.cuda.synchronize()
    return torch.stack(ys)


def _same(a, b, what):
    assert torch.equal(a, b), f"{what} differs"


def test_noalloc_step_matches_step(rs):
    L = rs.lib()
    w = synth.WORKLOADS["4b"]
    # call 1: every slot of a batch-256 layer, 20 steps (a commit at step 16)
    ref, new = _pair(rs, w, w.batch, "f32", 0)
    ins = [t.cuda() for t in synth.token_inputs(w, 0, 20, stream=41)]
    print("[no-alloc] call 1: 4b layout, batch 256, 20 steps", flush=True)
    y_ref = _run(rs, L, ref, L.replayssm_step, ins, w.batch, None)
    y_new = _run(rs, L, new, L.replayssm_step_noalloc, ins, w.batch, None)
    _same(y_new, y_ref, "outputs (call 1)")
    for k, v in ref.tensors().items():
        _same(new.tensors()[k], v, f"{k} (call 1)")
    rs.check_device_errors(new)
    # call 2: a smaller input -- 5 rows mapped onto a 7-slot split-bf16 state
    ref, new = _pair(rs, w, 7, "split-bf16", 1)
    slots = torch.tensor([6, 0, 3, -1, 2], dtype=torch.int32, device="cuda")
    ins = [t.cuda() for t in synth.token_inputs(w, 1, 18, batch=5, stream=42)]
    print("[no-alloc] call 2: split-bf16, 5 rows on 7 slots, 18 steps", flush=True)
    y_ref = _run(rs, L, ref, L.replayssm_step, ins, 5, slots)
    y_new = _run(rs, L, new, L.replayssm_step_noalloc, ins, 5, slots)
    _same(y_new[:, [0, 1, 2, 4]], y_ref[:, [0, 1, 2, 4]], "outputs (call 2)")
    assert torch.isnan(y_new[:, 3]).all() and torch.isnan(y_ref[:, 3]).all()   # padding row untouched
    for k, v in ref.tensors().items():
        _same(new.tensors()[k], v, f"{k} (call 2)")
    assert new.pos.cpu().tolist() == [2, 0, 2, 2, 0, 0, 2]
    rs.check_device_errors(new)


def test_noalloc_rejects_too_many_slots(rs):
    L = rs.lib()
    d = rs._make_desc(70000, 8, 64, 128, 1, 16, 1, rs.F32)
    st = rs.RssmState()
    rc = L.replayssm_step_noalloc(ctypes.byref(d), ctypes.byref(st), None, None, None, None, None, None)
    assert rc == -3 and b"library scratch" in L.replayssm_last_error()
