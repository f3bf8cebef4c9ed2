"""GPU parity of the continuous-batching boundary: a call's rows are mapped
to state slots of a larger pool (rssm_state.slot_idx; -1 = padding row).

Serving context (article "NVIDIA ReplaySSM: hybrid model SSM decoding with a
state buffer", section 2: batched requests): slots join (load_checkpoint into
a slot), decode at their own interval phase, and leave (flush the slot, copy
its checkpoint out).  A mapped call must give each slot exactly what an
unmapped call gives it (bit for bit, the per-row arithmetic is the same),
must not touch unmapped slots, and must leave padding rows' outputs alone.
"""
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


def _idx(v):
    return torch.tensor(v, dtype=torch.int32, device="cuda")


def test_mapped_steps_equal_unmapped(rs):
    """Pool of 8 slots, rows -> [6, 1, -1, 3, 0]; 37 steps (two commits + tail)
    against an unmapped layer holding the same four slots in row order."""
    w = synth.WORKLOADS["tiny"]
    A, D = synth.layer_params(w, 0)
    S0 = synth.init_state(w, 0, batch=8)
    smap = [6, 1, -1, 3, 0]
    live = [r for r, b in enumerate(smap) if b >= 0]
    x, Bm, Cm, dt = synth.token_inputs(w, 0, 37, batch=len(smap), stream=31)
    pool = rs.LayerState(8, w.heads, w.groups, A, D, in_dtype=x.dtype)
    rs.load_checkpoint(pool, S0.cuda())
    ref = rs.LayerState(len(live), w.heads, w.groups, A, D, in_dtype=x.dtype)
    rs.load_checkpoint(ref, S0[[smap[r] for r in live]].contiguous().cuda())
    untouched = {k: v.clone() for k, v in pool.tensors().items()}
    idx = _idx(smap)
    for t in range(37):
        y = torch.full((len(smap), w.heads, 64), 7.0, device="cuda")
        rs.step(pool, x[t].cuda(), Bm[t].cuda(), Cm[t].cuda(), dt[t].cuda(), y=y, slots=idx)
        yr = rs.step(ref, x[t, live].contiguous().cuda(), Bm[t, live].contiguous().cuda(),
                     Cm[t, live].contiguous().cuda(), dt[t, live].contiguous().cuda())
        assert torch.equal(y[live], yr), t
        assert (y[2] == 7.0).all()      # padding row untouched
    rs.check_device_errors(pool)
    for i, r in enumerate(live):
        b = smap[r]
        assert torch.equal(pool.ckpt[b], ref.ckpt[i])
        assert pool.pos[b].item() == ref.pos[i].item() == 37 % 16
        assert pool.intv[b].item() == ref.intv[i].item() == 2
    for b in (2, 4, 5, 7):
        assert torch.equal(pool.ckpt[b], untouched["ckpt"][b])
        assert pool.pos[b].item() == 0 and pool.intv[b].item() == 0
        assert torch.equal(pool.xbuf[b], untouched["xbuf"][b])


def test_admission_stagger_and_eviction(rs):
    """Slots join one per step (staggered interval phases), decode together,
    and slot 2 leaves after 30 steps: every output and the evicted state
    follow each slot's own recurrence (oracle)."""
    w = synth.WORKLOADS["4b"]
    S, steps = 5, 30
    A, D = synth.layer_params(w, 1)
    S0 = synth.init_state(w, 1, batch=S)
    x, Bm, Cm, dt = synth.token_inputs(w, 1, steps, batch=S, stream=32)
    pool = rs.LayerState(S, w.heads, w.groups, A, D, in_dtype=x.dtype)
    got = {b: [] for b in range(S)}
    tok = [0] * S
    for t in range(steps):
        if t < S:                      # slot t joins
            rs.load_checkpoint(pool, S0[t:t + 1].contiguous().cuda(), slots=_idx([t]))
        active = list(range(min(t + 1, S)))
        rows = [(b, tok[b]) for b in active]
        xi = torch.stack([x[i, b] for b, i in rows]).cuda()
        Bi = torch.stack([Bm[i, b] for b, i in rows]).cuda()
        Ci = torch.stack([Cm[i, b] for b, i in rows]).cuda()
        di = torch.stack([dt[i, b] for b, i in rows]).cuda()
        y = rs.step(pool, xi, Bi, Ci, di, slots=_idx(active)).cpu()
        for r, (b, i) in enumerate(rows):
            got[b].append(y[r])
            tok[b] += 1
    rs.check_device_errors(pool)
    assert sorted(pool.pos.cpu().tolist()) == sorted([n % 16 for n in tok])   # phases differ
    rs.commit(pool, slots=_idx([2]))     # eviction: flush, then the checkpoint is the slot's state
    evicted = pool.ckpt[2].cpu()
    for b in range(S):
        n = tok[b]
        Sb, y_ref = oracle.recurrent(S0[b:b + 1], x[:n, b:b + 1], Bm[:n, b:b + 1], Cm[:n, b:b + 1],
                                     dt[:n, b:b + 1], A, D, w.groups)
        for i in range(n):
            assert_close(got[b][i], y_ref[i, 0], f"slot {b} token {i}")
        if b == 2:
            assert_close(evicted, Sb[0], "evicted state")
            assert pool.pos[2].item() == 0


@pytest.mark.parametrize("deferred", [False, True])
def test_mapped_speculative_rounds(rs, deferred):
    """Verify + accept on a permuted subset of a pool equals the unmapped run."""
    w = synth.WORKLOADS["spec"]
    import dataclasses
    w = dataclasses.replace(w, heads=16, groups=2)
    T, R = w.drafts + 1, 12
    A, D = synth.layer_params(w, 0)
    S0 = synth.init_state(w, 0, batch=6)
    smap = [4, 0, 5, 2]
    x, Bm, Cm, dt = synth.token_inputs(w, 0, R, batch=4, tokens=T, stream=33)
    nk = synth.n_keep(w, R, batch=4, stream=33)
    kw = dict(interval=w.interval, max_draft=T, in_dtype=x.dtype, deferred_commit=deferred)
    pool = rs.LayerState(6, w.heads, w.groups, A, D, **kw)
    rs.load_checkpoint(pool, S0.cuda())
    ref = rs.LayerState(4, w.heads, w.groups, A, D, **kw)
    rs.load_checkpoint(ref, S0[smap].contiguous().cuda())
    acc = rs.accept_deferred if deferred else rs.accept
    idx = _idx(smap)
    bt = lambda t: t.transpose(0, 1).contiguous().cuda()
    for r in range(R):
        ins = (bt(x[r]), bt(Bm[r]), bt(Cm[r]), bt(dt[r]))
        yp = rs.verify(pool, *ins, slots=idx)
        yr = rs.verify(ref, *ins)
        assert torch.equal(yp, yr), r
        acc(pool, nk[r].contiguous().cuda(), T, slots=idx)
        acc(ref, nk[r].contiguous().cuda(), T)
    rs.commit(pool, slots=idx)
    rs.commit(ref)
    assert torch.equal(pool.ckpt[smap], ref.ckpt)
    assert torch.equal(pool.ckpt[[1, 3]], S0[[1, 3]].cuda())


def test_split_stream_keyed_by_slot(rs):
    """Precision split: the rounding stream is keyed by the state slot, so a
    permuted call over the whole pool writes the same bytes as the unmapped
    call."""
    w = synth.WORKLOADS["split"]
    batch, steps = 4, 20
    A, D = synth.layer_params(w, 0)
    S0 = synth.init_state(w, 0, batch=batch)
    x, Bm, Cm, dt = synth.token_inputs(w, 0, steps, batch=batch, stream=34)
    perm = [2, 0, 3, 1]
    inv = [perm.index(b) for b in range(batch)]
    la = rs.LayerState(batch, w.heads, w.groups, A, D, in_dtype=x.dtype, state_format="split-bf16", seed=9)
    lb = rs.LayerState(batch, w.heads, w.groups, A, D, in_dtype=x.dtype, state_format="split-bf16", seed=9)
    rs.load_checkpoint(la, S0.cuda())
    rs.load_checkpoint(lb, S0[perm].contiguous().cuda(), slots=_idx(perm))
    for t in range(steps):
        ya = rs.step(la, x[t].cuda(), Bm[t].cuda(), Cm[t].cuda(), dt[t].cuda())
        yb = rs.step(lb, x[t, perm].contiguous().cuda(), Bm[t, perm].contiguous().cuda(),
                     Cm[t, perm].contiguous().cuda(), dt[t, perm].contiguous().cuda(), slots=_idx(perm))
        assert torch.equal(ya[perm], yb), t
    for k in ("ckpt", "out_q", "out_scale", "pos", "intv"):
        assert torch.equal(getattr(la, k), getattr(lb, k)), k
    assert inv  # (permutation sanity)


def test_slot_out_of_range_is_flagged_and_skipped(rs):
    w = synth.WORKLOADS["tiny"]
    A, D = synth.layer_params(w, 0)
    x, Bm, Cm, dt = synth.token_inputs(w, 0, 1, batch=2, stream=35)
    pool = rs.LayerState(3, w.heads, w.groups, A, D, in_dtype=x.dtype)
    before = {k: v.clone() for k, v in pool.tensors().items()}
    y = torch.full((2, w.heads, 64), 3.0, device="cuda")
    rs.step(pool, x[0].cuda(), Bm[0].cuda(), Cm[0].cuda(), dt[0].cuda(), y=y, slots=_idx([99, 1]))
    with pytest.raises(rs.ReplaySSMError, match="device"):
        rs.check_device_errors(pool)
    assert (y[0] == 3.0).all()
    assert pool.pos[1].item() == 1 and pool.pos[0].item() == 0 and pool.pos[2].item() == 0
    assert torch.equal(pool.ckpt[0], before["ckpt"][0]) and torch.equal(pool.ckpt[2], before["ckpt"][2])


def test_prefill_into_slots(rs):
    """Prefill of two prompts into slots 2 and 0 of a pool of 3."""
    w = synth.WORKLOADS["tiny"]
    A, D = synth.layer_params(w, 2)
    S0 = synth.init_state(w, 2, batch=3)
    x, Bm, Cm, dt = synth.token_inputs(w, 2, 21, batch=2, stream=36)
    pool = rs.LayerState(3, w.heads, w.groups, A, D, in_dtype=x.dtype)
    rs.load_checkpoint(pool, S0.cuda())
    bt = lambda t: t.transpose(0, 1).contiguous().cuda()
    y = rs.prefill(pool, bt(x), bt(Bm), bt(Cm), bt(dt), slots=_idx([2, 0]))
    for r, b in enumerate([2, 0]):
        Sb, y_ref = oracle.recurrent(S0[b:b + 1], x[:, r:r + 1], Bm[:, r:r + 1], Cm[:, r:r + 1],
                                     dt[:, r:r + 1], A, D, w.groups)
        assert_close(pool.ckpt[b].cpu(), Sb[0], f"slot {b} state")
        for t in range(21):
            assert_close(y[r, t].cpu(), y_ref[t, 0], f"slot {b} token {t}")
    assert torch.equal(pool.ckpt[1], S0[1].cuda())


@pytest.mark.parametrize("heads,batch", [(8, 16), (96, 40)])
def test_duplicate_slots_are_flagged(rs, heads, batch):
    """Every row of a call on one slot (a race the caller must avoid): the
    position-publishing kernel sees more arrivals on the slot than one row
    brings and records it in the sticky error word.  All accesses stay in
    bounds (the racing rows write the same slot's valid entries), so the
    kernels end normally; only the slot's contents are undefined.  Both step
    kernels: 16 rows of 8 one-head workgroups (row split) and 40 rows of 24
    four-head tiles."""
    w = synth.WORKLOADS["tiny"] if heads == 8 else synth.WORKLOADS["4b"]
    A, D = synth.layer_params(w, 0)
    x, Bm, Cm, dt = synth.token_inputs(w, 0, 1, batch=batch, stream=37)
    pool = rs.LayerState(3, w.heads, w.groups, A, D, in_dtype=x.dtype)
    before = {k: v.clone() for k, v in pool.tensors().items()}
    rs.step(pool, x[0].cuda(), Bm[0].cuda(), Cm[0].cuda(), dt[0].cuda(), slots=_idx([1] * batch))
    with pytest.raises(rs.ReplaySSMError, match="same slot"):
        rs.check_device_errors(pool)
    for b in (0, 2):   # the other slots are untouched
        assert torch.equal(pool.ckpt[b], before["ckpt"][b]) and pool.pos[b].item() == 0
    rs.check_device_errors(pool)   # the flag was cleared by the read


@pytest.mark.parametrize("fmt", ["split-bf16", "low-e4m3"])
def test_duplicate_slots_are_flagged_low_precision(rs, fmt):
    """The same race on a low-precision state: the step marks each row's
    slot once, and the commit pass that follows it (which also moves the
    positions on) finds a slot marked by 40 rows and raises the flag; the
    other slots' bytes and positions are untouched."""
    w = synth.WORKLOADS["4b"]
    A, D = synth.layer_params(w, 0)
    x, Bm, Cm, dt = synth.token_inputs(w, 0, 1, batch=40, stream=38)
    pool = rs.LayerState(3, w.heads, w.groups, A, D, in_dtype=x.dtype, state_format=fmt)
    before = {k: v.clone() for k, v in pool.tensors().items()}
    rs.step(pool, x[0].cuda(), Bm[0].cuda(), Cm[0].cuda(), dt[0].cuda(), slots=_idx([1] * 40))
    with pytest.raises(rs.ReplaySSMError, match="same slot"):
        rs.check_device_errors(pool)
    for b in (0, 2):
        for k, v in pool.tensors().items():
            if v is not None and v.dim() > 0 and v.shape[0] == 3:
                assert torch.equal(v[b], before[k][b]), f"{k} of slot {b} changed"
    rs.check_device_errors(pool)
