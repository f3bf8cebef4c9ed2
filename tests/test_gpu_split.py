"""GPU parity of the precision split (article section 4) against the oracle.

Bars:
* quantised bytes (update checkpoint, FP4 codes and scales) bit-exact against
  the oracle's independent quantisers applied to the same fp32 values;
* outputs within 2e-5 * max(1, |y|) of the oracle recurrence replayed from
  the exactly decoded output source;
* the fp32 commit values (dumped before rounding) within 2e-5 * max(1, |S|)
  of the oracle recurrence replayed from the decoded update checkpoint.
The free-running low-precision trajectory is a measurement (drift), not a
parity check: commit values differ from the oracle's fp64 ones by ~1 ulp, so
the teacher-forced scheme re-anchors the oracle on the GPU's stored bytes at
every interval.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_close, need_gpu

pytestmark = pytest.mark.gpu

SPLIT_FORMATS = ["split-bf16", "split-e4m3", "shared-fp4", "low-bf16", "low-e4m3"]
SEED, LAYER = 0x5EED_0000_1234_ABCD, 3


@pytest.fixture(scope="module")
def rs():
    need_gpu()
    import state_space_recurrence_amd as rs
    rs.lib()
    return rs


def _ufmt(fmt):
    return {"split-bf16": "bf16", "low-bf16": "bf16", "split-e4m3": "e4m3", "low-e4m3": "e4m3"}.get(fmt)


def _decode_u(fmt, ckpt):
    u = ckpt.cpu().numpy()
    if _ufmt(fmt) == "bf16":
        return oracle.bf16_decode_array(u.view(np.uint16))
    return oracle.e4m3_decode_array(u)


def _decode_o(ls):
    return oracle.fp4_dequantize(ls.out_q.cpu().numpy(), ls.out_scale.cpu().numpy())


def _sources(fmt, ls):
    """(decoded state the outputs read, decoded state the updates read)."""
    if fmt == "shared-fp4":
        o = _decode_o(ls)
        return o, o
    u = _decode_u(fmt, ls.ckpt)
    if fmt.startswith("split"):
        return _decode_o(ls), u
    return u, u


def _check_quantised(fmt, ls, values, interval):
    """The GPU's stored bytes equal the oracle's quantisation of `values`."""
    v = values.cpu().numpy().astype(np.float32)
    if _ufmt(fmt):
        ref = oracle.sr_quantize(v.reshape(-1), _ufmt(fmt), SEED, LAYER, interval).reshape(v.shape)
        got = ls.ckpt.cpu().numpy()
        got = got.view(np.uint16) if _ufmt(fmt) == "bf16" else got
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"{fmt}: {len(bad)} update-checkpoint codes differ, first {bad[:3].tolist()}"
    if fmt.startswith("split") or fmt == "shared-fp4":
        codes, scales = oracle.fp4_quantize(v)
        assert np.array_equal(ls.out_scale.cpu().numpy(), scales), f"{fmt}: FP4 scales differ"
        assert np.array_equal(ls.out_q.cpu().numpy(), codes), f"{fmt}: FP4 codes differ"


def _special_state(shape, gen):
    """fp32 values exercising the quantisers: normal spread, tiny (E4M3
    subnormal / underflow), large (near and beyond 448), signed zeros, exact
    FP4 thresholds relative to a block scale, bf16 ties of the low 16 bits."""
    S = torch.randn(shape, generator=gen) * 0.1
    flat = S.view(-1, 128)
    n = flat.shape[0]
    flat[0:n:7] *= 1e-4
    flat[1:n:7] *= 3e3
    flat[2:n:7, :16] = 0.0
    flat[2:n:7, 16:32] = -0.0
    # one block per row with amax exactly 6 (scale 1.0) and values on the thresholds
    thr = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5,
                        -5.0, -6.0] * 2)
    flat[3:n:7, 32:64] = thr
    # values whose dropped bf16 bits are exactly 0x8000 (a stochastic-rounding midpoint)
    mid = (torch.randn(n // 7 + 1, 32).view(torch.int32) & ~0xFFFF | 0x8000).view(torch.float32)
    flat[4:n:7, 64:96] = mid[: flat[4:n:7].shape[0]]
    return S.contiguous()


@pytest.mark.parametrize("fmt", SPLIT_FORMATS)
def test_load_checkpoint_quantisers_bit_exact(rs, fmt):
    B, H, G = 5, 8, 2
    A, D = torch.full((H,), -1.0), torch.zeros(H)
    ls = rs.LayerState(B, H, G, A, D, in_dtype=torch.float32, state_format=fmt, seed=SEED, layer_id=LAYER)
    g = torch.Generator().manual_seed(11)
    S = _special_state((B, H, 64, 128), g)
    for interval in (0, 7):
        ls.intv.fill_(interval)
        rs.load_checkpoint(ls, S.cuda())
        torch.cuda.synchronize()
        _check_quantised(fmt, ls, S, interval)
        assert ls.pos.cpu().tolist() == [0] * B


def _run_intervals(rs, fmt, w, batch, n_intervals, tail, layer=0):
    """Standard decoding with teacher-forced oracle checks at every interval."""
    L = w.interval
    steps = n_intervals * L + tail
    A, D = synth.layer_params(w, layer)
    S0 = synth.init_state(w, layer, batch=batch)
    x, Bm, Cm, dt = synth.token_inputs(w, layer, steps, batch=batch)
    ls = rs.LayerState(batch, w.heads, w.groups, A, D, interval=L, in_dtype=x.dtype, state_format=fmt,
                       seed=SEED, layer_id=LAYER, debug_prequant=True)
    rs.load_checkpoint(ls, S0.cuda())
    xs, Bs, Cs, ds = (t.cuda() for t in (x, Bm, Cm, dt))
    t = 0
    for it in range(n_intervals + 1):
        n = L if it < n_intervals else tail
        if n == 0:
            break
        out_src, upd_src = _sources(fmt, ls)
        ys = [rs.step(ls, xs[t + i], Bs[t + i], Cs[t + i], ds[t + i]).cpu() for i in range(n)]
        sl = slice(t, t + n)
        _, y_ref = oracle.recurrent(out_src, x[sl], Bm[sl], Cm[sl], dt[sl], A, D, w.groups)
        for i in range(n):
            assert_close(ys[i], y_ref[i], f"{fmt} y at step {t + i}")
        if n == L:   # the step that closed the interval committed
            S_new, _ = oracle.recurrent(upd_src, x[sl], Bm[sl], Cm[sl], dt[sl], A, D, w.groups)
            dump = ls.debug_prequant.cpu()
            assert_close(dump, S_new, f"{fmt} commit values of interval {it}")
            _check_quantised(fmt, ls, dump, it + 1)
            assert ls.intv.cpu().tolist() == [it + 1] * batch
        t += n
    rs.check_device_errors(ls)
    return ls


@pytest.mark.parametrize("fmt", SPLIT_FORMATS)
def test_split_decode_teacher_forced(rs, fmt):
    w = dataclasses.replace(synth.WORKLOADS["split"], heads=16, groups=2)
    _run_intervals(rs, fmt, w, batch=3, n_intervals=3, tail=5)


@pytest.mark.parametrize("fmt", ["split-bf16", "split-e4m3", "shared-fp4"])
@pytest.mark.parametrize("L", [24, 32])
def test_split_decode_long_intervals(rs, fmt, L):
    """Intervals longer than 16 run the 32-entry step and commit instances
    (their decay sums span two DPP rows); outputs and commit values against
    the oracle, stored bytes bit-exact, over two intervals and a tail."""
    w = dataclasses.replace(synth.WORKLOADS["split"], heads=16, groups=2, interval=L)
    _run_intervals(rs, fmt, w, batch=3, n_intervals=2, tail=5)


@pytest.mark.parametrize("fmt,batch", [("split-bf16", 90)] + [(f, 300) for f in SPLIT_FORMATS])
def test_split_commit_long_lists(rs, fmt, batch):
    """Every slot closes its interval on the same step: at 16 heads on
    MI355X (3,072 or 4,096 resident commit waves), 90 listed slots make the
    commit pass give each wave half a head and 300 whole heads, several per
    wave (the short lists of the other tests give it single quarters); every
    format's update source goes through the coalesced loads."""
    w = dataclasses.replace(synth.WORKLOADS["split"], heads=16, groups=2)
    _run_intervals(rs, fmt, w, batch=batch, n_intervals=1, tail=1)


def test_split_decode_4b_layout(rs):
    """The 4B-class head layout (H=96, G=8), bf16 inputs, split-bf16."""
    w = synth.WORKLOADS["split"]
    _run_intervals(rs, "split-bf16", w, batch=2, n_intervals=2, tail=3)


def test_update_checkpoint_ignores_output_copy(rs):
    """Article section 4: the output copy is not used for the next update.
    Bit-exact: the bf16 update checkpoint evolves identically with the FP4
    copy (split) and without it (one bf16 checkpoint)."""
    w = dataclasses.replace(synth.WORKLOADS["split"], heads=16, groups=2)
    batch, steps = 3, 3 * w.interval + 4
    A, D = synth.layer_params(w, 1)
    S0 = synth.init_state(w, 1, batch=batch).cuda()
    x, Bm, Cm, dt = (t.cuda() for t in synth.token_inputs(w, 1, steps, batch=batch))
    cks = []
    for fmt in ("split-bf16", "low-bf16"):
        ls = rs.LayerState(batch, w.heads, w.groups, A, D, in_dtype=x.dtype, state_format=fmt, seed=SEED,
                           layer_id=LAYER)
        rs.load_checkpoint(ls, S0)
        for t in range(steps):
            rs.step(ls, x[t], Bm[t], Cm[t], dt[t])
        cks.append(ls.ckpt.clone())
    assert torch.equal(cks[0], cks[1])


@pytest.mark.parametrize("fmt,L", [("split-bf16", 16), ("split-e4m3", 16), ("shared-fp4", 16),
                                   ("split-bf16", 24), ("shared-fp4", 8)])
def test_split_speculative_rounds(rs, fmt, L):
    """Verify reads the output source; accept commits from the update source
    once the position count reaches L (teacher-forced at every commit).
    With 5 positions the buffer holds 20 entries at L = 16 (the 24-entry
    verify instance), 28 at L = 24 (the 32-entry one) and 12 at L = 8."""
    w = dataclasses.replace(synth.WORKLOADS["spec"], heads=16, groups=2, in_dtype="bf16", interval=L)
    batch, R = 4, 14 * max(1, L // 16)
    T = w.drafts + 1
    A, D = synth.layer_params(w, 0)
    S0 = synth.init_state(w, 0, batch=batch)
    x, Bm, Cm, dt = synth.token_inputs(w, 0, R, batch=batch, tokens=T)
    nk = synth.n_keep(w, R, batch=batch)
    ls = rs.LayerState(batch, w.heads, w.groups, A, D, interval=w.interval, max_draft=T, in_dtype=x.dtype,
                       state_format=fmt, seed=SEED, layer_id=LAYER, debug_prequant=True)
    rs.load_checkpoint(ls, S0.cuda())
    bt = lambda t: t.transpose(0, 1).contiguous().cuda()
    out_src, upd_src = _sources(fmt, ls)
    hist = [[] for _ in range(batch)]   # accepted (round, position) since the last commit
    pos = np.zeros(batch, dtype=int)
    for r in range(R):
        y = rs.verify(ls, bt(x[r]), bt(Bm[r]), bt(Cm[r]), bt(dt[r])).cpu()
        for b in range(batch):
            idx = hist[b]
            xs = torch.stack([x[rr, tt, b] for rr, tt in idx] + [x[r, tt, b] for tt in range(T)])[:, None]
            Bs = torch.stack([Bm[rr, tt, b] for rr, tt in idx] + [Bm[r, tt, b] for tt in range(T)])[:, None]
            Cs = torch.stack([Cm[rr, tt, b] for rr, tt in idx] + [Cm[r, tt, b] for tt in range(T)])[:, None]
            ds = torch.stack([dt[rr, tt, b] for rr, tt in idx] + [dt[r, tt, b] for tt in range(T)])[:, None]
            _, yref = oracle.recurrent(out_src[b:b + 1], xs, Bs, Cs, ds, A, D, w.groups)
            assert_close(y[b], yref[len(idx):, 0], f"{fmt} verify round {r} slot {b}")
        rs.accept(ls, nk[r].cuda(), T)
        new_pos = pos + nk[r].numpy()
        committed = new_pos >= w.interval
        dump = ls.debug_prequant.cpu()
        out_next, upd_next = _sources(fmt, ls)
        for b in range(batch):
            hist[b] += [(r, tt) for tt in range(int(nk[r, b]))]
            if committed[b]:
                idx = hist[b]
                xs = torch.stack([x[rr, tt, b] for rr, tt in idx])[:, None]
                Bs = torch.stack([Bm[rr, tt, b] for rr, tt in idx])[:, None]
                Cs = torch.stack([Cm[rr, tt, b] for rr, tt in idx])[:, None]
                ds = torch.stack([dt[rr, tt, b] for rr, tt in idx])[:, None]
                S_new, _ = oracle.recurrent(upd_src[b:b + 1], xs, Bs, Cs, ds, A, D, w.groups)
                assert_close(dump[b:b + 1], S_new, f"{fmt} commit values slot {b} round {r}")
                hist[b] = []
        if committed.any():
            # bytes of committed slots == oracle quantisation of their dumped values
            for b in np.nonzero(committed)[0]:
                v = dump[b].numpy().astype(np.float32)
                interval = int(ls.intv[b])
                e0 = b * w.heads * 64 * 128
                if _ufmt(fmt):
                    ref = oracle.sr_quantize(v.reshape(-1), _ufmt(fmt), SEED, LAYER, interval, elem0=e0)
                    got = ls.ckpt[b].cpu().numpy().reshape(-1)
                    got = got.view(np.uint16) if _ufmt(fmt) == "bf16" else got
                    assert np.array_equal(got, ref), f"{fmt} update bytes slot {b} round {r}"
                codes, scales = oracle.fp4_quantize(v)
                assert np.array_equal(ls.out_q[b].cpu().numpy(), codes), f"{fmt} FP4 codes slot {b}"
                assert np.array_equal(ls.out_scale[b].cpu().numpy(), scales), f"{fmt} FP4 scales slot {b}"
        # sources for the next round: committed slots re-anchor on the new bytes
        for b in range(batch):
            if committed[b]:
                out_src[b], upd_src[b] = out_next[b], upd_next[b]
        pos = np.where(committed, 0, new_pos)
        assert np.array_equal(ls.pos.cpu().numpy(), pos)
    rs.check_device_errors(ls)


def test_split_drift_ordering(rs):
    """Sanity (article section 4, not a parity bar): outputs drift less from
    the fp32 trajectory with the split than with one shared FP4 state.  The
    decay rates are scaled down 100x so the state has a long memory (with the
    workload's rates it forgets within a few tokens and all formats drift
    alike)."""
    w = dataclasses.replace(synth.WORKLOADS["split"], heads=16, groups=2)
    batch, steps = 4, 8 * w.interval
    A, D = synth.layer_params(w, 0)
    A = A * 0.01
    S0 = synth.init_state(w, 0, batch=batch).cuda()
    x, Bm, Cm, dt = (t.cuda() for t in synth.token_inputs(w, 0, steps, batch=batch))
    ys = {}
    for fmt in ("f32", "split-bf16", "shared-fp4"):
        ls = rs.LayerState(batch, w.heads, w.groups, A, D, in_dtype=x.dtype, state_format=fmt, seed=SEED)
        rs.load_checkpoint(ls, S0)
        ys[fmt] = torch.stack([rs.step(ls, x[t], Bm[t], Cm[t], dt[t]).clone() for t in range(steps)])
    ref = ys["f32"]
    drift = {f: float((ys[f] - ref)[-w.interval:].norm() / ref[-w.interval:].norm()) for f in ys if f != "f32"}
    print("drift over the last interval:", drift)
    assert drift["split-bf16"] < drift["shared-fp4"]


def test_device_conversions_exhaustive(rs):
    """The matrix-core commit takes FP4 codes from gfx950's f32 -> E2M1
    conversion of v / scale bracketed from both sides, and rounds bf16 by
    integer addition.  Over every non-NaN fp32 bit pattern the conversion
    equals the exact threshold encoding (round to nearest even, saturating
    at 6, sign kept) and the addition form equals the selecting form; the
    bit-exact byte checks of the other tests then rest on no untested input.
    The E4M3 stochastic rounding the kernels use (carry form in the normal
    range, exact floor split below it) equals the grid-split form, which the
    decode tests pin to the oracle, for every pattern with two draws each."""
    assert rs.check_conversions(0, 1 << 32) == (0, 0, 0)


@pytest.mark.parametrize("fmt", ["low-e4m3", "split-e4m3", "shared-fp4"])
def test_e4m3_decode_of_every_code(rs, fmt):
    """Every E4M3 code (OCP E4M3FN: subnormals, signed zeros, 448, NaN) is
    decoded exactly, compared with the oracle's decode table.  One step at
    position 0 with x = 0, dt = 0 and C = e_0 outputs exactly the decoded
    column 0 of each row of the output source (Lambda = exp(0) = 1, no
    buffer term): for the single E4M3 checkpoint that is the stored code; for
    the FP4 copy, element 0 holds E2M1 1.0 and the row's first block scale is
    the code under test, so the output is the decoded scale."""
    w = dataclasses.replace(synth.WORKLOADS["tiny"])
    Bsz, H, G, P, N = w.batch, w.heads, w.groups, 64, 128
    A, D = synth.layer_params(w, 0)
    ls = rs.LayerState(Bsz, H, G, A, D, interval=w.interval, in_dtype=torch.float32, state_format=fmt,
                       layer_id=LAYER, seed=SEED)
    codes = (torch.arange(Bsz * H * P, dtype=torch.int64) % 256).to(torch.uint8).reshape(Bsz, H, P)
    if fmt == "low-e4m3":
        ls.ckpt.copy_(codes[..., None].expand(Bsz, H, P, N).contiguous().cuda())
    else:
        q = torch.zeros(Bsz, H, P, N // 2, dtype=torch.uint8)
        q[..., 0] = 0x02                               # element 0: E2M1 code 2 = 1.0; the rest 0
        sc = torch.full((Bsz, H, P, N // 32), 0x38, dtype=torch.uint8)   # 1.0 for the zero blocks
        sc[..., 0] = codes
        ls.out_q.copy_(q.cuda())
        ls.out_scale.copy_(sc.cuda())
    x = torch.zeros(Bsz, H, P, device="cuda")
    Bm = torch.zeros(Bsz, G, N, device="cuda")
    Cm = torch.zeros(Bsz, G, N, device="cuda")
    Cm[..., 0] = 1.0
    dt = torch.zeros(Bsz, H, device="cuda")
    y = rs.step(ls, x, Bm, Cm, dt).cpu().double().numpy()
    rs.check_device_errors(ls)
    ref = oracle.e4m3_decode_array(codes.numpy())
    assert np.array_equal(y, ref, equal_nan=True), (
        f"{fmt}: codes decoded differently: {sorted(set(codes.numpy()[~np.isclose(y, ref, rtol=0, atol=0, equal_nan=True)].tolist()))[:16]}")
    assert np.isnan(y).sum() == np.isnan(ref).sum() > 0


def _quant_bytes(ls):
    """Stored bytes of every slot: update checkpoint (if any), FP4 codes, scales."""
    return [t.cpu().clone() for t in (ls.ckpt, ls.out_q, ls.out_scale) if t is not None]


@pytest.mark.parametrize("fmt", SPLIT_FORMATS)
def test_split_decode_staggered_phases(rs, fmt):
    """Continuous batching: slot b joins at step b mod L through the slot
    map (rows in reverse slot order), so after the first interval every step
    carries committing and non-committing slots in one launch.  Teacher
    forced per slot: each output from the oracle replaying the slot's tokens
    since its last commit from the decoded output source; each commit's
    pre-rounding values from the decoded update source; the committing
    slots' bytes bit-exact against the oracle's quantisation of those values
    with the slot's own interval index and element offset; every other
    slot's bytes unchanged."""
    w = dataclasses.replace(synth.WORKLOADS["split"], heads=16, groups=2)
    L, batch = w.interval, 20
    steps = 2 * L + 6
    A, D = synth.layer_params(w, 2)
    S0 = synth.init_state(w, 2, batch=batch)
    x, Bm, Cm, dt = synth.token_inputs(w, 2, steps, batch=batch, stream=5)
    ls = rs.LayerState(batch, w.heads, w.groups, A, D, interval=L, in_dtype=x.dtype, state_format=fmt,
                       seed=SEED, layer_id=LAYER, debug_prequant=True)
    rs.load_checkpoint(ls, S0.cuda())
    out_src, upd_src = _sources(fmt, ls)
    hist = [[] for _ in range(batch)]
    joined = [b % L for b in range(batch)]
    elems = w.heads * 64 * 128
    n_commits = 0
    for t in range(steps):
        rows = [b for b in range(batch) if joined[b] <= t][::-1]
        idx = torch.tensor(rows, dtype=torch.int32, device="cuda")
        before = _quant_bytes(ls)
        y = rs.step(ls, x[t, rows].cuda(), Bm[t, rows].cuda(), Cm[t, rows].cuda(), dt[t, rows].cuda(),
                    slots=idx).cpu()
        committed = [b for b in rows if len(hist[b]) == L - 1]
        after = _quant_bytes(ls)
        if committed:
            dump = ls.debug_prequant.cpu()
            out_next, upd_next = _sources(fmt, ls)
            intv = ls.intv.cpu()
        for r, b in enumerate(rows):
            hist[b].append(t)
            tt = hist[b]
            sel = lambda a: a[tt, b:b + 1]
            _, yref = oracle.recurrent(out_src[b:b + 1], sel(x), sel(Bm), sel(Cm), sel(dt), A, D, w.groups)
            assert_close(y[r], yref[-1, 0], f"{fmt} y of slot {b} at step {t}")
        for b in range(batch):
            if b not in committed:
                for k, (u, v) in enumerate(zip(before, after)):
                    assert torch.equal(u[b], v[b]), f"{fmt}: bytes {k} of non-committing slot {b} changed at step {t}"
                continue
            tt = hist[b]
            sel = lambda a: a[tt, b:b + 1]
            S_new, _ = oracle.recurrent(upd_src[b:b + 1], sel(x), sel(Bm), sel(Cm), sel(dt), A, D, w.groups)
            assert_close(dump[b:b + 1], S_new, f"{fmt} commit values of slot {b} at step {t}")
            v = dump[b].numpy().astype(np.float32)
            if _ufmt(fmt):
                ref = oracle.sr_quantize(v.reshape(-1), _ufmt(fmt), SEED, LAYER, int(intv[b]), elem0=b * elems)
                got = ls.ckpt[b].cpu().numpy().reshape(-1)
                got = got.view(np.uint16) if _ufmt(fmt) == "bf16" else got
                assert np.array_equal(got, ref), f"{fmt} update bytes of slot {b} at step {t}"
            if fmt.startswith("split") or fmt == "shared-fp4":
                codes, scales = oracle.fp4_quantize(v)
                assert np.array_equal(ls.out_q[b].cpu().numpy(), codes), f"{fmt} FP4 codes of slot {b}"
                assert np.array_equal(ls.out_scale[b].cpu().numpy(), scales), f"{fmt} FP4 scales of slot {b}"
            out_src[b], upd_src[b] = out_next[b], upd_next[b]
            hist[b] = []
            n_commits += 1
        exp_pos = np.array([len(h) for h in hist], dtype=np.int32)
        assert np.array_equal(ls.pos.cpu().numpy(), exp_pos), f"positions after step {t}"
    rs.check_device_errors(ls)
    assert n_commits == sum((steps - j) // L for j in joined)
    assert ls.intv.cpu().tolist() == [(steps - joined[b]) // L for b in range(batch)]


@pytest.mark.parametrize("fmt", ["split-bf16", "split-e4m3"])
def test_split_largest_pool_element_index(rs, fmt):
    """The largest pool a low-precision state accepts (its flat element
    index must fit 32 bits: at 16 heads, 32,767 slots), with rows mapped to
    slots on both sides of element 2^31 and to the last slot, so the
    rounding draws' element index must be carried unsigned (a signed 32-bit
    index would turn negative past 2^31).  The loaded checkpoint and one
    interval's commit are checked bit-exact against the oracle's
    quantisation with each slot's own element offset, and every output of
    the interval against the oracle's replay (one slot more is refused by
    the descriptor check, tested on the host)."""
    w = dataclasses.replace(synth.WORKLOADS["split"], heads=16, groups=2)
    L = w.interval
    elems = w.heads * 64 * 128
    nslots = 0xFFFFFFFF // elems
    slots = [0, (1 << 31) // elems - 1, (1 << 31) // elems, nslots - 1]
    assert slots[1] * elems < (1 << 31) <= slots[2] * elems
    rows = len(slots)
    A, D = synth.layer_params(w, 1)
    S0 = _special_state((rows, w.heads, 64, 128), torch.Generator().manual_seed(21))
    x, Bm, Cm, dt = synth.token_inputs(w, 1, L, batch=rows, stream=9)
    ls = rs.LayerState(nslots, w.heads, w.groups, A, D, interval=L, in_dtype=x.dtype, state_format=fmt,
                       seed=SEED, layer_id=LAYER, debug_prequant=True)
    idx = torch.tensor(slots, dtype=torch.int32, device="cuda")
    rs.load_checkpoint(ls, S0.cuda(), slots=idx)
    sl = idx.long()

    def check_bytes(values, interval, what):
        got_u = ls.ckpt[sl].cpu().numpy()
        got_u = got_u.view(np.uint16) if _ufmt(fmt) == "bf16" else got_u
        for r, b in enumerate(slots):
            v = values[r].numpy().astype(np.float32)
            ref = oracle.sr_quantize(v.reshape(-1), _ufmt(fmt), SEED, LAYER, interval, elem0=b * elems)
            assert np.array_equal(got_u[r].reshape(-1), ref), f"{fmt} {what}: update bytes of slot {b}"
            codes, scales = oracle.fp4_quantize(v)
            assert np.array_equal(ls.out_q[b].cpu().numpy(), codes), f"{fmt} {what}: FP4 codes of slot {b}"
            assert np.array_equal(ls.out_scale[b].cpu().numpy(), scales), f"{fmt} {what}: FP4 scales of slot {b}"

    check_bytes(S0, 0, "load")
    out_src = oracle.fp4_dequantize(ls.out_q[sl].cpu().numpy(), ls.out_scale[sl].cpu().numpy())
    upd_src = _decode_u(fmt, ls.ckpt[sl])
    ys = [rs.step(ls, x[t].cuda(), Bm[t].cuda(), Cm[t].cuda(), dt[t].cuda(), slots=idx).cpu() for t in range(L)]
    _, y_ref = oracle.recurrent(out_src, x, Bm, Cm, dt, A, D, w.groups)
    for t in range(L):
        assert_close(ys[t], y_ref[t], f"{fmt} y at step {t}")
    S_new, _ = oracle.recurrent(upd_src, x, Bm, Cm, dt, A, D, w.groups)
    dump = ls.debug_prequant[sl].cpu()
    assert_close(dump, S_new, f"{fmt} commit values")
    check_bytes(dump, 1, "commit")
    assert ls.intv[sl].cpu().tolist() == [1] * rows and ls.pos[sl].cpu().tolist() == [0] * rows
    rs.check_device_errors(ls)


@pytest.mark.parametrize("fmt", ["split-bf16", "split-e4m3", "shared-fp4"])
def test_split_flush_commits_open_slots(rs, fmt):
    """A flush commits every slot holding entries, each from its own count
    (slots at different positions, one at 0): values against the oracle's
    recurrence from the update source, stored bytes bit-exact, positions 0
    and interval counts moved on only where a commit happened."""
    w = dataclasses.replace(synth.WORKLOADS["split"], heads=16, groups=2)
    batch, steps = 4, 11
    A, D = synth.layer_params(w, 0)
    S0 = synth.init_state(w, 0, batch=batch)
    x, Bm, Cm, dt = synth.token_inputs(w, 0, steps, batch=batch)
    ls = rs.LayerState(batch, w.heads, w.groups, A, D, interval=w.interval, in_dtype=x.dtype, state_format=fmt,
                       seed=SEED, layer_id=LAYER, debug_prequant=True)
    rs.load_checkpoint(ls, S0.cuda())
    counts = [11, 5, 0, 1]   # entries per slot before the flush
    for t in range(steps):
        rows = [b for b in range(batch) if counts[b] > t]
        idx = torch.tensor(rows, dtype=torch.int32, device="cuda")
        rs.step(ls, x[t, rows].cuda(), Bm[t, rows].cuda(), Cm[t, rows].cuda(), dt[t, rows].cuda(), slots=idx)
    assert ls.pos.cpu().tolist() == counts
    _, upd_src = _sources(fmt, ls)
    ls.debug_prequant.zero_()
    rs.commit(ls)
    rs.check_device_errors(ls)
    assert ls.pos.cpu().tolist() == [0] * batch
    assert ls.intv.cpu().tolist() == [1 if c else 0 for c in counts]
    dump = ls.debug_prequant.cpu()
    for b, c in enumerate(counts):
        if c == 0:
            continue
        S_new, _ = oracle.recurrent(upd_src[b:b + 1], x[:c, b:b + 1], Bm[:c, b:b + 1], Cm[:c, b:b + 1],
                                    dt[:c, b:b + 1], A, D, w.groups)
        assert_close(dump[b:b + 1], S_new, f"{fmt} flush values of slot {b}")
    # bytes: committed slots from the dumped values (stream index 1), the
    # untouched slot kept its load-time bytes (stream index 0)
    v = dump.numpy().astype(np.float32)
    if _ufmt(fmt):
        got = ls.ckpt.cpu().numpy()
        got = got.view(np.uint16) if _ufmt(fmt) == "bf16" else got
        for b, c in enumerate(counts):
            if c:
                ref = oracle.sr_quantize(v[b].reshape(-1), _ufmt(fmt), SEED, LAYER, 1, elem0=b * v[b].size)
                assert np.array_equal(got[b].reshape(-1), ref), f"{fmt} update bytes of slot {b}"
    codes, scales = oracle.fp4_quantize(v)
    for b, c in enumerate(counts):
        if c:
            assert np.array_equal(ls.out_q[b].cpu().numpy(), codes[b]), f"{fmt} FP4 codes of slot {b}"
            assert np.array_equal(ls.out_scale[b].cpu().numpy(), scales[b]), f"{fmt} FP4 scales of slot {b}"


@pytest.mark.parametrize("fmt", ["split-bf16", "shared-fp4"])
def test_split_accept_flags(rs, fmt):
    """Low-precision accepts flag n_keep outside 0..T (clamped) and two rows
    on one slot, like the fp32 accept."""
    w = dataclasses.replace(synth.WORKLOADS["spec"], heads=16, groups=2, in_dtype="bf16")
    batch = 2
    T = w.drafts + 1
    A, D = synth.layer_params(w, 0)
    x, Bm, Cm, dt = synth.token_inputs(w, 0, 1, batch=batch, tokens=T)
    bt = lambda t: t[0].transpose(0, 1).contiguous().cuda()
    ls = rs.LayerState(batch, w.heads, w.groups, A, D, interval=w.interval, max_draft=T, in_dtype=x.dtype,
                       state_format=fmt, seed=SEED, layer_id=LAYER)
    rs.load_checkpoint(ls, synth.init_state(w, 0, batch=batch).cuda())
    rs.verify(ls, bt(x), bt(Bm), bt(Cm), bt(dt))
    rs.accept(ls, torch.tensor([9, -1], dtype=torch.int32, device="cuda"), T)
    with pytest.raises(rs.ReplaySSMError, match="device"):
        rs.check_device_errors(ls)
    assert ls.pos.cpu().tolist() == [T, 0]
    rs.verify(ls, bt(x), bt(Bm), bt(Cm), bt(dt), slots=torch.tensor([0, 1], dtype=torch.int32, device="cuda"))
    rs.accept(ls, torch.tensor([1, 1], dtype=torch.int32, device="cuda"), T,
              slots=torch.tensor([1, 1], dtype=torch.int32, device="cuda"))
    with pytest.raises(rs.ReplaySSMError, match="same slot"):
        rs.check_device_errors(ls)
