"""GPU parity of every checkpoint row written by the fused interval commit,
and of the fp32 path's degenerate cases.

Commit rows: the replay step rewrites the checkpoint in the step that closes
an interval (article section 1: the state is written once per interval).
A build whose last commit store of a wave (rows 62-63 of a head, the store
whose data VGPRs the next instruction overwrote) wrote wrong values for
single heads of late slots; here, in the launch configuration the benchmark
times (4B-class heads, batch 256, workgroups of 4 heads: every wave index),
the whole checkpoint of the first and last slots and of three more is
compared with the oracle, element by element, after every fused commit, and
so are every output of those slots.  The 120B-class shape (32 workgroups of
4 heads per slot) is covered the same way.

Degenerate cases (every output and checkpoint against the oracle, plus the
closed form each reduces to, on both step kernels):
* decay underflow inside one interval: sum of A dt far below log(FLT_MIN),
  where a ratio of prefix products would give 0/0;
* dt = 0: Lambda = 1, no input term, so y = S0 . C + D x and the committed
  checkpoint equals S0 bit for bit;
* x = 0: pure decay, y = Lambda_k (S0 . C) and S_L = Lambda_L S0;
* B orthogonal to C and S0 = 0: every Gram entry is 0, so y = D x.
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


@pytest.mark.parametrize("name", ["4b", "120b"])
def test_fused_commit_rows_every_head(rs, name):
    w = synth.WORKLOADS[name]
    dev = torch.device("cuda")
    L = w.interval
    steps = 4 * L + 3
    slots = [0, 1, w.batch // 2, w.batch - 2, w.batch - 1]
    sl = torch.tensor(slots, device=dev)
    layer = 1
    print(f"[commit-rows] {w.describe()} steps={steps} slots={slots}", flush=True)
    A, D = synth.layer_params(w, layer, device=dev)
    S0 = synth.init_state(w, layer, device=dev)
    x, Bm, Cm, dt = synth.token_inputs(w, layer, steps, device=dev, stream=21)
    ls = rs.LayerState(w.batch, w.heads, w.groups, A, D, interval=L, in_dtype=x.dtype, device=dev,
                       layer_id=layer)
    rs.load_checkpoint(ls, S0)
    y = torch.empty(steps, w.batch, w.heads, 64, device=dev)
    cks = []
    for t in range(steps):
        rs.step(ls, x[t], Bm[t], Cm[t], dt[t], y=y[t])
        if (t + 1) % L == 0:
            cks.append(ls.ckpt[sl].cpu())
    rs.check_device_errors(ls)
    y_s = y[:, sl].cpu()
    ins = [t[:, sl].cpu() for t in (x, Bm, Cm, dt)]
    S0s = S0[sl].cpu()
    del x, Bm, Cm, dt, y, ls
    torch.cuda.empty_cache()
    y_ref, ck_ref = oracle.decode_run(S0s, *ins, A.cpu(), D.cpu(), w.groups, L)
    assert len(cks) == len(ck_ref) == 4
    for i, (c, r) in enumerate(zip(cks, ck_ref)):
        for k, b in enumerate(slots):
            for h0 in range(0, w.heads, 4):   # one workgroup (4 waves) at a time, for the message
                assert_close(c[k, h0:h0 + 4], r[k, h0:h0 + 4],
                             f"{name}: checkpoint after interval {i}, slot {b}, heads {h0}..{h0 + 3}")
    assert_close(y_s, y_ref, f"{name}: outputs of slots {slots}")


def _edge_inputs(case, w, batch, steps, gen):
    """Inputs (fp32) of one degenerate case: (S0, x, Bm, Cm, dt, A, D)."""
    H, G, P, N = w.heads, w.groups, 64, 128
    A, D = synth.layer_params(w, 5)
    S0 = synth.init_state(w, 5, batch=batch)
    x, Bm, Cm, dt = synth.token_inputs(w, 5, steps, batch=batch, stream=31)
    if case == "underflow":
        # half the heads at A = -16 with dt in [2, 8): A dt <= -32 per token, so
        # the interval sum passes log(FLT_MIN) ~ -87.3 within 3 tokens
        A = A.clone()
        A[: H // 2] = -16.0
        dt = dt.clone()
        dt[..., : H // 2] = 2.0 + 6.0 * torch.rand(steps, batch, H // 2, generator=gen)
    elif case == "dt0":
        dt = torch.zeros_like(dt)
    elif case == "x0":
        x = torch.zeros_like(x)
    elif case == "orth":
        S0 = torch.zeros_like(S0)
        Bm = Bm.clone()
        Cm = Cm.clone()
        Bm[..., N // 2:] = 0.0    # B on the first half of the state dims,
        Cm[..., : N // 2] = 0.0   # C on the second half: B_j . C_t = 0 exactly
    return S0, x, Bm, Cm, dt, A, D


@pytest.mark.parametrize("batch", [3, 300])
@pytest.mark.parametrize("case", ["underflow", "dt0", "x0", "orth"])
def test_degenerate_cases(rs, case, batch):
    w = synth.WORKLOADS["tiny"]
    L = w.interval
    steps = 2 * L + 5
    gen = torch.Generator().manual_seed(77)
    S0, x, Bm, Cm, dt, A, D = _edge_inputs(case, w, batch, steps, gen)
    ls = rs.LayerState(batch, w.heads, w.groups, A, D, interval=L, in_dtype=torch.float32)
    rs.load_checkpoint(ls, S0.cuda())
    sl = [0, batch // 2, batch - 1]
    ys, cks = [], []
    for t in range(steps):
        ys.append(rs.step(ls, x[t].cuda(), Bm[t].cuda(), Cm[t].cuda(), dt[t].cuda()).cpu()[sl])
        if (t + 1) % L == 0:
            cks.append(ls.ckpt.cpu()[sl].clone())
    torch.cuda.synchronize()
    rs.check_device_errors(ls)
    y = torch.stack(ys).double().numpy()
    assert np.isfinite(y).all(), f"{case}: non-finite outputs"
    y_ref, ck_ref = oracle.decode_run(S0[sl], x[:, sl], Bm[:, sl], Cm[:, sl], dt[:, sl], A, D, w.groups, L)
    assert_close(torch.from_numpy(y), y_ref, f"{case}: outputs vs oracle (batch {batch})")
    for i, (c, r) in enumerate(zip(cks, ck_ref)):
        assert_close(c, r, f"{case}: checkpoint after interval {i} vs oracle (batch {batch})")

    # the closed form each case reduces to, in fp64 on the host
    S0d = S0[sl].double()
    g = torch.arange(w.heads) // (w.heads // w.groups)
    xd, Cd, dd = x[:, sl].double(), Cm[:, sl].double(), dt[:, sl].double()
    Dd, Ad = D.double(), A.double()
    if case == "dt0":
        y_cf = torch.einsum("bhpn,tbhn->tbhp", S0d, Cd[:, :, g]) + Dd[None, None, :, None] * xd
        assert_close(torch.from_numpy(y), y_cf.numpy(), "dt0: y = S0 . C + D x")
        for c in cks:
            assert torch.equal(c, S0[sl]), "dt0: a commit must leave the checkpoint unchanged"
    elif case == "x0":
        cum = torch.cumsum(Ad[None, None, :] * dd, 0)          # [t, b, h]: decay sums from step 0
        start = lambda t: cum[t] if t >= 0 else torch.zeros_like(cum[0])
        S_start = [S0d * torch.exp(start(k * L - 1))[..., None, None] for k in range(steps // L + 1)]
        y_cf = torch.stack([torch.exp(cum[t] - start(t // L * L - 1))[..., None]
                            * torch.einsum("bhpn,bhn->bhp", S_start[t // L], Cd[t][:, g]) for t in range(steps)])
        assert_close(torch.from_numpy(y), y_cf.numpy(), "x0: y = Lambda (S0 . C)")
        for i, c in enumerate(cks):
            assert_close(c, S_start[i + 1].numpy(), f"x0: S_L = Lambda_L S0 after interval {i}")
    elif case == "orth":
        y_cf = Dd[None, None, :, None] * xd
        assert_close(torch.from_numpy(y), y_cf.numpy(), "orth: y = D x")
