"""Full-size parity in the launch configuration the benchmark times.

The whole workload runs on the GPU (every slot, every layer, every step) and
the fp64 oracle recomputes a seeded sample of slots one by one (slots are
independent, so a sample is exact for those slots).  Bar: every output of
every sampled slot, every step and layer, within 2e-5 * max(1, |y|); the
checkpoint of the sampled slots after the run within the same bar.

Workloads: 4B-class (batch 256, 4 layers, 96 heads, 8 groups, 512 steps),
120B-class (batch 256, 8 layers, 128 heads, 256 steps), speculative
(batch 512, 4 layers, 128 heads, 4 drafts, 200 rounds).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_close, need_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def rs():
    need_gpu()
    import state_space_recurrence_amd as rs
    rs.lib()
    return rs


def _sample(batch, n=3, seed=0):
    g = np.random.default_rng(seed)
    mid = sorted(g.choice(np.arange(1, batch - 1), size=n - 2, replace=False).tolist())
    return [0] + mid + [batch - 1]


@pytest.mark.parametrize("name", ["4b", "120b"])
def test_standard_decode_full_size(rs, name):
    w = synth.WORKLOADS[name]
    dev = torch.device("cuda")
    slots = _sample(w.batch, 3, seed=w.seed)
    print(f"[fullsize] {w.describe()} steps={w.steps} slots={slots}", flush=True)
    for layer in range(w.layers):
        A, D = synth.layer_params(w, layer, device=dev)
        S0 = synth.init_state(w, layer, device=dev)
        x, Bm, Cm, dt = synth.token_inputs(w, layer, w.steps, device=dev)
        ls = rs.LayerState(w.batch, w.heads, w.groups, A, D, interval=w.interval,
                           in_dtype=x.dtype, device=dev, layer_id=layer)
        rs.load_checkpoint(ls, S0)
        y = torch.empty(w.steps, w.batch, w.heads, 64, device=dev)
        for t in range(w.steps):
            rs.step(ls, x[t], Bm[t], Cm[t], dt[t], y=y[t])
        rs.check_device_errors(ls)
        sl = torch.tensor(slots, device=dev)
        ck = ls.ckpt[sl].cpu()
        y_s = y[:, sl].cpu()
        ins = [t[:, sl].cpu() for t in (x, Bm, Cm, dt)]
        S0s = S0[sl].cpu()
        del x, Bm, Cm, dt, y, ls
        torch.cuda.empty_cache()
        y_ref, cks = oracle.decode_run(S0s, *ins, A.cpu(), D.cpu(), w.groups, w.interval)
        assert_close(y_s, y_ref, f"{name} layer {layer} outputs (all steps, sampled slots)")
        assert_close(ck, cks[-1], f"{name} layer {layer} final checkpoint")


def test_speculative_full_size(rs):
    w = synth.WORKLOADS["spec"]
    T = w.drafts + 1
    dev = torch.device("cuda")
    slots = _sample(w.batch, 3, seed=w.seed)
    R = w.rounds
    nk = synth.n_keep(w, R, device=dev)
    print(f"[fullsize] {w.describe()} rounds={R} T={T} slots={slots}", flush=True)
    for layer in range(w.layers):
        A, D = synth.layer_params(w, layer, device=dev)
        S0 = synth.init_state(w, layer, device=dev)
        ls = rs.LayerState(w.batch, w.heads, w.groups, A, D, interval=w.interval, max_draft=T,
                           in_dtype=torch.bfloat16, device=dev, layer_id=layer)
        rs.load_checkpoint(ls, S0)
        sl = torch.tensor(slots, device=dev)
        ys, ins_s, pos_s = [], [[], [], [], []], []
        chunk = 25   # rounds of inputs generated at a time
        for r0 in range(0, R, chunk):
            x, Bm, Cm, dt = synth.token_inputs(w, layer, chunk, device=dev, tokens=T, stream=r0)
            bt = lambda t: t.transpose(1, 2).contiguous()   # [R,T,B,..] -> [R,B,T,..]
            xb, Bb, Cb, db = bt(x), bt(Bm), bt(Cm), bt(dt)
            for i in range(chunk):
                y = rs.verify(ls, xb[i], Bb[i], Cb[i], db[i])
                rs.accept(ls, nk[r0 + i].contiguous(), T)
                ys.append(y[sl].cpu())
                pos_s.append(ls.pos[sl].cpu())
            for k, t in enumerate((x, Bm, Cm, dt)):
                ins_s[k].append(t[:, :, sl].cpu())
            del x, Bm, Cm, dt, xb, Bb, Cb, db
        rs.check_device_errors(ls)
        rs.commit(ls)
        ck = ls.ckpt[sl].cpu()
        del ls
        torch.cuda.empty_cache()
        ins = [torch.cat(v) for v in ins_s]
        ref = oracle.spec_run(S0[sl].cpu(), *ins, A.cpu(), D.cpu(), nk[:, sl].cpu().numpy(),
                              w.groups, w.interval, keep_states=False)
        y_gpu = torch.stack(ys).transpose(1, 2)   # [R,T,b,H,P]
        assert_close(y_gpu, ref["y"], f"spec layer {layer} verify outputs (all rounds)")
        assert np.array_equal(torch.stack(pos_s).numpy(), ref["pos"]), f"layer {layer} positions"
        assert_close(ck, ref["state"][-1], f"spec layer {layer} flushed state")
