"""Pins of the oracle's speculative round and its position bookkeeping.

Article section 3 ("Roll back incorrect predictions using buffer
positions"): verification produces the outputs of all draft positions with no
intermediate states, and only positions up to the last accepted token count;
rejected drafts need no restore.  The pins compare the oracle's round with
plain sequential decoding of the accepted prefix and check that rejected
contents leave no trace.
"""
import numpy as np
import pytest

import oracle

rng = np.random.default_rng(99)


def _inputs(T, batch, H, G, P, N):
    S0 = rng.normal(0, 0.3, (batch, H, P, N))
    x = rng.normal(0, 1, (T, batch, H, P))
    Bm = rng.normal(0, 1, (T, batch, G, N))
    Cm = rng.normal(0, 1, (T, batch, G, N))
    dt = rng.uniform(0.01, 0.5, (T, batch, H))
    A = -rng.uniform(1, 8, H)
    D = rng.normal(0, 1, H)
    return S0, x, Bm, Cm, dt, A, D


@pytest.mark.parametrize("keep", [0, 1, 3, 5])
def test_round_equals_sequential_prefix(keep):
    T, batch, H, G, P, N = 5, 3, 4, 2, 3, 4
    S0, x, Bm, Cm, dt, A, D = _inputs(T, batch, H, G, P, N)
    nk = np.full(batch, keep, dtype=np.int32)
    S, y = oracle.spec_round(S0, x, Bm, Cm, dt, A, D, nk, G)
    # outputs of all T positions == sequential decoding of all T tokens
    _, yseq = oracle.recurrent(S0, x, Bm, Cm, dt, A, D, G)
    np.testing.assert_array_equal(y, yseq)
    # state == sequential decoding of the accepted prefix only
    if keep == 0:
        np.testing.assert_array_equal(S, S0)
    else:
        Sk, _ = oracle.recurrent(S0, x[:keep], Bm[:keep], Cm[:keep], dt[:keep], A, D, G)
        np.testing.assert_array_equal(S, Sk)


def test_rejected_drafts_leave_no_trace():
    T, batch, H, G, P, N = 5, 4, 2, 1, 3, 4
    S0, x, Bm, Cm, dt, A, D = _inputs(T, batch, H, G, P, N)
    nk = np.array([0, 1, 2, 4], dtype=np.int32)
    S_a, y_a = oracle.spec_round(S0, x, Bm, Cm, dt, A, D, nk, G)
    x2, B2, C2, dt2 = x.copy(), Bm.copy(), Cm.copy(), dt.copy()
    for b, k in enumerate(nk):
        x2[k:, b] = np.nan
        B2[k:, b] = 1e6
        dt2[k:, b] = 3.0
    S_b, y_b = oracle.spec_round(S0, x2, B2, C2, dt2, A, D, nk, G)
    np.testing.assert_array_equal(S_a, S_b)
    for b, k in enumerate(nk):   # causality: accepted outputs unchanged
        np.testing.assert_array_equal(y_a[:k, b], y_b[:k, b])


def test_spec_run_positions_and_commits():
    T, batch, H, G, P, N, R, L = 5, 6, 2, 1, 2, 3, 12, 16
    S0 = rng.normal(0, 0.3, (batch, H, P, N))
    x = rng.normal(0, 1, (R, T, batch, H, P))
    Bm = rng.normal(0, 1, (R, T, batch, G, N))
    Cm = rng.normal(0, 1, (R, T, batch, G, N))
    dt = rng.uniform(0.01, 0.5, (R, T, batch, H))
    A = -rng.uniform(1, 8, H)
    D = rng.normal(0, 1, H)
    nk = rng.integers(0, T + 1, (R, batch)).astype(np.int32)
    out = oracle.spec_run(S0, x, Bm, Cm, dt, A, D, nk, G, L)
    pos = np.zeros(batch, dtype=np.int64)
    total = np.zeros(batch, dtype=np.int64)
    for r in range(R):
        pos = pos + nk[r]
        total += nk[r]
        com = pos >= L
        assert np.array_equal(out["commit"][r], com)
        pos[com] = 0
        assert np.array_equal(out["pos"][r], pos)
        assert np.all(out["pos"][r] < L)
    # final state == sequential decoding of every accepted token in order
    for b in range(batch):
        xs = np.concatenate([x[r, :nk[r, b], b:b + 1] for r in range(R)])
        Bs = np.concatenate([Bm[r, :nk[r, b], b:b + 1] for r in range(R)])
        Cs = np.concatenate([Cm[r, :nk[r, b], b:b + 1] for r in range(R)])
        ds = np.concatenate([dt[r, :nk[r, b], b:b + 1] for r in range(R)])
        Sb, _ = oracle.recurrent(S0[b:b + 1], xs, Bs, Cs, ds, A, D, G)
        np.testing.assert_allclose(out["state"][-1][b:b + 1], Sb, rtol=1e-13, atol=1e-14)
        assert xs.shape[0] == total[b]
