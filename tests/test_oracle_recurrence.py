"""Pins of the fp64 oracle's recurrence against results fixed by mathematics.

The recurrence is the conventional SSM decode update the article ("NVIDIA
ReplaySSM: hybrid model SSM decoding with a state buffer", section 1) says
every token performs; ReplaySSM's outputs must equal it within floating-point
error (same section).  None of the checks below re-types the oracle's update:
each compares it with a different closed form or identity, chosen so that a
dropped term, a wrong sign, an off-by-one in which dt decays what, a
pre-update instead of post-update output, a transposed outer product or a
wrong head-to-group map fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle

rng = np.random.default_rng(1234)


def _rand_inputs(steps, batch, H, G, P, N, dt_scale=0.3):
    S0 = rng.normal(0, 0.5, (batch, H, P, N))
    x = rng.normal(0, 1, (steps, batch, H, P))
    Bm = rng.normal(0, 1, (steps, batch, G, N))
    Cm = rng.normal(0, 1, (steps, batch, G, N))
    dt = rng.uniform(0.01, dt_scale, (steps, batch, H))
    A = -rng.uniform(1, 4, H)
    D = rng.normal(0, 1, H)
    return S0, x, Bm, Cm, dt, A, D


def _const_over_time(a, steps):
    return np.broadcast_to(a, (steps,) + a.shape).copy()


@pytest.mark.parametrize("P,N,H,G", [(3, 5, 2, 1), (2, 7, 4, 2), (4, 3, 3, 3)])
def test_closed_form_constant_inputs(P, N, H, G):
    """Constant x, B, C, dt: geometric series.
    S_t = a^t S0 + dt (1 - a^t)/(1 - a) x (outer) B
    y_t = a^t (S0 . C) + dt (1 - a^t)/(1 - a) (B . C) x + D x."""
    steps, batch = 37, 2
    S0, x1, B1, C1, dt1, A, D = _rand_inputs(1, batch, H, G, P, N)
    x = _const_over_time(x1[0], steps)
    Bm = _const_over_time(B1[0], steps)
    Cm = _const_over_time(C1[0], steps)
    dt = _const_over_time(dt1[0], steps)
    S, y = oracle.recurrent(S0, x, Bm, Cm, dt, A, D, G)
    hpg = H // G
    for b in range(batch):
        for h in range(H):
            g = h // hpg
            d = dt1[0, b, h]
            a = math.exp(d * A[h])
            xv, Bv, Cv = x1[0, b, h], B1[0, b, g], C1[0, b, g]
            for t in range(1, steps + 1):
                geo = d * (1 - a ** t) / (1 - a)
                yt = a ** t * (S0[b, h] @ Cv) + geo * (Bv @ Cv) * xv + D[h] * xv
                np.testing.assert_allclose(y[t - 1, b, h], yt, rtol=1e-12, atol=1e-12)
            St = a ** steps * S0[b, h] + d * (1 - a ** steps) / (1 - a) * np.outer(xv, Bv)
            np.testing.assert_allclose(S[b, h], St, rtol=1e-12, atol=1e-12)


def test_closed_form_no_decay():
    """A = 0 gives a = 1: S_t = S0 + t dt x (outer) B."""
    P, N, H, G, steps = 3, 4, 2, 1, 20
    S0, x1, B1, C1, dt1, _, D = _rand_inputs(1, 1, H, G, P, N)
    A = np.zeros(H)
    x, Bm, Cm, dt = (_const_over_time(v[0], steps) for v in (x1, B1, C1, dt1))
    S, y = oracle.recurrent(S0, x, Bm, Cm, dt, A, D, G)
    for h in range(H):
        d = dt1[0, 0, h]
        St = S0[0, h] + steps * d * np.outer(x1[0, 0, h], B1[0, 0, 0])
        np.testing.assert_allclose(S[0, h], St, rtol=1e-12, atol=1e-12)
        y1 = (S0[0, h] + d * np.outer(x1[0, 0, h], B1[0, 0, 0])) @ C1[0, 0, 0] + D[h] * x1[0, 0, h]
        np.testing.assert_allclose(y[0, 0, h], y1, rtol=1e-12, atol=1e-12)


def test_steady_state():
    """Constant inputs, |a| < 1: y -> dt/(1-a) (B . C) x + D x."""
    P, N, H, G, steps = 2, 3, 2, 1, 3000
    S0, x1, B1, C1, dt1, A, D = _rand_inputs(1, 1, H, G, P, N)
    x, Bm, Cm, dt = (_const_over_time(v[0], steps) for v in (x1, B1, C1, dt1))
    _, y = oracle.recurrent(S0, x, Bm, Cm, dt, A, D, G)
    for h in range(H):
        d = dt1[0, 0, h]
        a = math.exp(d * A[h])
        yinf = d / (1 - a) * (B1[0, 0, 0] @ C1[0, 0, 0]) * x1[0, 0, h] + D[h] * x1[0, 0, h]
        np.testing.assert_allclose(y[-1, 0, h], yinf, rtol=1e-10, atol=1e-10)


def test_impulse_response():
    """S0 = 0 and a single nonzero input at token j: for t >= j
    y_t = exp(A sum_{i=j+1..t} dt_i) dt_j (B_j . C_t) x_j  (+ D x_j at t = j),
    and y_t = 0 before j.  The decay of the token's own step is not applied
    to its own input, and the output sees the post-update state."""
    P, N, H, G, steps, j = 3, 4, 2, 1, 12, 5
    _, x, Bm, Cm, dt, A, D = _rand_inputs(steps, 1, H, G, P, N)
    S0 = np.zeros((1, H, P, N))
    x[:] = 0.0
    x[j] = rng.normal(0, 1, x[j].shape)
    _, y = oracle.recurrent(S0, x, Bm, Cm, dt, A, D, G)
    for h in range(H):
        for t in range(steps):
            if t < j:
                exp_y = np.zeros(P)
            else:
                decay = math.exp(A[h] * dt[j + 1:t + 1, 0, h].sum())
                exp_y = decay * dt[j, 0, h] * (Bm[j, 0, 0] @ Cm[t, 0, 0]) * x[j, 0, h]
                if t == j:
                    exp_y = exp_y + D[h] * x[j, 0, h]
            np.testing.assert_allclose(y[t, 0, h], exp_y, rtol=1e-12, atol=1e-13)


def test_zero_dt_is_identity_update():
    """dt = 0: no decay, no input; S stays S0 and y = S0 . C + D x."""
    P, N, H, G, steps = 4, 6, 3, 1, 5
    S0, x, Bm, Cm, dt, A, D = _rand_inputs(steps, 2, H, G, P, N)
    dt[:] = 0.0
    S, y = oracle.recurrent(S0, x, Bm, Cm, dt, A, D, G)
    assert np.array_equal(S, S0)
    for t in range(steps):
        exp_y = np.einsum("bhpn,bn->bhp", S0, Cm[t, :, 0]) + D[None, :, None] * x[t]
        np.testing.assert_allclose(y[t], exp_y, rtol=1e-13, atol=1e-13)


def test_zero_input_is_pure_decay():
    """x = 0: S_t = exp(A sum dt) S0 and y_t = S_t . C_t."""
    P, N, H, G, steps = 3, 5, 2, 1, 9
    S0, x, Bm, Cm, dt, A, D = _rand_inputs(steps, 1, H, G, P, N)
    x[:] = 0.0
    S, y = oracle.recurrent(S0, x, Bm, Cm, dt, A, D, G)
    for h in range(H):
        np.testing.assert_allclose(S[0, h], math.exp(A[h] * dt[:, 0, h].sum()) * S0[0, h],
                                   rtol=1e-12)
        for t in range(steps):
            St = math.exp(A[h] * dt[:t + 1, 0, h].sum()) * S0[0, h]
            np.testing.assert_allclose(y[t, 0, h], St @ Cm[t, 0, 0], rtol=1e-12, atol=1e-14)


def test_contiguous_head_groups():
    """Heads h share the B/C of group h // (H/G): zero group 1's B and C and
    start from S0 = 0; then heads of group 1 output exactly D x."""
    P, N, H, G, steps = 2, 3, 4, 2, 6
    _, x, Bm, Cm, dt, A, D = _rand_inputs(steps, 1, H, G, P, N)
    S0 = np.zeros((1, H, P, N))
    Bm[:, :, 1] = 0.0
    Cm[:, :, 1] = 0.0
    _, y = oracle.recurrent(S0, x, Bm, Cm, dt, A, D, G)
    for h in (2, 3):
        np.testing.assert_array_equal(y[:, 0, h], D[h] * x[:, 0, h])
    for h in (0, 1):
        assert np.abs(y[:, 0, h] - D[h] * x[:, 0, h]).max() > 1e-3


def test_replay_identity():
    """The article's claim that replay from the interval checkpoint plus the
    buffered inputs reproduces the conventional outputs: with
    l_i = A dt_i, Lambda_k = exp(sum_{i<=k} l_i), w_kj = dt_j exp(sum_{j<i<=k} l_i),
      y_k = Lambda_k (S0 . C_k) + sum_{j<=k} w_kj (B_j . C_k) x_j + D x_k
      S_k = Lambda_k S0 + sum_{j<=k} w_kj x_j (outer) B_j."""
    P, N, H, G, steps = 5, 6, 4, 2, 16
    S0, x, Bm, Cm, dt, A, D = _rand_inputs(steps, 2, H, G, P, N, dt_scale=1.0)
    S, y = oracle.recurrent(S0, x, Bm, Cm, dt, A, D, G)
    hpg = H // G
    for b in range(2):
        for h in range(H):
            g = h // hpg
            l = A[h] * dt[:, b, h]
            for k in range(steps):
                Lam = math.exp(l[:k + 1].sum())
                w = np.array([dt[j, b, h] * math.exp(l[j + 1:k + 1].sum()) for j in range(k + 1)])
                gram = Bm[:k + 1, b, g] @ Cm[k, b, g]
                yk = Lam * (S0[b, h] @ Cm[k, b, g]) + (w * gram) @ x[:k + 1, b, h] + D[h] * x[k, b, h]
                np.testing.assert_allclose(y[k, b, h], yk, rtol=1e-11, atol=1e-12)
            Sk = math.exp(l.sum()) * S0[b, h] + sum(
                dt[j, b, h] * math.exp(l[j + 1:].sum()) * np.outer(x[j, b, h], Bm[j, b, g])
                for j in range(steps))
            np.testing.assert_allclose(S[b, h], Sk, rtol=1e-11, atol=1e-12)


def test_mpmath_brute_force_precision():
    """The fp64 evaluation is accurate to ~1e-13 against 50-digit arithmetic
    on tiny shapes over 64 steps (rounding, not formula, is what this checks)."""
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    for (H, P, N) in [(1, 1, 1), (2, 2, 2), (1, 2, 1)]:
        S0, x, Bm, Cm, dt, A, D = _rand_inputs(64, 1, H, 1, P, N)
        _, y = oracle.recurrent(S0, x, Bm, Cm, dt, A, D, 1)
        for h in range(H):
            S = [[mpmath.mpf(S0[0, h, p, n]) for n in range(N)] for p in range(P)]
            for t in range(64):
                d = mpmath.mpf(dt[t, 0, h])
                a = mpmath.exp(d * mpmath.mpf(A[h]))
                for p in range(P):
                    acc = mpmath.mpf(0)
                    for n in range(N):
                        S[p][n] = a * S[p][n] + d * mpmath.mpf(x[t, 0, h, p]) * mpmath.mpf(Bm[t, 0, 0, n])
                        acc += S[p][n] * mpmath.mpf(Cm[t, 0, 0, n])
                    ref = acc + mpmath.mpf(D[h]) * mpmath.mpf(x[t, 0, h, p])
                    assert abs(float(ref) - y[t, 0, h, p]) <= 1e-13 * max(1.0, abs(float(ref)))


def test_decode_run_checkpoints_are_interval_states():
    P, N, H, G, steps, L = 3, 4, 2, 1, 40, 16
    S0, x, Bm, Cm, dt, A, D = _rand_inputs(steps, 2, H, G, P, N)
    y, cks = oracle.decode_run(S0, x, Bm, Cm, dt, A, D, G, L)
    assert len(cks) == 2
    S16, y16 = oracle.recurrent(S0, x[:16], Bm[:16], Cm[:16], dt[:16], A, D, G)
    np.testing.assert_array_equal(cks[0], S16)
    _, yall = oracle.recurrent(S0, x, Bm, Cm, dt, A, D, G)
    np.testing.assert_array_equal(y, yall)
