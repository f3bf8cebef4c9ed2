"""Whole-run drivers of the fp64 oracle -- TEST INFRASTRUCTURE ONLY.

Each driver strings together the plain per-token definition in ``oracle.c``
in the order the article ("NVIDIA ReplaySSM: hybrid model SSM decoding with a
state buffer", devotd.net) describes the method's life cycle:

* standard decoding (sections 1-2): tokens arrive one at a time; the state at
  every interval boundary (every L tokens) is what the checkpoint must hold
  after its once-per-interval rewrite;
* speculative decoding (section 3): rounds of T draft positions, only the
  accepted prefix of each round becomes part of the sequence; the position
  count since the last checkpoint decides when the checkpoint is rewritten.
"""
from __future__ import annotations

import numpy as np

from . import recurrent, spec_round, _f64


def decode_run(S0, x, Bm, Cm, dt, A, D, groups: int, L: int):
    """Standard decoding of ``steps`` tokens from state S0.

    Returns (y [steps, batch, H, P] fp64, checkpoints) where checkpoints[i] is
    the state after (i + 1) * L tokens -- the value the interval checkpoint
    holds once interval i has been committed."""
    steps = x.shape[0]
    S = _f64(S0)
    ys, cks = [], []
    for t0 in range(0, steps, L):
        t1 = min(t0 + L, steps)
        S, y = recurrent(S, x[t0:t1], Bm[t0:t1], Cm[t0:t1], dt[t0:t1], A, D, groups)
        ys.append(y)
        if t1 - t0 == L:
            cks.append(S.copy())
    return np.concatenate(ys, axis=0), cks


def spec_run(S0, x, Bm, Cm, dt, A, D, n_keep, groups: int, L: int, keep_states: bool = True):
    """Speculative decoding over R rounds of T draft positions.

    x [R, T, batch, H, P]; Bm, Cm [R, T, batch, G, N]; dt [R, T, batch, H];
    n_keep [R, batch] in 0..T.

    Positions are counted from the last checkpoint: after round r a slot holds
    pos + n_keep accepted positions; once that count reaches L the checkpoint
    is rewritten to the state after all of them and the count restarts at 0.

    Returns dict with
      y      [R, T, batch, H, P]  outputs of every draft position,
      pos    [R, batch]           position count after each round,
      commit [R, batch]           whether the checkpoint was rewritten,
      state  list of R arrays     true state after each round (fp64); only the
                                  last round's when keep_states is False."""
    R, T, batch = x.shape[0], x.shape[1], x.shape[2]
    n_keep = np.asarray(n_keep, dtype=np.int32)
    S = _f64(S0)
    pos = np.zeros(batch, dtype=np.int64)
    ys, poss, commits, states = [], [], [], []
    for r in range(R):
        S, y = spec_round(S, x[r], Bm[r], Cm[r], dt[r], A, D, n_keep[r], groups)
        pos = pos + n_keep[r]
        c = pos >= L
        pos = np.where(c, 0, pos)
        ys.append(y)
        poss.append(pos.copy())
        commits.append(c)
        if keep_states or r == R - 1:
            states.append(S.copy())
    return {"y": np.stack(ys), "pos": np.stack(poss), "commit": np.stack(commits),
            "state": states}
