"""The benchmark's algorithmic byte model, checked against a brute-force
enumeration of what each call moves.

The roofline figures divide these byte counts by measured kernel time, so
they are pinned here independently: the closed forms in bench.py average
over the buffer positions of an interval, while the enumeration below walks
the positions one step at a time and lists every tensor a step (or verify)
reads and writes, straight from the data layout (fp32 checkpoint of H x P x
N, buffer entries of x [H, P], B [G, N], dt [H] in the input dtype, fp32
outputs).  Also: bench.py refuses more than one GPU before touching any.
"""
import subprocess
import sys

import pytest

import bench

P, N = 64, 128


def _entry(H, G, ib):
    return (H * P + G * N + H) * ib          # one buffered token: x, B, dt


def _inputs(H, G, ib):
    return (H * P + 2 * G * N + H) * ib      # one token's x, B, C, dt


def _step_bytes(H, G, L, k, ib=2, sb=4):
    """One decode step of one slot in one layer at buffer position k."""
    moved = H * P * N * sb                   # the checkpoint is read every step
    moved += _inputs(H, G, ib)               # the current token's inputs
    moved += k * _entry(H, G, ib)            # the k buffered entries are replayed
    moved += H * P * 4                       # y, fp32
    if k == L - 1:
        moved += H * P * N * sb              # the interval closes: the checkpoint is rewritten
    else:
        moved += _entry(H, G, ib)            # otherwise the token is appended
    return moved


@pytest.mark.parametrize("H,G,L", [(96, 8, 16), (128, 8, 16), (8, 1, 16), (96, 8, 4), (96, 8, 64)])
def test_replay_bytes_match_enumeration(H, G, L):
    brute = sum(_step_bytes(H, G, L, k) for k in range(L)) / L
    assert bench.replay_bytes_per_token(H, G, L=L) == pytest.approx(brute, rel=1e-12)


@pytest.mark.parametrize("pos0,steps", [(0, 16), (0, 32), (5, 20), (0, 20), (15, 1), (3, 0)])
def test_window_bytes_count_the_commits_inside(pos0, steps):
    H, G, L = 96, 8, 16
    brute = sum(_step_bytes(H, G, L, (pos0 + i) % L) for i in range(steps))
    assert bench.replay_window_bytes(H, G, L, pos0, steps) == brute
    if pos0 == 0 and steps % L == 0:   # whole intervals: exactly the per-token average
        assert bench.replay_window_bytes(H, G, L, pos0, steps) == pytest.approx(
            steps * bench.replay_bytes_per_token(H, G, L=L), rel=1e-12)


def test_replay_bytes_headline_value():
    # 4B-class layer (H=96, G=8, L=16, bf16 inputs): the per-token figure the
    # roofline uses (x 256 slots = 897,553,408 bytes per launch)
    assert bench.replay_bytes_per_token(96, 8, L=16) == 3_506_068
    assert bench.replay_bytes_per_token(96, 8, L=16) * 256 == 897_553_408


@pytest.mark.parametrize("H,G", [(96, 8), (128, 8)])
def test_recurrent_bytes_match_enumeration(H, G):
    brute = 2 * H * P * N * 4 + _inputs(H, G, 2) + H * P * 4   # state read + written, inputs, y
    assert bench.recurrent_bytes_per_token(H, G) == brute


@pytest.mark.parametrize("T,k", [(5, 0), (5, 9), (5, 15), (1, 3), (8, 7)])
def test_verify_bytes_match_enumeration(T, k):
    H, G = 128, 8
    brute = H * P * N * 4                                    # checkpoint read once, nothing written
    brute += sum(_inputs(H, G, 2) + _entry(H, G, 2) + H * P * 4 for _ in range(T))   # per draft
    brute += k * _entry(H, G, 2)                             # buffered entries replayed
    assert bench.verify_bytes_per_slot(H, G, T, k) == brute


@pytest.mark.parametrize("fmt,out_b,upd_b,write_b", [
    ("split-bf16", 0.5 + 1 / 32, 2, 2 + 0.5 + 1 / 32),       # FP4 copy read; bf16 U read + written, copy written
    ("split-e4m3", 0.5 + 1 / 32, 1, 1 + 0.5 + 1 / 32),
    ("shared-fp4", 0.5 + 1 / 32, 0.5 + 1 / 32, 0.5 + 1 / 32),
    ("low-bf16", 2, 0, 2),                                    # outputs and updates read U
    ("low-e4m3", 1, 0, 1),
])
def test_split_bytes_match_enumeration(fmt, out_b, upd_b, write_b):
    H, G, L = 96, 8, 16
    elems = H * P * N
    total = 0.0
    for k in range(L):
        moved = elems * out_b + _inputs(H, G, 2) + k * _entry(H, G, 2) + H * P * 4
        if k == L - 1:
            moved += elems * (upd_b + write_b)                # the commit reads the update source, writes
        else:
            moved += _entry(H, G, 2)
        total += moved
    assert bench.split_bytes_per_token(fmt, H, G, L=L) == pytest.approx(total / L, rel=1e-12)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=bench.ROOT, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
