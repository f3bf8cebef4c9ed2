"""Host model of the fp32 state stream's index maps and the step kernel's LDS.

The step kernel (one wave64 per head, 64 x 128 fp32 = 32 KB) moves the
checkpoint with 16-byte accesses: lane l = 32*hf + c touches columns
4c..4c+3 of rows 2i+hf, i = c' + 4m in chunk c' (m = 0..7), at byte offset
vo + row_offset with vo = (hf*128 + 4c)*4 and row_offset = i * 1024.  Partial
row dots are reduce-scattered across lanes (v_permlane16_swap, DPP
row_mirror / row_half_mirror inside a chunk, quad permutes across the four
chunk values) so that lane (hf, c) ends with row 2c + hf.  Commit
coefficients w_j x_j[r] sit in LDS at cs_index(hf, c', j, m) for row
r = 2(c' + 4m) + hf.  This model checks, without a GPU:

* the stream touches every byte of the head exactly once and stays inside
  it (the scalar row offset is not covered by the buffer range check);
* the reduce-scatter, simulated lane by lane with the documented DPP and
  permlane16_swap semantics, leaves row 2c + hf in lane (hf, c);
* the commit coefficient written for a row (prologue, accept/flush
  prologue) is the one read for that row (commit_chunk_lds), the index is a
  bijection inside the wave's 64*KMAX floats;
* the StepSmem layout (gram, cs, the x-rows / B union) reproduces the LDS
  size the compiler assigned to every replay_step_kernel instance, and the
  accesses of each barrier-separated phase are race-free: no byte written
  by one wave is touched by another wave in the same phase, and the x rows
  are last read one barrier before the B entries overwrite them.
"""
import glob
import os

import numpy as np
import pytest

P, N, WAVE, CHUNKS, PER_CHUNK, MAX_HPW = 64, 128, 64, 4, 8, 4


def chunk_index(c, m):
    return c + 4 * m


def vo(lane):
    hf, c = lane >> 5, lane & 31
    return (hf * N + 4 * c) * 4


def row_offset(c, m):
    return chunk_index(c, m) * 2 * N * 4


def test_stream_covers_the_head_once():
    seen = np.zeros(P * N * 4, dtype=np.int32)
    for ch in range(CHUNKS):
        for m in range(PER_CHUNK):
            for lane in range(WAVE):
                off = vo(lane) + row_offset(ch, m)
                assert 0 <= off and off + 16 <= P * N * 4
                seen[off:off + 16] += 1
                # the bytes are row 2i + hf, columns 4c..4c+3
                i, hf, c = chunk_index(ch, m), lane >> 5, lane & 31
                assert off == ((2 * i + hf) * N + 4 * c) * 4
    assert (seen == 1).all()


# ---- cross-lane operations (wave64) -------------------------------------
def dpp_row_mirror(v):        # lane i <- lane 15 - i within each 16-lane row
    return np.array([v[(l & ~15) | (15 - (l & 15))] for l in range(WAVE)])


def dpp_row_half_mirror(v):   # lane i <- lane 7 - i within each 8 lanes
    return np.array([v[(l & ~7) | (7 - (l & 7))] for l in range(WAVE)])


def dpp_quad_rev(v):          # quad_perm [3,2,1,0]
    return np.array([v[(l & ~3) | (3 - (l & 3))] for l in range(WAVE)])


def dpp_quad_swap1(v):        # quad_perm [1,0,3,2]
    return np.array([v[l ^ 1] for l in range(WAVE)])


def permlane16_swap(a, b):
    """v_permlane16_swap: odd 16-lane rows of the first operand trade places
    with the even rows of the second.  Returns (new first, new second)."""
    a2, b2 = a.copy(), b.copy()
    for l in range(WAVE):
        row = l >> 4
        if row & 1:               # odd row of a <- even row of b (lanes l - 16)
            a2[l] = b[l - 16]
        else:                     # even row of b <- odd row of a (lanes l + 16)
            b2[l] = a[l + 16]
    return a2, b2


def rs_stage(v, op, H, bit):
    up = (np.arange(WAVE) & bit) != 0
    out = [None] * H
    for i in range(H):
        lo = v[i] + op(v[i])
        hi = v[i + H] + op(v[i + H])
        out[i] = np.where(up, hi, lo)
    return out + v[H:]


def chunk_reduce8(v):
    v = list(v)
    for m in range(4):
        a, b = permlane16_swap(v[m], v[m + 4])
        v[m] = a + b
    v = rs_stage(v, dpp_row_mirror, 2, 8)
    v = rs_stage(v, dpp_row_half_mirror, 1, 4)
    return v[0]


def chunk_combine4(r):
    r = rs_stage(list(r), dpp_quad_rev, 2, 2)
    r = rs_stage(r, dpp_quad_swap1, 1, 1)
    return r[0]


def test_reduce_scatter_lands_row_2c_plus_hf():
    # partial of lane l for (chunk ch, slot m) = one-hot code of its row, so
    # the final sum identifies which rows (and how many lanes) reached a lane
    code = lambda row: 1 << row
    r = []
    for ch in range(CHUNKS):
        v = []
        for m in range(PER_CHUNK):
            rows = np.array([2 * chunk_index(ch, m) + (l >> 5) for l in range(WAVE)])
            v.append(np.array([code(int(x)) for x in rows], dtype=object))
        r.append(chunk_reduce8(v))
    tot = chunk_combine4(r)
    for l in range(WAVE):
        row = 2 * (l & 31) + (l >> 5)
        assert tot[l] == 32 * code(row), (l, tot[l])


# ---- commit coefficients -------------------------------------------------
def cs_index(kmax, hf, c, j, m):
    return ((hf * CHUNKS + c) * kmax + j) * PER_CHUNK + m


@pytest.mark.parametrize("kmax", [16, 24, 32, 64])
def test_commit_coefficient_maps_agree(kmax):
    written = {}
    for lane in range(WAVE):
        prow = 2 * (lane & 31) + (lane >> 5)
        i, hf = prow >> 1, prow & 1
        for j in range(kmax):
            # step prologue and accept/flush prologue use the same index for row prow
            idx = cs_index(kmax, hf, i & 3, j, i >> 2)
            assert idx not in written
            written[idx] = (prow, j)
    assert sorted(written) == list(range(P * kmax))
    for lane in range(WAVE):
        hf, c = lane >> 5, lane & 31
        for ch in range(CHUNKS):
            for j in range(kmax):
                for m in range(PER_CHUNK):
                    # commit_chunk_lds applies coefficient m of chunk ch to row 2(ch + 4m) + hf
                    assert written[cs_index(kmax, hf, ch, j, m)] == (2 * chunk_index(ch, m) + hf, j)


# ---- StepSmem layout and phases --------------------------------------------
def step_smem(tin_bytes, kmax):
    """Byte ranges of the step kernel's LDS fields (natural layout, 16-byte
    aligned struct): StepSmem<TIn, KMAX> (gram, coefficient table, x rows and
    fp32 B in a union), or for KMAX = 64 StepSmemX<TIn, KMAX> (gram, x rows,
    then B as stored; no table)."""
    gram = (0, 4 * kmax)
    if kmax == 64:
        u0 = (gram[1] + 15) // 16 * 16
        b0 = u0 + tin_bytes * MAX_HPW * kmax * P
        b1 = b0 + tin_bytes * kmax * N
        size = (b1 + 15) // 16 * 16
        return {"gram": gram, "cs": None, "u": (u0, b0), "B": (b0, b1), "b_bytes": tin_bytes,
                "b_phase": 1, "size": size}
    cs0 = gram[1]
    cs = (cs0, cs0 + 4 * MAX_HPW * P * kmax)
    u0 = (cs[1] + 15) // 16 * 16
    usz = max(tin_bytes * MAX_HPW * kmax * P, 4 * kmax * N)
    size = (u0 + usz + 15) // 16 * 16
    return {"gram": gram, "cs": cs, "u": (u0, u0 + usz), "B": (u0, u0 + 4 * kmax * N), "b_bytes": 4,
            "b_phase": 2, "size": size}


def _phases(tin_bytes, kmax, K, commit):
    """(phase, wave, 'r'|'w', byte start, byte end) of one workgroup's LDS
    accesses in the step prologue and the commit loop.  Phases are separated
    by the prologue's barriers."""
    L = step_smem(tin_bytes, kmax)
    acc = []
    g0, u0 = L["gram"][0], L["u"][0]
    cs0 = L["cs"][0] if L["cs"] else None
    b0, bb, bph = L["B"][0], L["b_bytes"], L["b_phase"]
    xe = 16 // tin_bytes                       # x elements per 16-byte load
    lpr = P // xe                              # lanes per x row
    for w in range(MAX_HPW):
        for lane in range(WAVE):
            t = w * WAVE + lane
            grp, t16 = t >> 4, t & 15
            # phase 0: Gram rows (threads t16 == 0 of groups < K), x rows of entries < K
            if t16 == 0:
                for j in range(grp, K, MAX_HPW * WAVE // 16):
                    acc.append((0, w, "w", g0 + 4 * j, g0 + 4 * j + 4))
            for i in range((kmax + WAVE * xe // P - 1) // (WAVE * xe // P)):
                j = i * (WAVE * xe // P) + lane // lpr
                if i * (WAVE * xe // P) < K and j < K:
                    col = xe * (lane % lpr)
                    a = u0 + ((w * kmax + j) * P + col) * tin_bytes
                    acc.append((0, w, "w", a, a + 16))
            # phase 1: Gram entries, x rows of this head (row prow), coefficients
            prow = 2 * (lane & 31) + (lane >> 5)
            if lane < K:
                acc.append((1, w, "r", g0 + 4 * lane, g0 + 4 * lane + 4))
            for j in range(K):
                a = u0 + ((w * kmax + j) * P + prow) * tin_bytes
                acc.append((1, w, "r", a, a + tin_bytes))
            if commit:
                i, hf = prow >> 1, prow & 1
                if cs0 is not None:
                    for j in range(kmax):
                        a = cs0 + 4 * (w * P * kmax + cs_index(kmax, hf, i & 3, j, i >> 2))
                        acc.append((1, w, "w", a, a + 4))
                # phase b_phase: every thread stages B entries (pieces of 4) -- over the
                # union after a barrier (StepSmem), or into B next to the x rows (StepSmemX)
                for q in range(t, kmax * N // 4, MAX_HPW * WAVE):
                    j, n = q // (N // 4), 4 * (q % (N // 4))
                    a = b0 + bb * (j * N + n)
                    acc.append((bph, w, "w", a, a + 4 * bb))
                # phase 3: commit loop reads B and the coefficients (table, or x rows)
                kr = (K + 3) & ~3
                hf, c = lane >> 5, lane & 31
                for ch in range(CHUNKS):
                    for j in range(kr):
                        a = b0 + bb * (j * N + 4 * c)
                        acc.append((3, w, "r", a, a + 4 * bb))
                        if cs0 is not None:
                            a = cs0 + 4 * (w * P * kmax + cs_index(kmax, hf, ch, j, 0))
                            acc.append((3, w, "r", a, a + 32))
                        else:
                            for m in range(8):
                                row = 2 * (ch + 4 * m) + hf
                                a = u0 + ((w * kmax + j) * P + row) * tin_bytes
                                acc.append((3, w, "r", a, a + tin_bytes))
    return acc, L


@pytest.mark.parametrize("tin_bytes", [2, 4])
@pytest.mark.parametrize("kmax", [16, 32, 64])
def test_step_lds_phases_race_free(tin_bytes, kmax):
    for K, commit in [(1, False), (kmax // 2, False), (kmax - 1, False), (kmax // 2, True), (kmax, True)]:
        acc, L = _phases(tin_bytes, kmax, K, commit)
        for p, w, rw, a, b in acc:
            assert 0 <= a < b <= L["size"], (p, w, rw, a, b)
        for ph in range(4):
            W = np.zeros((MAX_HPW, L["size"]), dtype=np.int32)
            R = np.zeros((MAX_HPW, L["size"]), dtype=bool)
            for p, w, rw, a, b in acc:
                if p == ph:
                    if rw == "w":
                        W[w, a:b] += 1
                    else:
                        R[w, a:b] = True
            for w1 in range(MAX_HPW):
                for w2 in range(MAX_HPW):
                    if w1 != w2:
                        clash = (W[w1] > 0) & ((W[w2] > 0) | R[w2])
                        assert not clash.any(), f"phase {ph}: waves {w1}/{w2} share byte {np.argmax(clash)}"
            if ph == 2 and commit and L["b_phase"] == 2:   # B staging covers the B part of the union once
                cnt = W.sum(0)
                u0, u1 = L["B"]
                assert (cnt[u0:u1] == 1).all() and cnt[:u0].sum() == 0 and cnt[u1:].sum() == 0
            if ph == 1 and commit and L["b_phase"] == 1:   # B staging covers B once, next to the x rows
                cnt = W.sum(0)
                u0, u1 = L["B"]
                assert (cnt[u0:u1] == 1).all() and cnt[u1:].sum() == 0


def _resources():
    from state_space_recurrence_amd import isa_check
    objs = glob.glob(os.path.join(os.path.dirname(isa_check.__file__), "_build", "replay_kernels.hip.o"))
    if not objs:
        pytest.skip("library not built")
    return isa_check.kernel_resources(objs[0])


def test_step_smem_matches_compiled_lds():
    res = _resources()
    for tin, tb in (("t", 2), ("f", 4)):
        for kmax in (16, 32, 64):
            name = f"_ZN4rssm12_GLOBAL__N_118replay_step_kernelI{tin}Li{kmax}EEEvNS_12ReplayParamsE"
            assert res[name]["lds"] == step_smem(tb, kmax)["size"], name
