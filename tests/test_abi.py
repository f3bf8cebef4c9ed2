"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "replayssm.h")


@pytest.fixture(scope="module")
def rs():
    import state_space_recurrence_amd as rs
    if not os.path.exists(rs.LIB_PATH):
        from state_space_recurrence_amd import build
        build.build()
    rs.lib()
    return rs


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(replayssm_\w+)\s*\(", src)))


def test_header_declares_the_calls():
    names = _declared()
    for n in ("replayssm_step", "replayssm_verify", "replayssm_accept", "replayssm_commit",
              "replayssm_recurrent_step"):
        assert n in names


def test_every_declared_symbol_is_exported(rs):
    L = rs.lib()
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing, missing


def _desc(rs, **kw):
    d = dict(batch=4, heads=8, head_dim=64, d_state=128, groups=1, interval=16, max_draft=1,
             in_dtype=rs.F32)
    d.update(kw)
    return rs._make_desc(d["batch"], d["heads"], d["head_dim"], d["d_state"], d["groups"],
                         d["interval"], d["max_draft"], d["in_dtype"],
                         ckpt_dtype=d.get("ckpt_dtype", rs.F32), out_dtype=d.get("out_dtype", rs.NONE),
                         shared_lowp=d.get("shared_lowp", 0), deferred_commit=d.get("deferred_commit", 0))


@pytest.mark.parametrize("kw,code", [
    ({}, 0),
    ({"head_dim": 32}, -2),
    ({"d_state": 64}, -2),
    ({"heads": 6, "groups": 4}, -1),
    ({"groups": 0}, -1),
    ({"batch": -1}, -1),
    ({"interval": 0}, -1),
    ({"max_draft": 0}, -3),
    ({"max_draft": 9}, -3),
    ({"interval": 30, "max_draft": 4}, 0),       # Lcap 33: step / flush only
    ({"interval": 64, "max_draft": 1}, 0),
    ({"interval": 62, "max_draft": 4}, -3),      # Lcap 65
    ({"interval": 30, "max_draft": 4, "ckpt_dtype": 1, "out_dtype": 3}, -3),
    ({"in_dtype": 2}, -2),
    ({"shared_lowp": 2}, -1),
    ({"deferred_commit": 1, "max_draft": 5}, 0),
    ({"deferred_commit": 2, "max_draft": 5}, -1),
    ({"deferred_commit": 1, "max_draft": 1}, -2),
    ({"deferred_commit": 1, "max_draft": 5, "ckpt_dtype": 1, "out_dtype": 3}, -2),
    ({"deferred_commit": 1, "max_draft": 5, "interval": 28}, -3),
    # low-precision states: the flat element index must fit 32 bits
    ({"batch": 32767, "heads": 16, "groups": 2, "ckpt_dtype": 1, "out_dtype": 3}, 0),
    ({"batch": 32768, "heads": 16, "groups": 2, "ckpt_dtype": 1, "out_dtype": 3}, -1),
    ({"batch": 32768, "heads": 16, "groups": 2}, 0),                # fp32 checkpoint: no rounding stream
])
def test_descriptor_validation(rs, kw, code):
    L = rs.lib()
    d = _desc(rs, **kw)
    assert L.replayssm_check_desc(ctypes.byref(d)) == code
    if code:
        assert L.replayssm_last_error().decode()


def test_null_arguments_rejected_before_launch(rs):
    L = rs.lib()
    d = _desc(rs)
    st = rs.RssmState()
    assert L.replayssm_step(None, ctypes.byref(st), None, None, None, None, None, None) == -1
    assert L.replayssm_step(ctypes.byref(d), None, None, None, None, None, None, None) == -1
    assert L.replayssm_step(ctypes.byref(d), ctypes.byref(st), None, None, None, None, None, None) == -1
    assert "ckpt" in L.replayssm_last_error().decode()
    assert L.replayssm_commit(ctypes.byref(d), ctypes.byref(st), None) == -1
    assert L.replayssm_recurrent_step(ctypes.byref(d), None, None, None, None, None, None, None, None,
                                      None) == -1


def test_draft_count_checked(rs):
    L = rs.lib()
    d = _desc(rs, max_draft=5)
    st = rs.RssmState()
    assert L.replayssm_verify(ctypes.byref(d), ctypes.byref(st), 6, None, None, None, None, None, None) == -3
    assert L.replayssm_verify(ctypes.byref(d), ctypes.byref(st), 0, None, None, None, None, None, None) == -3
    d = _desc(rs, interval=30, max_draft=4)      # verify is built for Lcap <= 32
    assert L.replayssm_verify(ctypes.byref(d), ctypes.byref(st), 2, None, None, None, None, None, None) == -3
    assert L.replayssm_accept(ctypes.byref(d), ctypes.byref(st), None, 9, None) == -3
    assert L.replayssm_accept_deferred(ctypes.byref(d), ctypes.byref(st), None, 6, None) == -3
    assert L.replayssm_recurrent_accept(ctypes.byref(d), None, None, 7, None) == -3


def test_deferred_accept_needs_the_declaration(rs):
    """replayssm_accept_deferred is refused on the host unless the descriptor
    declares deferred commits (which is itself limited to F32 checkpoints
    and speculative rounds, see test_descriptor_validation)."""
    L = rs.lib()
    st = rs.RssmState()
    d = _desc(rs, max_draft=5)
    assert L.replayssm_accept_deferred(ctypes.byref(d), ctypes.byref(st), None, 5, None) == -1
    assert "deferred_commit" in L.replayssm_last_error().decode()
    d = _desc(rs, max_draft=5, deferred_commit=1)
    assert L.replayssm_accept_deferred(ctypes.byref(d), ctypes.byref(st), None, 5, None) == -1
    assert "state" in L.replayssm_last_error().decode()


def test_prefill_arguments_checked(rs):
    L = rs.lib()
    st = rs.RssmState()
    d = _desc(rs)
    assert L.replayssm_prefill(ctypes.byref(d), ctypes.byref(st), -1, 0, None, None, None, None, None, None) == -1
    assert L.replayssm_prefill(ctypes.byref(d), ctypes.byref(st), 4, 2, None, None, None, None, None, None) == -1
    # a low-precision state is accepted (the missing state buffers are what is refused)
    d = _desc(rs, ckpt_dtype=rs.BF16, out_dtype=rs.FP4_E2M1)
    assert L.replayssm_prefill(ctypes.byref(d), ctypes.byref(st), 4, 0, None, None, None, None, None, None) == -1
    assert "state" in L.replayssm_last_error().decode()
    d = _desc(rs, batch=0)
    assert L.replayssm_prefill(ctypes.byref(d), ctypes.byref(st), 4, 0, None, None, None, None, None, None) == 0


def test_slot_map_arguments_checked(rs):
    """Without a slot map the call's rows are slots 0..batch-1, so batch may
    not exceed n_slots; with one, any row count is allowed."""
    L = rs.lib()
    st = rs.RssmState(*([1] * 11))          # non-NULL placeholders, no launch happens on error
    d = _desc(rs, batch=6)
    d.n_slots = 4
    assert L.replayssm_step(ctypes.byref(d), ctypes.byref(st), None, None, None, None, None, None) == -1
    assert "n_slots" in L.replayssm_last_error().decode()
    d.n_slots = -2
    assert L.replayssm_check_desc(ctypes.byref(d)) == -1


def test_empty_batch_is_a_noop_without_device(rs):
    L = rs.lib()
    d = _desc(rs, batch=0)
    st = rs.RssmState()
    assert L.replayssm_step(ctypes.byref(d), ctypes.byref(st), None, None, None, None, None, None) == 0
    assert L.replayssm_commit(ctypes.byref(d), ctypes.byref(st), None) == 0


def test_buffer_capacity_and_strings(rs):
    L = rs.lib()
    assert L.replayssm_buffer_capacity(ctypes.byref(_desc(rs, interval=16, max_draft=5))) == 20
    assert L.replayssm_buffer_capacity(ctypes.byref(_desc(rs, head_dim=7))) == 0
    for code in (0, -1, -2, -3, -4, -5):
        assert L.replayssm_status_string(code)
    assert L.replayssm_version().decode().startswith("replayssm")


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import state_space_recurrence_amd as rs
    monkeypatch.setattr(rs, "_LIB", None)
    monkeypatch.setattr(rs, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(rs.ReplaySSMError, match="missing"):
        rs.lib()


def test_conversion_check_arguments_checked(rs):
    """The conversion self-check refuses a NULL counter array and a range
    outside 0..2^32 on the host, before any launch."""
    L = rs.lib()
    assert L.replayssm_check_conversions(0, 16, None, None) == -1
    assert "counts" in L.replayssm_last_error().decode()
    buf = (ctypes.c_uint64 * 2)()
    assert L.replayssm_check_conversions(8, 4, buf, None) == -1
    assert L.replayssm_check_conversions(0, (1 << 32) + 1, buf, None) == -1
