"""The post-build check for wide-store data hazards (state_space_recurrence_amd.isa_check).

A store of more than 64 bits of data reads its data VGPRs after it issues;
LLVM's gfx950 hazard model puts two wait states between such a store and a
VALU write of those VGPRs, except for buffer stores whose scalar offset is a
register.  A build whose last commit store was followed at once by a VALU
write of its data wrote wrong checkpoint rows (the fixture below is that
build's assembly); the kernels now keep store offsets in the vector operand
and the build refuses any object with the pattern.
"""
import glob
import os

import pytest

from state_space_recurrence_amd import isa_check

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "commit_store_hazard.s")


def _one(body: str) -> str:
    return "_Zkern:\n" + "\n".join("\t" + l for l in body.strip().splitlines()) + "\n"


def test_flags_the_failing_build():
    hits = isa_check.scan(open(GOLDEN).read())
    assert len(hits) == 1, hits
    fn, _, store, offender = hits[0]
    assert "replay_step_kernel" in fn
    assert store.startswith("buffer_store_dwordx4 v[2:5]") and "s0" in store
    assert offender.startswith("v_and_b32_e32 v2")


@pytest.mark.parametrize("body, flagged", [
    # the data VGPRs overwritten at zero and at one wait state
    ("buffer_store_dwordx4 v[2:5], v1, s[4:7], s8 offen nt\nv_mov_b32_e32 v3, 0", True),
    ("buffer_store_dwordx4 v[2:5], v1, s[4:7], s8 offen nt\ns_movk_i32 s0, 0x10\nv_mov_b32_e32 v5, 0", True),
    ("buffer_store_dwordx4 v[2:5], v1, s[4:7], s8 offen nt\ns_nop 0\nv_mov_b32_e32 v5, 0", True),
    ("global_store_dwordx4 v1, v[10:13], s[0:1] nt\nv_add_f32_e32 v11, v1, v2", True),
    ("buffer_store_dwordx3 v[2:4], v1, s[4:7], 0 offen\nv_mov_b32_e32 v4, 0", True),
    # two wait states, other registers, the address operand, 64-bit data
    ("buffer_store_dwordx4 v[2:5], v1, s[4:7], s8 offen nt\ns_nop 1\nv_mov_b32_e32 v5, 0", False),
    ("buffer_store_dwordx4 v[2:5], v1, s[4:7], s8 offen nt\ns_mov_b32 s0, 1\ns_mov_b32 s1, 1\nv_mov_b32_e32 v2, 0",
     False),
    ("buffer_store_dwordx4 v[2:5], v1, s[4:7], s8 offen nt\nv_mov_b32_e32 v6, 0\nv_mov_b32_e32 v1, 0", False),
    ("global_store_dwordx4 v1, v[10:13], s[0:1]\nv_mov_b32_e32 v1, 0", False),
    ("buffer_store_dwordx2 v[2:3], v1, s[4:7], s8 offen\nv_mov_b32_e32 v2, 0", False),
    # objdump form, with '//' encodings
    ("buffer_store_dwordx4 v[46:49], v58, s[28:31], s4 offen nt  // 00000002BD58: E07E1000 04072E3A\n"
     "v_mov_b32_e32 v47, 0  // 00000002BD60: 7E5E0280", True),
])
def test_scan_rules(body, flagged):
    assert bool(isa_check.scan(_one(body))) == flagged


def test_built_objects_are_clean():
    """The device code of the built library has no such hazard (the build
    runs the same check and refuses to link otherwise)."""
    objs = sorted(glob.glob(os.path.join(os.path.dirname(isa_check.__file__), "_build", "*.hip.o")))
    if not objs:
        pytest.skip("library not built")
    assert isa_check.check_objects(objs) > 1000   # the step, commit, prefill and split stores are all seen
