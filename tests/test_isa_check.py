"""The build-time check of untracked loads (lm_head_gumbel_amd/isa_check.py):
pinned on small hand-written listings whose verdict is known, then run on the
assembly hipcc emits for the row-streaming kernels."""
import os
import re
import shutil
import subprocess

import pytest

from lm_head_gumbel_amd import isa_check
from lm_head_gumbel_amd import build as fs_build

HEAD = "_Zk:\n"
TAIL = "\ts_endpgm\n.Lfunc_end0:\n"


def untracked(dst, addr):
    return "\t;;#ASMSTART\n\tglobal_load_dwordx4 %s, %s, off\n\t;;#ASMEND\n" % (dst, addr)


def errors(body):
    return isa_check.check_text(HEAD + body + TAIL)


def test_use_after_counted_wait_is_clean():
    body = (untracked("v[4:7]", "v[0:1]") + untracked("v[8:11]", "v[2:3]")
            + "\ts_waitcnt vmcnt(1)\n\tv_mov_b32 v20, v4\n"
            + "\ts_waitcnt vmcnt(0)\n\tv_mov_b32 v21, v8\n")
    assert errors(body) == []


def test_use_before_wait_is_caught():
    body = untracked("v[4:7]", "v[0:1]") + "\tv_mov_b32 v20, v5\n\ts_waitcnt vmcnt(0)\n"
    assert len(errors(body)) == 1


def test_wait_counting_too_few_loads_is_caught():
    # vmcnt(1) leaves the younger load in flight
    body = (untracked("v[4:7]", "v[0:1]") + untracked("v[8:11]", "v[2:3]")
            + "\ts_waitcnt vmcnt(1)\n\tv_mov_b32 v21, v8\n\ts_waitcnt vmcnt(0)\n")
    assert len(errors(body)) == 1


def test_spill_of_register_in_flight_is_caught():
    body = (untracked("v[4:7]", "v[0:1]")
            + "\tscratch_store_dwordx4 off, v[4:7], off\n\ts_waitcnt vmcnt(0)\n")
    assert len(errors(body)) == 1


def test_redefinition_in_flight_is_caught():
    body = (untracked("v[4:7]", "v[0:1]") + "\tv_mov_b32 v6, 0\n\ts_waitcnt vmcnt(0)\n")
    assert len(errors(body)) == 1


def test_stores_do_not_retire_loads():
    # a younger store may complete first: vmcnt(1) does not prove the load done
    body = (untracked("v[4:7]", "v[0:1]") + "\tglobal_store_dword v[2:3], v9, off\n"
            + "\ts_waitcnt vmcnt(1)\n\tv_mov_b32 v20, v4\n\ts_waitcnt vmcnt(0)\n")
    assert len(errors(body)) == 1


def test_tracked_loads_count_as_younger():
    body = (untracked("v[4:7]", "v[0:1]") + "\tglobal_load_dword v9, v[2:3], off\n"
            + "\ts_waitcnt vmcnt(1)\n\tv_mov_b32 v20, v4\n\ts_waitcnt vmcnt(0)\n")
    assert errors(body) == []


def test_loop_back_edge_carries_loads():
    # the load issued at the bottom of the loop is used at its top before any wait
    body = ("\ts_mov_b32 s0, 4\n" + untracked("v[4:7]", "v[0:1]")
            + ".LBB0_1:\n\tv_add_f32 v20, v4, v20\n" + untracked("v[4:7]", "v[0:1]")
            + "\ts_sub_u32 s0, s0, 1\n\ts_cbranch_scc1 .LBB0_1\n\ts_waitcnt vmcnt(0)\n")
    assert len(errors(body)) >= 1
    fixed = body.replace(".LBB0_1:\n", ".LBB0_1:\n\ts_waitcnt vmcnt(0)\n")
    assert errors(fixed) == []


def test_merge_takes_the_weaker_path():
    # one path issues a younger load, the other does not: vmcnt(1) is not enough
    body = (untracked("v[4:7]", "v[0:1]") + "\ts_cbranch_scc1 .LBB0_2\n"
            + "\tglobal_load_dword v9, v[2:3], off\n.LBB0_2:\n"
            + "\ts_waitcnt vmcnt(1)\n\tv_mov_b32 v20, v4\n\ts_waitcnt vmcnt(0)\n")
    assert len(errors(body)) == 1


def test_flat_and_calls_are_rejected():
    assert errors("\tflat_load_dword v1, v[2:3]\n\ts_waitcnt vmcnt(0) lgkmcnt(0)\n")
    assert errors("\ts_swappc_b64 s[30:31], s[4:5]\n")


def test_vacuous_listing_is_rejected():
    assert isa_check.check_text(HEAD + "\tv_mov_b32 v1, 0\n" + TAIL, require_untracked=True)


def _hipcc():
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not installed")
def test_rows_kernels_pass(tmp_path):
    out = tmp_path / "rows.s"
    cmd = [_hipcc()] + fs_build.common_flags() + [
        "--cuda-device-only", "-S", os.path.join(fs_build.CSRC, "fs_rows.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    text = out.read_text()
    assert isa_check.check_text(text, require_untracked=True) == []
    # every instantiation was analysed (3 shapes x lean flat, general flat,
    # logits; grouped at 64 and 128 columns), and no loop that issues MFMAs
    # spills: a reload there would bring a compiler wait for every load in
    # flight
    funcs = isa_check._functions(text.splitlines())
    assert len(funcs) == 11, [n for n, _ in funcs]
    assert mfma_loop_spills(text) == []


def mfma_loop_spills(text):
    """Scratch instructions in blocks of loops (by the compiler's loop
    annotations) that contain an MFMA."""
    block, loop_of, ops = None, {}, []
    for line in text.splitlines():
        m = re.match(r"^\.(LBB\d+_\d+):(.*)", line)
        if m:
            block = m.group(1)
            h = re.search(r"Header=(BB\d+_\d+)", m.group(2))
            # a loop is named by its header block (BBx_y, the label without ".L")
            loop_of[block] = h.group(1) if h else (block[1:] if "Loop Header" in m.group(2) else None)
            continue
        t = line.strip()
        if t and block is not None and not t.startswith((";", ".")):
            ops.append((block, t.split()[0]))
    mfma_loops = {loop_of[b] for b, op in ops if op.startswith("v_mfma") and loop_of.get(b)}
    return [(b, op) for b, op in ops if op.startswith("scratch_") and loop_of.get(b) in mfma_loops]


def test_long_jumps_are_branches():
    jump = ("\ts_getpc_b64 s[98:99]\n.Lpost_getpc0:\n"
            "\ts_add_u32 s98, s98, (.LBB0_2-.Lpost_getpc0)&4294967295\n"
            "\ts_addc_u32 s99, s99, (.LBB0_2-.Lpost_getpc0)>>32\n\ts_setpc_b64 s[98:99]\n")
    # the block skipped by the jump is never reached: its early use is no error
    body = (untracked("v[4:7]", "v[0:1]") + jump + ".LBB0_1:\n\tv_mov_b32 v20, v4\n"
            + ".LBB0_2:\n\ts_waitcnt vmcnt(0)\n\tv_mov_b32 v21, v4\n")
    assert errors(body) == []
    # the jump target's use before the wait is
    bad = body.replace(".LBB0_2:\n", ".LBB0_2:\n\tv_mov_b32 v22, v5\n")
    assert len(errors(bad)) == 1
