"""Host-side checks of the library's launch planning and workspace layout
(lm_head_gumbel_amd/csrc/fs_plan.cpp, plain C++ with no HIP), built here on
the CPU with address and undefined-behaviour sanitizers.  The check program
plans every variant over a grid of shapes, extreme ones included (B up to
2^20, d up to 2^20, V and v_offset + V at the int32 limit, 16-row tiles,
k = 1024 with the largest candidate lists), on 1 to 304 compute units, and
verifies the plans' invariants and that every workspace array is aligned,
in bounds and disjoint.  Integer overflow or an out-of-bounds access in the
size arithmetic stops it with a sanitizer report."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lm_head_gumbel_amd", "csrc")


@pytest.fixture(scope="module")
def plan_check(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("plan") / "plan_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "fs_plan.cpp"), os.path.join(ROOT, "tests", "helpers", "plan_check.cpp"),
           "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def test_plans_and_layouts_under_sanitizers(plan_check):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([plan_check], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    last = r.stdout.strip().splitlines()[-1]
    assert last.startswith("ok "), last
    assert int(last.split()[1]) > 100000
    plans = {}
    for line in r.stdout.splitlines():
        if line.startswith("plan "):
            f = line.split()
            kv = dict(x.split("=") for x in f[2:])
            plans[(f[1], int(kv["var"]))] = kv
    # the headline call: the register-resident kernel, one workgroup per CU,
    # last units by ticket; the largest batch: the 256-column row-streaming kernel
    h = plans[("headline_b32", 0)]
    assert (h["kind"], h["G"], h["grid_y"], h["rcfg"]) == ("2", "256", "1", "2,1,4,8,16,0")
    assert int(h["dyn_k0"]) == 9496 // 256 - 2
    # grouped on the resident kernel: a record per 16-row unit, strided and
    # ticket order like flat
    g = plans[("headline_b32", 1)]
    assert (g["unit_rec"], g["P"], g["dyn_k0"]) == ("1", "9496", h["dyn_k0"])
    assert plans[("mid_b64", 1)]["unit_rec"] == "1"            # block records from the rows kernel
    sw = plans[("sweep_b256", 0)]   # one group of 256 columns, a workgroup per CU
    assert (sw["kind"], sw["nt"], sw["grid_y"], sw["G"]) == ("4", "256", "1", "256")
    assert plans[("sweep_b128", 0)]["nt"] == "128"
    assert plans[("mid_b64", 1)]["kind"] == "4"               # grouped B = 64: the rows kernel
    assert plans[("topk_b32", 3)]["rcfg"] == "2,1,2,8,18,2"   # d = 5120: H partly in LDS
    assert plans[("tiny_b4", 0)]["kind"] == "1"                # d = 256: the streaming kernel
    # the parity cases of the row-streaming kernel reach it, flat and logits,
    # at each column width, with several tiles per range and two column groups
    for name, nt, gy in [("rows_b33", 64, 1), ("rows_b40", 64, 1), ("rows_b100", 128, 1),
                         ("rows_b128", 128, 1), ("rows_b150", 256, 1), ("rows_b256", 256, 1),
                         ("rows_b300", 256, 2)]:
        for var in (0, 2):   # flat, logits
            pl = plans[(name, var)]
            assert (pl["kind"], pl["nt"], pl["grid_y"]) == ("4", str(nt), str(gy)), (name, pl)
    assert plans[("rows_b300", 0)]["xcd"] == "1"
    # grouped on the row-streaming kernel too (block records), at most 128
    # columns per workgroup: larger batches in paired column groups
    for name, nt, gy in [("rows_b33", 64, 1), ("rows_b100", 128, 1), ("rows_b128", 128, 1),
                         ("rows_b200_d512", 128, 2)]:
        pl = plans[(name, 1)]
        assert (pl["kind"], pl["nt"], pl["grid_y"], pl["unit_rec"]) == ("4", str(nt), str(gy), "1"), \
            (name, pl)
    # ranges of 17 or 18 blocks (272 or 288 rows: a 256-row tile and a short
    # one) and of 25 blocks (400 rows: the last tile of 144 rows runs whole)
    assert plans[("rows_b128", 0)]["G"] == "256"
    assert plans[("rows_b256", 0)]["G"] == "256"
    pl = plans[("rows_b100_tail144", 0)]
    assert (pl["kind"], pl["nt"], pl["G"]) == ("4", "128", "256")
