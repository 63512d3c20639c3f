"""Build libfs.so (HIP, gfx950) in-tree with hipcc.

    python -m lm_head_gumbel_amd.build          # build (always recompiles)
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfs.so")
SOURCES = ["fs_api.hip", "fs_plan.cpp", "fs_stage1.hip", "fs_stream.hip", "fs_resident.hip", "fs_wide.hip",
           "fs_rows.hip", "fs_stage2.hip", "fs_probe.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


# Extra device-compiler flags per source.  fs_resident.hip: no wave-level
# rewriting of atomics (it would read the ticket back at once, waiting for
# every load in flight; the kernel uses it only after the contraction).
EXTRA_FLAGS = {"fs_resident.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


# Sources whose kernels issue untracked loads from inline assembly and count
# their waits by hand: the build also emits their assembly and proves that the
# compiler touches no register of such a load before a wait retires it
# (isa_check.py); a failure stops the build.
ISA_CHECKED = ["fs_rows.hip"]


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # no packed-FP32 instructions in device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def compile_commands(objdir):
    """(source, object, command) per source file."""
    out = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        if src.endswith(".cpp"):   # host-only C++ (no device code)
            cmd = [hipcc(), "-O2", "-std=c++17", "-fPIC", "-Wall", "-x", "c++",
                   "-I", os.path.join(ROOT, "include"), "-I", CSRC]
        else:
            cmd = [hipcc()] + common_flags() + EXTRA_FLAGS.get(src, [])
        cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
        out.append((src, obj, cmd))
    return out


def build(verbose=False):
    """Compile every HIP source (in parallel) and link libfs.so next to this
    file (atomic replace)."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    tmp = LIB + ".tmp%d" % os.getpid()
    with tempfile.TemporaryDirectory(prefix="fs_build_") as objdir:
        jobs = compile_commands(objdir)

        def run(job):
            src, obj, cmd = job
            if verbose:
                print(" ".join(cmd), flush=True)
            return src, subprocess.run(cmd, capture_output=True, text=True)

        asm_jobs = []
        for src in ISA_CHECKED:
            out = os.path.join(objdir, os.path.splitext(src)[0] + ".s")
            cmd = [hipcc()] + common_flags() + EXTRA_FLAGS.get(src, []) + \
                ["--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
            asm_jobs.append((src + " (assembly)", out, cmd))

        workers = max(1, min(len(jobs) + len(asm_jobs), os.cpu_count() or 1, 8))
        with ThreadPoolExecutor(workers) as ex:
            results = list(ex.map(run, jobs + asm_jobs))
        failed = [(src, r) for src, r in results if r.returncode != 0]
        for src, r in failed:
            sys.stderr.write(f"--- {src}\n" + r.stdout + r.stderr)
        if failed:
            raise RuntimeError("hipcc failed building libfs.so: " + ", ".join(s for s, _ in failed))
        from . import isa_check
        for src, out, _ in asm_jobs:
            with open(out) as f:
                errors = isa_check.check_text(f.read(), require_untracked=True)
            if errors:
                sys.stderr.write("\n".join(errors[:20]) + "\n")
                raise RuntimeError("%s: %d register(s) of untracked loads touched in flight"
                                   % (src, len(errors)))
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + \
            [obj for _, obj, _ in jobs]
        if verbose:
            print(" ".join(link), flush=True)
        res = subprocess.run(link, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError("hipcc failed linking libfs.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
