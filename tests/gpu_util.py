"""Helpers for the GPU tests: move seeded inputs to the device, call libfs
through its C ABI, and compare the results with the oracle."""
import sys

import numpy as np

import lm_head_gumbel_amd as fs

TOL_GAP = 1e-2      # indices must agree when the oracle's top-two noisy scores differ by more
TOL_VALUE = 2e-3    # per-tile max and log-mass, absolute
TOL_X = 1e-3        # top-k / top-p picks: robust to logit errors up to TOL_X / 2 per id
TOL_MASS = 1e-4     # top-p cut: exclusive masses this far from top_p
MIN_PINNED = 0.9    # full-size tests: at least this fraction of rows compared index for index


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch():
    import torch as _t
    return _t


def dev(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a)).to("cuda")


def dev_bf16(bits):
    return dev(np.ascontiguousarray(bits, np.uint16).view(np.int16))


def host(t):
    return t.detach().cpu().numpy()


def workspace(p, variant, k=0):
    n = fs.fs_workspace_bytes(p, variant, k)
    assert n > 0, "workspace query failed"
    return torch().empty(n, dtype=torch().uint8, device="cuda")


class Inputs:
    """Device copies of one problem (H, W as bf16 bit patterns)."""

    def __init__(self, Hb, Wb, temp=None, allow=None):
        self.B, self.d = Hb.shape
        self.V = Wb.shape[0]
        self.H = dev_bf16(Hb)
        self.W = dev_bf16(Wb)
        self.temp = None if temp is None else dev(np.asarray(temp, np.float32))
        self.allow = None if allow is None else dev(np.asarray(allow, np.uint32).view(np.int32))

    def params(self, **kw):
        return fs.params(self.B, self.d, self.V, **kw)


def run_flat(x, p):
    t = torch()
    idx = t.full((x.B,), -7, dtype=t.int32, device="cuda")
    score = t.full((x.B,), 7.0, dtype=t.float32, device="cuda")
    ws = workspace(p, fs.FS_VARIANT_FLAT)
    fs.check(fs.fs_sample(p, x.H, x.W, x.temp, x.allow, idx, score, ws), "fs_sample")
    t.cuda.synchronize()
    return host(idx).astype(np.int64), host(score).astype(np.float64)


def run_grouped(x, p, with_sample=True):
    t = torch()
    T = fs.fs_num_tiles(p)
    m = t.full((x.B, T), 7.0, dtype=t.float32, device="cuda")
    idx = t.full((x.B, T), -7, dtype=t.int32, device="cuda")
    L = t.full((x.B, T), 7.0, dtype=t.float32, device="cuda")
    out = t.full((x.B,), -7, dtype=t.int32, device="cuda") if with_sample else None
    ws = workspace(p, fs.FS_VARIANT_GROUPED)
    fs.check(fs.fs_sample_grouped(p, x.H, x.W, x.temp, x.allow, m, idx, L, out, ws),
             "fs_sample_grouped")
    t.cuda.synchronize()
    res = [host(m).astype(np.float64), host(idx).astype(np.int64), host(L).astype(np.float64)]
    res.append(host(out).astype(np.int64) if with_sample else None)
    return res


def run_topk(x, p, k):
    t = torch()
    idx = t.full((x.B,), -7, dtype=t.int32, device="cuda")
    ws = workspace(p, fs.FS_VARIANT_TOPK, k)
    fs.check(fs.fs_sample_topk(p, x.H, x.W, x.temp, x.allow, k, idx, ws), "fs_sample_topk")
    t.cuda.synchronize()
    return host(idx).astype(np.int64)


def run_topp(x, p, k, top_p):
    t = torch()
    idx = t.full((x.B,), -7, dtype=t.int32, device="cuda")
    ws = workspace(p, fs.FS_VARIANT_TOPK, k)
    fs.check(fs.fs_sample_topk_topp(p, x.H, x.W, x.temp, x.allow, k, top_p, idx, ws),
             "fs_sample_topk_topp")
    t.cuda.synchronize()
    return host(idx).astype(np.int64)


# top-p cut pinned when every exclusive mass next to the cut is this far from
# top_p: the GPU's masses come from FP32 x (relative error ~1e-6 each), the
# oracle's from float64 logits
TOL_CUT = 1e-4


def run_logits(x, p):
    t = torch()
    out = t.full((x.B, x.V), 7.0, dtype=t.float32, device="cuda")
    ws = workspace(p, fs.FS_VARIANT_LOGITS)
    fs.check(fs.fs_logits(p, x.H, x.W, out, ws), "fs_logits")
    t.cuda.synchronize()
    return host(out).astype(np.float64), out


def run_multinomial(x, p, logits_dev):
    t = torch()
    idx = t.full((x.B,), -7, dtype=t.int32, device="cuda")
    ws = workspace(p, fs.FS_VARIANT_MULTINOMIAL)
    fs.check(fs.fs_multinomial(p, logits_dev, x.temp, x.allow, idx, ws), "fs_multinomial")
    t.cuda.synchronize()
    return host(idx).astype(np.int64)


def run_merge(z, L, temp, seed, step, flags=0):
    t = torch()
    B, C = z.shape
    zd = dev(np.asarray(z, np.int32))
    Ld = dev(np.asarray(L, np.float32))
    td = None if temp is None else dev(np.asarray(temp, np.float32))
    out = t.full((B,), -7, dtype=t.int32, device="cuda")
    A = t.full((B,), 7.0, dtype=t.float32, device="cuda")
    fs.check(fs.fs_merge_online(B, C, zd, Ld, td, seed, step, flags, out, A), "fs_merge_online")
    t.cuda.synchronize()
    return host(out).astype(np.int64), host(A).astype(np.float64)


# ---------------------------------------------------------------------------
# comparisons
# ---------------------------------------------------------------------------
def check_index_rows(got, want, gap, s_oracle, id0=0, tol=TOL_GAP, what="index"):
    """Indices agree on every row whose oracle gap exceeds `tol`; on the other
    rows the GPU's pick must be a valid near-maximiser of the oracle scores.
    Returns the number of pinned rows."""
    got = np.asarray(got)
    want = np.asarray(want)
    pinned = np.asarray(gap) > tol
    bad = np.nonzero(pinned & (got != want))[0]
    assert bad.size == 0, f"{what}: rows {bad[:10]} got {got[bad[:10]]} want {want[bad[:10]]}"
    for b in np.nonzero(~pinned)[0]:
        if want[b] < 0:
            assert got[b] == -1, f"{what}: row {b} should be empty"
            continue
        j = got[b] - id0
        assert 0 <= j < s_oracle.shape[1], f"{what}: row {b} index {got[b]} out of range"
        assert s_oracle[b, j] >= s_oracle[b, want[b] - id0] - tol, \
            f"{what}: row {b} picked {got[b]} which is not a near-maximiser"
    return int(pinned.sum())


def assert_pinned(pin, what, min_frac=MIN_PINNED):
    """Log and require the fraction of rows compared index for index: a
    selection helper that wrongly marked rows as unpinned would otherwise
    empty the comparison without failing it."""
    pin = np.asarray(pin, bool)
    n = int(pin.sum())
    log(f"  {what}: {n}/{pin.size} rows pinned")
    assert pin.size == 0 or n >= min_frac * pin.size, \
        f"{what}: only {n}/{pin.size} rows pinned (< {min_frac:.0%})"
    return n


def check_grouped_unpinned(got, want, tile_idx, pinned, what="grouped"):
    """Rows whose hierarchical draw is not pinned: -1 only where the oracle
    row is empty, otherwise one of the row's own tile winners."""
    for b in np.nonzero(~np.asarray(pinned, bool))[0]:
        if want[b] < 0:
            assert got[b] == -1, f"{what}: row {b} should be empty, got {got[b]}"
        else:
            assert got[b] >= 0 and got[b] in set(np.asarray(tile_idx[b]).tolist()), \
                f"{what}: row {b} drew {got[b]}, not a tile winner of the row"


def check_values(got, want, tol=TOL_VALUE, what="value"):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: finiteness differs"
    assert np.array_equal(got[~fin], want[~fin]), f"{what}: infinities differ"
    if fin.any():
        err = np.abs(got[fin] - want[fin]).max()
        assert err <= tol, f"{what}: max abs error {err} > {tol}"
