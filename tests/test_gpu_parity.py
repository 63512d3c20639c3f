"""GPU parity of libfs against the CPU oracle on small shapes (several tiles,
ragged tails, masks, greedy rows, every entry point).  Acceptance:
Philox words bit-exact; per-tile max and log-mass within 2e-3; sampled
indices identical wherever the oracle's top-two noisy scores differ by more
than 1e-2 (elsewhere a valid near-maximiser); sample histograms pass
chi-square (p > 0.01) against the oracle's softmax; repeated calls
bit-identical."""
import math

import numpy as np
import pytest

import lm_head_gumbel_amd as fs
from lm_head_gumbel_amd.inputs import (bf16_bits_to_f32, f32_to_bf16_bits, hidden_bf16,
                                       normal_f32, tiny_reference, weights_bf16)
from oracle import fs_oracle as O
from oracle import philox as px
from gpu_util import (Inputs, TOL_CUT, TOL_GAP, TOL_VALUE, check_grouped_unpinned,
                      check_index_rows, check_values, host, log,
                      run_flat, run_grouped, run_logits, run_merge, run_multinomial, run_topk,
                      run_topp, torch)
from stats_util import chi_square_p, chi_square_rows_p, softmax

pytestmark = pytest.mark.gpu

SEED = 1234
MULTI_TOL = 1e-4   # CDF-boundary margin below which a multinomial draw is not pinned


@pytest.fixture(scope="module", autouse=True)
def _device():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a device"
    assert fs.fs_version()
    yield


# ---------------------------------------------------------------------------
# noise
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, SEED, 0xDEADBEEF12345678])
@pytest.mark.parametrize("stream_id", [0, 1, 2, 3])
def test_noise_words_bit_exact(seed, stream_id):
    t = torch()
    log(f"noise seed={seed:#x} stream={stream_id}")
    nb, ni = 3, 4099
    for i0 in (0, 151936 - 2048, (1 << 31) - 1024):
        words = t.zeros((nb, ni), dtype=t.int32, device="cuda")
        g = t.zeros((nb, ni), dtype=t.float32, device="cuda")
        fs.check(fs.fs_debug_noise(seed, 77, stream_id, 5, nb, i0, ni, words, g), "noise")
        t.cuda.synchronize()
        w = words.cpu().numpy().view(np.uint32)
        ids = i0 + np.arange(ni, dtype=np.int64)
        ref = px.noise_words(seed, 5 + np.arange(nb)[:, None], ids[None, :], 77, stream_id)
        assert np.array_equal(w, ref)
        gref = O.gumbel_from_word(ref)
        err = np.abs(g.cpu().numpy().astype(np.float64) - gref)
        # FP32 transform: error of a few ulps of |g| <= 22.9 plus the rounding of v
        assert err.max() < 2e-5, err.max()


def test_gumbel_extreme_words():
    t = torch()
    # find ids whose words are near 0 and near 2^32 among a long range, and check g there
    ni = 1 << 20
    words = t.zeros((1, ni), dtype=t.int32, device="cuda")
    g = t.zeros((1, ni), dtype=t.float32, device="cuda")
    fs.check(fs.fs_debug_noise(SEED, 0, 0, 0, 1, 0, ni, words, g), "noise")
    t.cuda.synchronize()
    w = words.cpu().numpy().view(np.uint32)[0]
    gv = g.cpu().numpy()[0].astype(np.float64)
    assert np.all(np.isfinite(gv))
    sel = np.concatenate([np.argsort(w)[:64], np.argsort(w)[-64:]])
    ref = O.gumbel_from_word(w[sel])
    assert np.abs(gv[sel] - ref).max() < 2e-5


# ---------------------------------------------------------------------------
# one full comparison of every entry point on one problem
# ---------------------------------------------------------------------------
def check_topk(x_in, p, r, k, v_offset=0, top_ps=(0.9, 0.5)):
    """Top-k and top-p after top-k against the oracle on the oracle's x and s."""
    B = x_in.B
    tk = run_topk(x_in, p, k)
    oi, ogap, omarg = O.topk_sample(r["x"], r["s"], k, v_offset)
    pin = (ogap > TOL_GAP) & (omarg > 1e-3)
    bad = np.nonzero(pin & (tk != oi))[0]
    assert bad.size == 0, f"top-{k} rows {bad} got {tk[bad]} want {oi[bad]}"
    for b in range(B):
        if oi[b] < 0:
            assert tk[b] == -1
        else:
            assert np.isfinite(r["x"][b, tk[b] - v_offset])
    # top-p after top-k; top_p = 1 is the top-k sample itself
    assert np.array_equal(run_topp(x_in, p, k, 1.0), tk)
    for top_p in top_ps:
        tp = run_topp(x_in, p, k, top_p)
        oi, ogap, omarg, ocut = O.topk_topp_sample(r["x"], r["s"], k, top_p, v_offset)
        pin = (ogap > TOL_GAP) & (omarg > 1e-3) & (ocut > TOL_CUT)
        bad = np.nonzero(pin & (tp != oi))[0]
        assert bad.size == 0, f"top-{k} top-p {top_p} rows {bad} got {tp[bad]} want {oi[bad]}"
        assert np.all((tp == -1) == (oi == -1))
    return int(pin.sum())


def compare_all(Hb, Wb, temp=None, n_valid=None, allow=None, tile_v=128, v_offset=0,
                seed=SEED, steps=(0,), flags=0, topk=(1, 7, 40), check_logits=True):
    B, d = Hb.shape
    V = Wb.shape[0]
    x_in = Inputs(Hb, Wb, temp, allow)
    l = O.logits_bf16(Hb, Wb)
    nv = v_offset + V if n_valid is None else n_valid
    if check_logits:
        p = x_in.params(n_valid=nv, v_offset=v_offset, tile_v=tile_v, seed=seed, flags=flags)
        gl, gl_dev = run_logits(x_in, p)
        scale = np.abs(O.bf16_bits_to_f64(Hb)).sum(1)[:, None] * \
            np.abs(O.bf16_bits_to_f64(Wb)).max() + 1e-30
        # FP32 accumulation: |error| <= d * 2^-24 * sum |H_k W_ik| (loose bound)
        assert np.all(np.abs(gl - l) <= max(d, 1) * 2.0 ** -24 * scale + 1e-30)
    for step in steps:
        p = x_in.params(n_valid=nv, v_offset=v_offset, tile_v=tile_v, seed=seed, step=step,
                        flags=flags)
        r = O.run_call(l, temp, nv, allow, seed, step, flags, tile_v, v_offset)
        # flat
        gi, gs = run_flat(x_in, p)
        npin = check_index_rows(gi, r["flat_idx"], r["flat_gap"], r["s"], v_offset,
                                what="flat")
        check_values(gs, r["flat_max"], what="flat score")
        # grouped
        m, ti, L, go = run_grouped(x_in, p)
        check_values(m, r["tile_m"], what="tile max")
        check_values(L, r["tile_L"], what="tile log-mass")
        for t in range(m.shape[1]):
            c0 = t * tile_v
            check_index_rows(ti[:, t], r["tile_idx"][:, t], r["tile_gap"][:, t],
                             r["s"][:, c0:c0 + tile_v], v_offset + c0, what=f"tile {t} idx")
        pinned = r["grp_gap"] > TOL_GAP
        for b in range(B):
            t = r["grp_tile"][b]
            if t >= 0 and r["tile_gap"][b, t] <= TOL_GAP:
                pinned[b] = False
        bad = np.nonzero(pinned & (go != r["grp_idx"]))[0]
        assert bad.size == 0, f"grouped sample rows {bad}"
        check_grouped_unpinned(go, r["grp_idx"], ti, pinned)
        # top-k
        for k in topk:
            check_topk(x_in, p, r, k, v_offset)
        # unfused baseline on the GPU's own logits
        if check_logits:
            mi = run_multinomial(x_in, p, gl_dev)
            oi, omarg = O.multinomial(r["x"], temp, seed, step, flags, v_offset)
            pin = omarg > MULTI_TOL
            bad = np.nonzero(pin & (mi != oi))[0]
            assert bad.size == 0, f"multinomial rows {bad} got {mi[bad]} want {oi[bad]}"
        log(f"  B={B} d={d} V={V} tile={tile_v} step={step}: {npin}/{B} flat rows pinned")
    return x_in


CASES = [
    # (B, d, V, tile_v, n_valid_cut, v_offset, temp kind, allow)
    (1, 64, 1000, 128, 10, 0, "one", False),       # V not a multiple of 16, ragged tail
    (5, 136, 3001, 64, 11, 32, "mixed", True),      # d not a multiple of 32, offset ids
    (16, 256, 2048, 512, 0, 0, "range", False),     # exactly one N-block
    (17, 96, 2500, 256, 285, 0, "range", True),     # two N-blocks, partial
    (40, 128, 1500, 48, 3, 16, "mixed", False),     # four N-blocks, odd tile size
    (3, 512, 4096, 16, 0, 0, "one", False),         # smallest tile
    # d with nks % 8 == 0 runs the resident-H kernel (one or two batch blocks)
    (7, 1024, 3000, 128, 7, 0, "mixed", True),
    (25, 1024, 2600, 64, 0, 32, "range", False),
    (20, 512, 1500, 256, 5, 0, "mixed", False),
    (2, 2048, 1111, 32, 1, 16, "range", True),
    # d = 4096 with two batch blocks and an allow mask (the shape of the
    # headline B = 32 call)
    (20, 4096, 3000, 128, 5, 0, "mixed", True),
    # B > 64 grouped runs the resident kernel in three batch groups, paired
    # on one XCD per row range
    (72, 512, 2000, 64, 0, 0, "mixed", True),
    # d = 5120 with two batch blocks: part of each wave's H slice lives in LDS
    (24, 5120, 2000, 128, 3, 16, "mixed", True),
    # d = 3072 (12 k-steps per wave, two and one batch blocks), d = 6144 and
    # 7168 (one batch block, four waves; two batch groups above 16 rows)
    (20, 3072, 3000, 128, 5, 0, "mixed", True),
    (9, 3072, 1700, 64, 0, 16, "range", False),
    (9, 6144, 2000, 64, 3, 16, "range", False),
    (24, 6144, 2500, 128, 0, 0, "mixed", True),
    (5, 7168, 1500, 256, 0, 0, "mixed", True),
    # no resident shape at d = 8192: flat and logits take the row-streaming
    # kernel at any batch (64 columns, most of them padding here)
    (3, 8192, 2000, 128, 0, 0, "mixed", True),
    # fewer than four vocab blocks: the workgroup-cooperative kernel
    (5, 64, 40, 16, 3, 0, "one", False),
    # B > 32 flat and logits with d % 512 == 0 (64 or 128 columns per
    # workgroup) or d % 256 == 0 (256): the row-streaming kernel; ragged
    # ranges, short last tiles (at most 128 rows skip block 1, more run
    # whole), and two column groups paired on one XCD
    (33, 512, 3001, 64, 7, 16, "mixed", True),
    (40, 4096, 3000, 128, 5, 0, "mixed", True),
    (100, 512, 3001, 64, 5, 0, "mixed", True),
    (128, 512, 70000, 2048, 0, 32, "range", False),
    (100, 512, 102400, 4096, 0, 0, "range", False),   # ranges of 400 rows
    (150, 256, 2000, 128, 5, 0, "mixed", True),
    (256, 256, 70000, 4096, 3, 0, "mixed", True),
    (300, 256, 5000, 64, 0, 0, "range", False),
    # grouped on the row-streaming kernel (a record per 16-row block, each
    # block in one wave) in two 128-column groups paired on one XCD
    (200, 512, 30000, 128, 5, 0, "mixed", True),
    # grouped at 128 columns, ranges of 17-18 blocks: one full tile and a
    # half tile
    (100, 512, 70000, 256, 5, 0, "mixed", True),
    # grouped at 64 columns, ranges of 68-69 blocks: the first 64 block
    # records held in LDS to the end of the kernel, the rest stored as their
    # tiles end (16-block vocabulary tiles mixing both)
    (40, 512, 280003, 256, 5, 0, "mixed", True),
    # B > 32 with other d: the streaming kernel
    (100, 192, 1700, 64, 0, 16, "range", False),
    # 32 < B <= 64: grouped records from the LDS-tiled kernel too; ranges of
    # 320 rows (two 256-row tiles) meeting several vocabulary tiles, and
    # 16-row vocabulary tiles (eight per range)
    (48, 256, 80000, 64, 7, 16, "mixed", True),
    (64, 128, 30000, 16, 0, 0, "range", False),
    # resident grouped (a record per 16-row block): 16-row tiles, with more
    # blocks per workgroup than its LDS store holds at once (stored in parts)
    (4, 1024, 45000, 16, 0, 0, "mixed", False),
    (3, 1024, 80000, 16, 9, 0, "range", True),
    (2, 512, 280000, 16, 5, 0, "mixed", False),
    # resident grouped, few large tiles: stage 2 splits a tile into runs of
    # blocks merged in a tree inside one wave (20 tiles, 32 runs each), across
    # two waves (5 tiles, 128 runs) and across all sixteen (one tile)
    (5, 2048, 20000, 1024, 3, 0, "mixed", True),
    (6, 1024, 40000, 8192, 5, 16, "range", False),
    (3, 512, 30000, 40000, 0, 0, "mixed", True),
    # resident grouped at a tiny vocabulary: one tile (stage 2 in one
    # workgroup per 32 rows), and 16 two-block tiles (two workgroups whose
    # row keys meet through the atomic pair)
    (3, 512, 100, 128, 0, 0, "mixed", False),
    (6, 1024, 500, 32, 4, 0, "range", True),
]


def make_case(B, d, V, temp_kind, allow_on, seed=0):
    rng = np.random.default_rng(100 + B + d + V)
    Hb = hidden_bf16(B, d, seed=11 + seed)
    Wb = weights_bf16(V, d, std=0.05, seed=12 + seed)
    if temp_kind == "one":
        temp = np.ones(B, np.float32)
    elif temp_kind == "range":
        temp = rng.uniform(0.3, 1.5, B).astype(np.float32)
    else:
        temp = rng.uniform(0.3, 1.5, B).astype(np.float32)
        temp[0] = 0.0
        if B > 2:
            temp[2] = -1.0
        if B > 3:
            temp[3] = np.nan
    allow = None
    if allow_on:
        words = (V + 31) // 32
        allow = rng.integers(0, 2 ** 32, size=(B, words), dtype=np.uint64).astype(np.uint32)
        allow |= rng.integers(0, 2 ** 32, size=(B, words), dtype=np.uint64).astype(np.uint32)
    return Hb, Wb, temp, allow


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}_d{c[1]}_V{c[2]}_t{c[3]}")
def test_parity_small(case):
    B, d, V, tile_v, cut, v_off, tk, al = case
    log(f"parity case {case}")
    Hb, Wb, temp, allow = make_case(B, d, V, tk, al)
    compare_all(Hb, Wb, temp, n_valid=v_off + V - cut, allow=allow, tile_v=tile_v,
                v_offset=v_off, steps=(0, 1))


# k above 64: lists of up to a whole workgroup range per row (the resident
# stage-1 kernel) and the binned stage-2 selection; k >= the valid ids keeps
# them all
LARGE_K_CASES = [
    # (B, d, V, n_valid_cut, v_offset, temp kind, allow, ks)
    (7, 1024, 3000, 7, 0, "mixed", True, (65, 300, 1024)),
    (25, 1024, 2600, 0, 32, "range", False, (100, 1000)),
    (24, 5120, 2000, 3, 16, "mixed", True, (128, 700)),
    (2, 2048, 1111, 1, 16, "range", True, (1024,)),
    (20, 512, 20000, 5, 0, "range", False, (200, 1024)),
    (9, 6144, 3000, 2, 0, "mixed", True, (100, 1000)),
]


@pytest.mark.parametrize("case", LARGE_K_CASES, ids=lambda c: f"B{c[0]}_d{c[1]}_V{c[2]}")
def test_topk_large_k(case):
    B, d, V, cut, v_off, tk, al, ks = case
    Hb, Wb, temp, allow = make_case(B, d, V, tk, al)
    x_in = Inputs(Hb, Wb, temp, allow)
    l = O.logits_bf16(Hb, Wb)
    nv = v_off + V - cut
    for step in (0, 1):
        p = x_in.params(n_valid=nv, v_offset=v_off, tile_v=128, seed=SEED, step=step)
        r = O.run_call(l, temp, nv, allow, SEED, step, 0, 128, v_off)
        for k in ks:
            log(f"large k: B={B} d={d} V={V} k={k} step={step}")
            npin = check_topk(x_in, p, r, k, v_off, top_ps=(0.95, 0.6))
            log(f"  {npin}/{B} rows pinned")


def test_topk_large_k_needs_the_resident_kernel():
    """k > 64 on a hidden size that only the cooperative kernel covers is
    reported, not run."""
    t = torch()
    Hb, Wb, temp, _ = make_case(3, 136, 900, "one", False)
    x = Inputs(Hb, Wb, temp)
    p = x.params(seed=SEED)
    assert fs.fs_workspace_bytes(p, fs.FS_VARIANT_TOPK, 65) == 0
    assert fs.fs_workspace_bytes(p, fs.FS_VARIANT_TOPK, 64) > 0
    idx = t.full((3,), -7, dtype=t.int32, device="cuda")
    ws = t.empty(1 << 24, dtype=t.uint8, device="cuda")
    assert fs.fs_sample_topk(p, x.H, x.W, x.temp, None, 65, idx, ws) == fs.FS_ERR_UNSUPPORTED
    assert fs.fs_sample_topk(p, x.H, x.W, x.temp, None, 1025, idx, ws) == fs.FS_ERR_UNSUPPORTED
    t.cuda.synchronize()
    assert np.all(idx.cpu().numpy() == -7)


def test_tiny_reference_config():
    wl, H, W = tiny_reference()
    log("tiny reference: B=4 d=256 V=4096 tile 512")
    Hb, Wb = f32_to_bf16_bits(H), f32_to_bf16_bits(W)
    compare_all(Hb, Wb, np.ones(4, np.float32), tile_v=512, steps=(0,))


def test_no_noise_is_greedy():
    Hb, Wb, temp, _ = make_case(9, 128, 1234, "range", False)
    log("no-noise flag")
    x = Inputs(Hb, Wb, temp)
    p = x.params(seed=SEED, flags=fs.FS_NO_NOISE, tile_v=64)
    l = O.logits_bf16(Hb, Wb)
    want = np.argmax(l, axis=1)
    gap = np.sort(l, axis=1)[:, -1] - np.sort(l, axis=1)[:, -2]
    ok = gap > 1e-4
    gi, _ = run_flat(x, p)
    assert np.array_equal(gi[ok], want[ok])
    _, _, _, go = run_grouped(x, p)
    assert np.array_equal(go[ok], want[ok])
    for k in (1, 5):
        assert np.array_equal(run_topk(x, p, k)[ok], want[ok])


def test_masked_rows_and_empty_shapes():
    t = torch()
    Hb, Wb, temp, _ = make_case(4, 64, 700, "one", False)
    x = Inputs(Hb, Wb, temp, np.zeros((4, (700 + 31) // 32), np.uint32))
    p = x.params(seed=SEED, tile_v=128)
    gi, gs = run_flat(x, p)
    assert np.all(gi == -1) and np.all(np.isneginf(gs))
    m, ti, L, go = run_grouped(x, p)
    assert np.all(ti == -1) and np.all(np.isneginf(m)) and np.all(np.isneginf(L))
    assert np.all(go == -1)
    assert np.all(run_topk(x, p, 3) == -1)
    x2 = Inputs(Hb, Wb, temp)
    gi, _ = run_flat(x2, x2.params(n_valid=0, seed=SEED))
    assert np.all(gi == -1)
    # V = 0: every row -1
    idx = t.full((4,), 5, dtype=t.int32, device="cuda")
    ws = t.empty(1 << 20, dtype=t.uint8, device="cuda")
    fs.check(fs.fs_sample(fs.params(4, 64, 0), x.H, x.W, None, None, idx, None, ws), "V=0")
    t.cuda.synchronize()
    assert np.all(idx.cpu().numpy() == -1)
    # B = 0: nothing is written
    fs.check(fs.fs_sample(fs.params(0, 64, 700), x.H, x.W, None, None, idx, None, ws), "B=0")
    # undersized workspace is reported, not run
    p = x.params(seed=SEED)
    n = fs.fs_workspace_bytes(p, fs.FS_VARIANT_FLAT)
    assert fs.fs_sample(p, x.H, x.W, None, None, idx, None, ws, n - 1) == fs.FS_ERR_WORKSPACE


def test_nan_logits_never_win():
    Hb, Wb, temp, _ = make_case(3, 64, 500, "one", False)
    Wb = Wb.copy()
    Wb[17, 5] = 0x7FC0   # NaN weight: id 17 has a NaN logit in every row
    x = Inputs(Hb, Wb, temp)
    p = x.params(seed=SEED, tile_v=16)
    l = O.logits_bf16(Hb, Wb)
    assert np.all(np.isnan(l[:, 17]))
    r = O.run_call(l, temp, None, None, SEED, 0, 0, 16)
    gi, _ = run_flat(x, p)
    check_index_rows(gi, r["flat_idx"], r["flat_gap"], r["s"])
    assert not np.any(gi == 17)
    m, ti, L, _ = run_grouped(x, p)
    check_values(L, r["tile_L"], what="tile log-mass with NaN")


@pytest.mark.parametrize("B,d", [(3, 1024), (24, 1024), (5, 136)])
def test_topk_exact_ties_take_lowest_ids(B, d):
    """W rows 300..499 are copies of one row aligned with every hidden state,
    so each batch row's largest logits are 200 exactly equal values.  The
    top-k set is then ids 300 .. 300+k-1 (ties go to the lower id), spread
    over several workgroups, and the sample is the largest noisy score among
    them."""
    V, lo, hi = 3000, 300, 500
    Hb, Wb, temp, _ = make_case(B, d, V, "range", False)
    Wb = Wb.copy()
    hsum = bf16_bits_to_f32(Hb).astype(np.float64).sum(axis=0)
    Wb[lo:hi] = f32_to_bf16_bits((20.0 / d * hsum).astype(np.float32))[None, :]
    x_in = Inputs(Hb, Wb, temp)
    l = O.logits_bf16(Hb, Wb)
    assert np.all(l[:, lo:hi] == l[:, lo:lo + 1]) and np.all(l[:, lo] > np.delete(l, np.s_[lo:hi], 1).max(1))
    for step in (0, 3):
        p = x_in.params(seed=SEED, step=step, tile_v=128)
        r = O.run_call(l, temp, None, None, SEED, step, 0, 128)
        for k in (1, 7, 40):
            log(f"ties B={B} d={d} k={k} step={step}")
            got = run_topk(x_in, p, k)
            assert np.all((got >= lo) & (got < lo + k)), got
            s = r["s"][:, lo:lo + k]
            want = lo + np.argmax(s, axis=1)
            top2 = np.sort(s, axis=1)
            gap = top2[:, -1] - top2[:, -2] if k > 1 else np.full(B, np.inf)
            pin = gap > TOL_GAP
            assert np.array_equal(got[pin], want[pin])
            oi, _, _ = O.topk_sample(r["x"], r["s"], k)
            assert np.array_equal(oi[pin], want[pin])


@pytest.mark.parametrize("V,k", [(200000, 64), (40000, 40), (1024, 8), (200000, 1024),
                                 (3000, 1000), (900, 1024)])
def test_topk_all_logits_equal(V, k):
    """Every W row is the same row, so all V logits of a batch row are equal
    and the top-k set is ids 0 .. k-1.  The sizes drive the selection into its
    less common branches: whole workgroup ranges of ties (768 and 160 rows
    per workgroup), stage-2 candidate sets that the lower bound cannot prune,
    and for large k the exact radix search (all candidates in one bin), the
    gathered sort and a row with fewer valid ids than k."""
    B, d = 3, 512
    Hb = hidden_bf16(B, d, seed=21)
    row = weights_bf16(1, d, std=0.05, seed=22)
    Wb = np.ascontiguousarray(np.broadcast_to(row, (V, d)))
    temp = np.array([1.0, 0.6, 0.0], np.float32)   # the last row greedy
    x_in = Inputs(Hb, Wb, temp)
    l = O.logits_bf16(Hb, row)
    p = x_in.params(seed=SEED, step=2)
    log(f"all-equal logits V={V} k={k}")
    got = run_topk(x_in, p, k)
    k_req, k = k, min(k, V)   # every id when there are fewer than k
    assert np.all((got >= 0) & (got < k)), got
    x = O.tempered(np.repeat(l, k, axis=1), temp)
    sc = O.scores(x, temp, SEED, 2, 0, 0)
    want = np.argmax(sc, axis=1)
    top2 = np.sort(sc, axis=1)
    pin = (top2[:, -1] - top2[:, -2]) > TOL_GAP
    pin[2] = True   # greedy row: equal scores, the lowest id
    assert want[2] == 0
    assert np.array_equal(got[pin], want[pin])
    # top-p 0.5 on k equal masses keeps the first ceil(k / 2): ids 0 .. ceil(k/2) - 1
    kept = (k + 1) // 2
    tp = run_topp(x_in, p, k_req, 0.5)
    assert np.all((tp >= 0) & (tp < kept)), tp
    want = np.argmax(sc[:, :kept], axis=1)
    top2 = np.sort(sc[:, :kept], axis=1)
    pin = (top2[:, -1] - top2[:, -2]) > TOL_GAP if kept > 1 else np.ones(B, bool)
    pin[2] = True
    assert np.array_equal(tp[pin], want[pin])


def test_repeated_calls_bit_identical():
    Hb, Wb, temp, allow = make_case(33, 256, 5000, "mixed", True)
    x = Inputs(Hb, Wb, temp, allow)
    p = x.params(seed=SEED, step=3, tile_v=256)
    a = run_flat(x, p)
    b = run_flat(x, p)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.int64), b[1].view(np.int64))
    g1 = run_grouped(x, p)
    g2 = run_grouped(x, p)
    for u, v in zip(g1, g2):
        assert np.array_equal(np.asarray(u), np.asarray(v))
    assert np.array_equal(run_topk(x, p, 40), run_topk(x, p, 40))


@pytest.mark.parametrize("tile_v", [128, 8192])
def test_grouped_block_records_are_deterministic(tile_v):
    """The resident kernel's block records on one reused workspace (its last
    units by ticket, so the workgroup that walks a block changes from call to
    call), merged per tile in stage 2 by several workgroups whose row keys meet
    through atomics: every output is identical from call to call and to a
    call on a fresh workspace."""
    t = torch()
    Hb, Wb, temp, allow = make_case(20, 1024, 30000, "mixed", True)
    x = Inputs(Hb, Wb, temp, allow)
    p = x.params(seed=SEED, step=5, tile_v=tile_v)
    T = fs.fs_num_tiles(p)
    ws = t.empty(fs.fs_workspace_bytes(p, fs.FS_VARIANT_GROUPED), dtype=t.uint8, device="cuda")
    outs = []
    for _ in range(4):
        m = t.full((x.B, T), 7.0, dtype=t.float32, device="cuda")
        ti = t.full((x.B, T), -7, dtype=t.int32, device="cuda")
        L = t.full((x.B, T), 7.0, dtype=t.float32, device="cuda")
        o = t.full((x.B,), -7, dtype=t.int32, device="cuda")
        fs.check(fs.fs_sample_grouped(p, x.H, x.W, x.temp, x.allow, m, ti, L, o, ws))
        t.cuda.synchronize()
        outs.append([host(m), host(ti), host(L), host(o)])
    for run in outs[1:]:   # bit for bit, floats compared as their bit patterns
        for u, v in zip(outs[0], run):
            assert np.array_equal(u.view(np.int32), v.view(np.int32))
    fresh = run_grouped(x, p)   # another workspace
    for u, v in zip(outs[0], fresh):
        assert np.array_equal(u.astype(np.float64), np.asarray(v, np.float64))


def test_online_merge_matches_oracle():
    # chunks of 320 ids over V = 2560 (8 chunks), records from the grouped entry point
    Hb, Wb, temp, _ = make_case(12, 128, 2560, "mixed", False)
    x = Inputs(Hb, Wb, temp)
    l = O.logits_bf16(Hb, Wb)
    for step in (0, 5):
        p = x.params(seed=SEED, step=step, tile_v=320)
        m, ti, L, _ = run_grouped(x, p, with_sample=False)
        gz, gA = run_merge(ti, L, temp, SEED, step)
        # oracle merge on the oracle's own chunk records
        r = O.run_call(l, temp, None, None, SEED, step, 0, 320)
        oz, oA, omarg = O.online_merge(r["tile_idx"], r["tile_L"], temp, SEED, step)
        check_values(gA, oA, tol=TOL_VALUE, what="merged log-mass")
        chunk_pinned = (r["tile_gap"] > TOL_GAP).all(axis=1)
        pin = (omarg > 1e-2) & chunk_pinned
        bad = np.nonzero(pin & (gz != oz))[0]
        assert bad.size == 0, f"merge rows {bad}"
        # the same merge on the GPU's records must follow the GPU's chunk winners
        oz2, _, om2 = O.online_merge(ti, L, temp, SEED, step)
        pin2 = om2 > 1e-2
        assert np.array_equal(gz[pin2], oz2[pin2])


def test_flat_histogram_chi_square():
    # one hidden state repeated over 10 rows, 500 decode steps: 5000 draws
    t = torch()
    V, d = 64, 64
    H1 = hidden_bf16(1, d, seed=3)
    Hb = np.repeat(H1, 10, axis=0)
    Wb = weights_bf16(V, d, std=0.15, seed=4)
    temp = np.full(10, 0.8, np.float32)
    x = Inputs(Hb, Wb, temp)
    l = O.logits_bf16(H1, Wb)[0]
    prob = softmax(l / 0.8)
    flat, grp, top = [], [], []
    for step in range(500):
        p = x.params(seed=SEED, step=step, tile_v=16)
        flat.append(run_flat(x, p)[0])
        grp.append(run_grouped(x, p)[3])
    flat = np.concatenate(flat)
    grp = np.concatenate(grp)
    pf = chi_square_p(flat, prob)
    pg = chi_square_p(grp, prob)
    log(f"chi-square p: flat {pf:.3f} grouped {pg:.3f}")
    assert pf > 0.01 and pg > 0.01
    # top-k 8: renormalised over the 8 largest logits
    keep = np.argsort(-l, kind="stable")[:8]
    pk = np.zeros(V)
    pk[keep] = softmax(l[keep] / 0.8)
    for step in range(500):
        p = x.params(seed=SEED, step=step)
        top.append(run_topk(x, p, 8))
    ptk = chi_square_p(np.concatenate(top), pk)
    log(f"chi-square p: top-8 {ptk:.3f}")
    assert ptk > 0.01


def test_read_probes_read_every_word_once():
    """Both HBM read probes (plain and nontemporal loads) read each 32-bit word
    of the buffer exactly once: the XOR over the sink equals the XOR of the
    buffer's words, with a grid-stride tail (a size that is not a multiple of
    the grid's loads per trip)."""
    t = torch()
    rng = np.random.default_rng(7)
    nbytes = (1 << 20) + 48 * 16
    words = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = t.from_numpy(words.view(np.int32).copy()).cuda()
    want = np.bitwise_xor.reduce(words)
    for grid in (8, 37):
        for probe in (fs.fs_debug_read_probe, fs.fs_debug_read_probe_nt):
            sink = t.zeros(grid * 256, dtype=t.int32, device="cuda")
            fs.check(probe(buf, nbytes, sink, grid), probe.__name__)
            t.cuda.synchronize()
            got = np.bitwise_xor.reduce(host(sink).view(np.uint32))
            assert got == want, (probe.__name__, grid)
