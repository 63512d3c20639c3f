"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (same entry points, same kernels).  The oracle computes the
rows it is given one by one (all rows up to B = 64, a sample of rows above).
Every comparison of sampled indices also requires that at least 90% of the
compared rows are pinned (their oracle result is robust by the stated
tolerances), so a mistake in a selection helper cannot empty a comparison.

Workloads (synthetic stand-ins for the pages' Qwen3-class decode LM heads):
  headline      d=4096, V=151936, B=32, T=1: the call the benchmark times,
                repeated on one workspace (last units by ticket)
  small model   d=2048, V=151936, B in {1, 8, 32}, T=0.7, tiles of 256;
                1000 decode steps (step = Philox counter word 2) for the
                histogram test
  mid-size      d=4096, V=151936, B in {1, 4, 16, 64}, T=1, last 285 ids
                masked, grouped records and hierarchical resample; 1000
                steps of the grouped sample for its histogram test
  compute-lean  d=4096, V=128256, B in {128, 256}, T_b ~ U[0.3, 1.5]; and
                B in {128, 256} at the headline vocabulary V=151936
  top-k/online  d=5120, V=152064, B=32, top-40 (and top-1000), online merge
                over 8 chunks of 19008 ids (and its histogram over 1000 steps)
  vocab shards  the headline call split into G in {2, 4, 8} shards of W with
                v_offset = g V / G, as a G-way tensor-parallel rank runs it
"""
import numpy as np
import pytest

import lm_head_gumbel_amd as fs
from lm_head_gumbel_amd.inputs import WORKLOADS, PHILOX_SEED, hidden_bf16, weights_bf16
from oracle import fs_oracle as O
from oracle import philox as px
from gpu_util import (Inputs, TOL_CUT, TOL_GAP, TOL_MASS, TOL_X, assert_pinned,
                      check_grouped_unpinned, check_index_rows, check_values, host, log, run_flat,
                      run_grouped, run_merge, run_topk, run_topp, torch)
from stats_util import chi_square_rows_p, softmax

pytestmark = pytest.mark.gpu

_W_CACHE = {}
D_HEAD, V_HEAD = 4096, 151936


def weights(V, d):
    key = (V, d)
    if key not in _W_CACHE:
        _W_CACHE.clear()
        log(f"generating W [{V}, {d}] bf16")
        _W_CACHE[key] = weights_bf16(V, d)
    return _W_CACHE[key]


def oracle_rows(Hb, Wb, rows, temp, n_valid, seed, step, tile_v=None, flags=0):
    """Oracle results for a subset of rows (row b keeps its own noise index b)."""
    l = O.logits_bf16(Hb[rows], Wb)
    t = None if temp is None else np.asarray(temp)[rows]
    x = O.tempered(l, t, n_valid)
    B, V = x.shape
    greedy = O.greedy_rows(t, B, flags)
    s = x.copy()
    ids = np.arange(V, dtype=np.int64)
    for j, b in enumerate(rows):
        if not greedy[j]:
            s[j] += O.gumbel_from_word(px.noise_words(seed, b, ids, step, px.STREAM_TOKEN))
    s[np.isneginf(x)] = -np.inf
    return l, x, s


def check_flat(gi, gs, x, s, rows, what="flat"):
    fidx, fmax, fgap = O.sample_flat(s)
    n = check_index_rows(gi[rows], fidx, fgap, s, what=what)
    check_values(gs[rows], fmax, what=f"{what} score")
    assert_pinned(fgap > TOL_GAP, what)
    return n


def sched_tagged(ws):
    """The unit-scheduler block of a flat workspace (its last 256 bytes)
    carries the initialisation tag: the next call takes its last units by
    ticket."""
    blk = host(ws[-256:]).view(np.uint64)
    return int(blk[0]) == 0x4C4D4847554D4231 and (int(blk[1]) >> 32) == 0x53434844


def test_headline_call_on_a_reused_workspace():
    """The call the benchmark times (B=32, d=4096, V=151936) on one workspace
    over four steps: from the second call on, the scheduler block is set up
    and stage 1 takes the last units of each workgroup by ticket.  Each such
    call must give the index and score, bit for bit, of the same call on a
    zeroed workspace (fixed strided order) and agree with the oracle."""
    t = torch()
    B = 32
    Hb = hidden_bf16(B, D_HEAD)
    Wb = weights(V_HEAD, D_HEAD)
    x_in = Inputs(Hb, Wb)
    rows = np.arange(B)
    p = x_in.params(seed=PHILOX_SEED)
    n = fs.fs_workspace_bytes(p, fs.FS_VARIANT_FLAT)
    ws = t.zeros(n, dtype=t.uint8, device="cuda")
    idx = t.empty(B, dtype=t.int32, device="cuda")
    score = t.empty(B, dtype=t.float32, device="cuda")
    for step in range(4):
        p.step = step
        tagged = sched_tagged(ws)
        assert tagged == (step > 0), f"step {step}: scheduler block tagged {tagged}"
        log(f"headline step {step}: {'ticket' if tagged else 'strided'} order")
        fs.check(fs.fs_sample(p, x_in.H, x_in.W, None, None, idx, score, ws), "fs_sample")
        t.cuda.synchronize()
        gi, gs = host(idx).astype(np.int64), host(score)
        # the same call on a fresh zeroed workspace: strided order only
        fresh = t.zeros(n, dtype=t.uint8, device="cuda")
        i2 = t.empty(B, dtype=t.int32, device="cuda")
        s2 = t.empty(B, dtype=t.float32, device="cuda")
        fs.check(fs.fs_sample(p, x_in.H, x_in.W, None, None, i2, s2, fresh), "fs_sample fresh")
        t.cuda.synchronize()
        assert np.array_equal(gi, host(i2)) and np.array_equal(gs.view(np.uint32),
                                                               host(s2).view(np.uint32))
        assert sched_tagged(ws)
        if step in (0, 3):
            _, x, s = oracle_rows(Hb, Wb, rows, None, None, PHILOX_SEED, step)
            check_flat(gi, gs.astype(np.float64), x, s, rows, what=f"headline step {step}")


def test_headline_grouped_on_a_reused_workspace():
    """Grouped records at the benchmark's shape (B=32, d=4096, V=151936,
    tiles of 128 ids): a record per 16-row unit, taken in the strided order
    and, from the second call on a workspace, the last units by ticket.  Every
    call's tile records and sample equal, bit for bit, those of the same call
    on a zeroed workspace, and agree with the oracle."""
    t = torch()
    B = 32
    Hb = hidden_bf16(B, D_HEAD)
    Wb = weights(V_HEAD, D_HEAD)
    x_in = Inputs(Hb, Wb)
    rows = np.arange(B)
    p = x_in.params(seed=PHILOX_SEED)
    n = fs.fs_workspace_bytes(p, fs.FS_VARIANT_GROUPED)
    T = fs.fs_num_tiles(p)
    ws = t.zeros(n, dtype=t.uint8, device="cuda")

    def call(wsx):
        m = t.empty((B, T), dtype=t.float32, device="cuda")
        ti = t.empty((B, T), dtype=t.int32, device="cuda")
        L = t.empty((B, T), dtype=t.float32, device="cuda")
        out = t.empty(B, dtype=t.int32, device="cuda")
        fs.check(fs.fs_sample_grouped(p, x_in.H, x_in.W, None, None, m, ti, L, out, wsx),
                 "fs_sample_grouped")
        t.cuda.synchronize()
        return [host(m), host(ti), host(L), host(out)]

    for step in range(3):
        p.step = step
        tagged = sched_tagged(ws)
        assert tagged == (step > 0), f"step {step}: scheduler block tagged {tagged}"
        log(f"grouped headline step {step}: {'ticket' if tagged else 'strided'} order")
        got = call(ws)
        want = call(t.zeros(n, dtype=t.uint8, device="cuda"))
        for g, w in zip(got, want):
            assert np.array_equal(g.view(np.uint32), w.view(np.uint32))
        assert sched_tagged(ws)
        if step in (0, 2):
            m, ti, L, go = (got[0].astype(np.float64), got[1].astype(np.int64),
                            got[2].astype(np.float64), got[3].astype(np.int64))
            _, x, s = oracle_rows(Hb, Wb, rows, None, None, PHILOX_SEED, step)
            om, oidx, oL, ogap = O.tile_records(x, s, 128)
            check_values(m, om, what="tile max")
            check_values(L, oL, what="tile log-mass")
            pinned = ogap > TOL_GAP
            assert np.array_equal(ti[pinned], oidx[pinned])
            assert_pinned(pinned.ravel(), "tiles")
            gidx, ggap, gt = O.sample_grouped(oidx, oL, None, PHILOX_SEED, step)
            pin = (ggap > TOL_GAP) & np.array([gt[b] < 0 or ogap[b, gt[b]] > TOL_GAP for b in rows])
            assert np.array_equal(go[pin], gidx[pin])
            assert_pinned(pin, "grouped")
            check_grouped_unpinned(go, gidx, ti, pin)


@pytest.mark.parametrize("B", [1, 8, 32])
def test_small_model_flat_and_grouped(B):
    wl = WORKLOADS[f"small_b{B}"]
    log(f"small model B={B} d={wl.d} V={wl.V}")
    Hb = hidden_bf16(B, wl.d)
    Wb = weights(wl.V, wl.d)
    temp = wl.temps()
    x_in = Inputs(Hb, Wb, temp)
    rows = np.arange(B)
    for step in (0, 999):
        p = x_in.params(tile_v=wl.tile_v, seed=PHILOX_SEED, step=step)
        gi, gs = run_flat(x_in, p)
        l, x, s = oracle_rows(Hb, Wb, rows, temp, None, PHILOX_SEED, step)
        check_flat(gi, gs, x, s, rows)
        m, ti, L, go = run_grouped(x_in, p)
        om, oidx, oL, ogap = O.tile_records(x, s, wl.tile_v)
        check_values(m, om, what="tile max")
        check_values(L, oL, what="tile log-mass")
        pinned = ogap > TOL_GAP
        assert np.array_equal(ti[pinned], oidx[pinned])
        assert_pinned(pinned.ravel(), f"step {step} tiles")


def test_small_model_histogram_1000_steps():
    """1000 decode steps of 8 rows: the per-row draws follow softmax(l/0.7)."""
    wl = WORKLOADS["small_b8"]
    Hb = hidden_bf16(8, wl.d)
    Wb = weights(wl.V, wl.d)
    temp = wl.temps()
    x_in = Inputs(Hb, Wb, temp)
    t = torch()
    idx = t.empty((1000, 8), dtype=t.int32, device="cuda")
    p = x_in.params(tile_v=wl.tile_v, seed=PHILOX_SEED)
    ws = t.empty(fs.fs_workspace_bytes(p, fs.FS_VARIANT_FLAT), dtype=t.uint8, device="cuda")
    for step in range(1000):
        p.step = step
        fs.check(fs.fs_sample(p, x_in.H, x_in.W, x_in.temp, None, idx[step], None, ws))
    draws = idx.cpu().numpy()
    l = O.logits_bf16(Hb, Wb)
    probs = [softmax(l[b] / float(temp[b])) for b in range(8)]
    pv = chi_square_rows_p([draws[:, b] for b in range(8)], probs)
    log(f"pooled chi-square over 8 rows x 1000 steps: p = {pv:.3f}")
    assert pv > 0.01


@pytest.mark.parametrize("B", [1, 4, 16, 64])
def test_mid_size_masked_grouped(B):
    wl = WORKLOADS[f"mid_b{B}"]
    log(f"mid-size B={B} d={wl.d} V={wl.V} n_valid={wl.n_valid}")
    Hb = hidden_bf16(B, wl.d)
    Wb = weights(wl.V, wl.d)
    temp = wl.temps()
    x_in = Inputs(Hb, Wb, temp)
    rows = np.arange(B)
    step = 3
    p = x_in.params(n_valid=wl.n_valid, tile_v=wl.tile_v, seed=PHILOX_SEED, step=step)
    gi, gs = run_flat(x_in, p)
    l, x, s = oracle_rows(Hb, Wb, rows, temp, wl.n_valid, PHILOX_SEED, step)
    check_flat(gi, gs, x, s, rows)
    assert np.all(gi < wl.n_valid)
    m, ti, L, go = run_grouped(x_in, p)
    om, oidx, oL, ogap = O.tile_records(x, s, wl.tile_v)
    check_values(m, om, what="tile max")
    check_values(L, oL, what="tile log-mass")
    pinned = ogap > TOL_GAP
    assert np.array_equal(ti[pinned], oidx[pinned])
    assert_pinned(pinned.ravel(), "tiles")
    # tiles 1185 and 1186 hold only masked ids; tile 1184 has 29 masked ids
    assert np.all(ti[:, 1185:] == -1) and np.all(np.isneginf(L[:, 1185:]))
    gidx, ggap, gt = O.sample_grouped(oidx, oL, temp, PHILOX_SEED, step)
    pin = (ggap > TOL_GAP) & np.array([gt[b] < 0 or ogap[b, gt[b]] > TOL_GAP for b in rows])
    assert np.array_equal(go[pin], gidx[pin])
    assert_pinned(pin, "grouped")
    check_grouped_unpinned(go, gidx, ti, pin)


def test_mid_size_grouped_histogram_1000_steps():
    """1000 steps of the hierarchical (Group-Gumbel-Max) sample at the
    mid-size shape, 4 rows, last 285 ids masked: the draws follow softmax(x)
    over the valid ids (the correctness paragraph's chi-square, p > 0.01)."""
    wl = WORKLOADS["mid_b4"]
    Hb = hidden_bf16(wl.B, wl.d)
    Wb = weights(wl.V, wl.d)
    temp = wl.temps()
    x_in = Inputs(Hb, Wb, temp)
    t = torch()
    p = x_in.params(n_valid=wl.n_valid, tile_v=wl.tile_v, seed=PHILOX_SEED)
    T = fs.fs_num_tiles(p)
    m = t.empty((wl.B, T), dtype=t.float32, device="cuda")
    ti = t.empty((wl.B, T), dtype=t.int32, device="cuda")
    L = t.empty((wl.B, T), dtype=t.float32, device="cuda")
    idx = t.empty((1000, wl.B), dtype=t.int32, device="cuda")
    ws = t.empty(fs.fs_workspace_bytes(p, fs.FS_VARIANT_GROUPED), dtype=t.uint8, device="cuda")
    for step in range(1000):
        p.step = step
        fs.check(fs.fs_sample_grouped(p, x_in.H, x_in.W, x_in.temp, None, m, ti, L, idx[step],
                                      ws))
    draws = host(idx)
    assert np.all((draws >= 0) & (draws < wl.n_valid))
    x = O.tempered(O.logits_bf16(Hb, Wb), temp, wl.n_valid)
    pv = chi_square_rows_p([draws[:, b] for b in range(wl.B)], [softmax(x[b]) for b in range(wl.B)])
    log(f"grouped: pooled chi-square over {wl.B} rows x 1000 steps: p = {pv:.3f}")
    assert pv > 0.01


def test_online_merge_histogram_1000_steps():
    """1000 steps of the online binary merge over 8 sequential chunks at the
    top-k shape (d=5120, V=152064, per-row temperatures): chunk records from
    the grouped entry point, then fs_merge_online; the draws of 8 rows follow
    softmax(x)."""
    wl = WORKLOADS["topk_b32"]
    B = 8
    Hb = hidden_bf16(wl.B, wl.d)[:B]
    Wb = weights(wl.V, wl.d)
    temp = wl.temps()[:B]
    x_in = Inputs(Hb, Wb, temp)
    t = torch()
    chunk = wl.V // wl.chunks
    p = x_in.params(tile_v=chunk, seed=PHILOX_SEED)
    C = fs.fs_num_tiles(p)
    assert C == wl.chunks
    m = t.empty((B, C), dtype=t.float32, device="cuda")
    ti = t.empty((B, C), dtype=t.int32, device="cuda")
    L = t.empty((B, C), dtype=t.float32, device="cuda")
    A = t.empty(B, dtype=t.float32, device="cuda")
    idx = t.empty((1000, B), dtype=t.int32, device="cuda")
    ws = t.empty(fs.fs_workspace_bytes(p, fs.FS_VARIANT_GROUPED), dtype=t.uint8, device="cuda")
    for step in range(1000):
        p.step = step
        fs.check(fs.fs_sample_grouped(p, x_in.H, x_in.W, x_in.temp, None, m, ti, L, None, ws))
        fs.check(fs.fs_merge_online(B, C, ti, L, x_in.temp, PHILOX_SEED, step, 0, idx[step], A))
    draws = host(idx)
    x = O.tempered(O.logits_bf16(Hb, Wb), temp, None)
    pv = chi_square_rows_p([draws[:, b] for b in range(B)], [softmax(x[b]) for b in range(B)])
    log(f"online merge: pooled chi-square over {B} rows x 1000 steps: p = {pv:.3f}")
    assert pv > 0.01


def _sampled_rows(B):
    return np.unique(np.concatenate([np.arange(0, B, 9), [B - 1]]))


@pytest.mark.parametrize("B", [128, 256])
def test_compute_lean_sampled_rows(B):
    wl = WORKLOADS[f"large_b{B}"]
    log(f"compute-leaning B={B} d={wl.d} V={wl.V}")
    Hb = hidden_bf16(B, wl.d)
    Wb = weights(wl.V, wl.d)
    temp = wl.temps()
    x_in = Inputs(Hb, Wb, temp)
    rows = _sampled_rows(B)
    for step in (0, 199):
        p = x_in.params(tile_v=wl.tile_v, seed=PHILOX_SEED, step=step)
        gi, gs = run_flat(x_in, p)
        l, x, s = oracle_rows(Hb, Wb, rows, temp, None, PHILOX_SEED, step)
        check_flat(gi, gs, x, s, rows, what=f"step {step} sampled rows")


@pytest.mark.parametrize("B", [128, 256])
def test_headline_vocab_large_batches(B):
    """B = 128 and 256 at the headline shape d=4096, V=151936 (the benchmark
    sweep's largest batches): the row-streaming kernel at 128 and 256 columns
    per workgroup, with a partial last tile in every workgroup range."""
    log(f"headline vocabulary B={B} d={D_HEAD} V={V_HEAD}")
    Hb = hidden_bf16(B, D_HEAD)
    Wb = weights(V_HEAD, D_HEAD)
    x_in = Inputs(Hb, Wb)
    rows = _sampled_rows(B)
    p = x_in.params(seed=PHILOX_SEED, step=5)
    gi, gs = run_flat(x_in, p)
    _, x, s = oracle_rows(Hb, Wb, rows, None, None, PHILOX_SEED, 5)
    check_flat(gi, gs, x, s, rows, what=f"B={B} sampled rows")


def test_topk_and_online_merge():
    wl = WORKLOADS["topk_b32"]
    log(f"top-k/online B={wl.B} d={wl.d} V={wl.V} k={wl.k} chunks={wl.chunks}")
    Hb = hidden_bf16(wl.B, wl.d)
    Wb = weights(wl.V, wl.d)
    temp = wl.temps()
    x_in = Inputs(Hb, Wb, temp)
    rows = np.arange(wl.B)
    step = 11
    p = x_in.params(tile_v=wl.tile_v, seed=PHILOX_SEED, step=step)
    l, x, s = oracle_rows(Hb, Wb, rows, temp, None, PHILOX_SEED, step)
    for k in (wl.k, 1000):
        # k = 1000, the pages' largest benchmarked k: lists of whole
        # workgroup ranges and the binned stage-2 selection
        tk = run_topk(x_in, p, k)
        oi, _, _ = O.topk_sample(x, s, k)
        pin = O.topk_pick_margin(x, s, k, TOL_X) > TOL_GAP
        assert np.array_equal(tk[pin], oi[pin])
        assert_pinned(pin, f"top-{k}")
    tp = run_topp(x_in, p, 1000, 0.95)
    oi, _, _, _ = O.topk_topp_sample(x, s, 1000, 0.95)
    pin = O.topp_pick_margin(x, s, 1000, 0.95, TOL_X, TOL_MASS) > TOL_GAP
    assert np.array_equal(tp[pin], oi[pin])
    assert_pinned(pin, "top-1000 top-p 0.95")
    # online merge over 8 sequential chunks of V/8 ids: chunk records from the
    # grouped entry point with one tile per chunk, then the binary merge
    chunk = wl.V // wl.chunks
    pc = x_in.params(tile_v=chunk, seed=PHILOX_SEED, step=step)
    m, ti, L, _ = run_grouped(x_in, pc, with_sample=False)
    assert ti.shape[1] == wl.chunks
    om, oidx, oL, cgap = O.tile_records(x, s, chunk)
    check_values(L, oL, what="chunk log-mass")
    gz, gA = run_merge(ti, L, temp, PHILOX_SEED, step)
    oz, oA, omarg = O.online_merge(oidx, oL, temp, PHILOX_SEED, step)
    check_values(gA, oA, what="merged log-mass")
    # the merge's decisions use the log-masses alone; the chunk it lands on
    # then gives its own winner, which must be pinned
    sel = np.where(oz >= 0, oz // chunk, 0)
    pin = (omarg > 1e-2) & (cgap[rows, sel] > TOL_GAP)
    assert np.array_equal(gz[pin], oz[pin])
    assert_pinned(pin, "online merge")
    # the merged log-mass is the log-sum-exp over the whole vocabulary
    check_values(gA, [O.log_sum_exp(x[b]) for b in rows], what="total log-mass")


def test_vocab_shards_merge_to_the_unsharded_call():
    """The headline call split over G vocabulary shards (rank g of a G-way
    tensor-parallel split holds W rows [g V/G, (g+1) V/G) and passes
    v_offset = g V/G).  The noise is keyed by the global id, so the best of
    the shards' flat winners (largest score, lowest id on ties) is the
    unsharded sample bit for bit; the shards' (winner, log-mass) records
    merged by the online binary merge agree with the oracle's merge of its
    own shard records (FlashSampling Abstract and explainer, tensor-parallel
    paragraph)."""
    t = torch()
    B = 32
    Hb = hidden_bf16(B, D_HEAD)
    Wb = weights(V_HEAD, D_HEAD)
    x_in = Inputs(Hb, Wb)
    rows = np.arange(B)
    step = 7
    p = x_in.params(seed=PHILOX_SEED, step=step)
    full_i, full_s = run_flat(x_in, p)
    _, x, s = oracle_rows(Hb, Wb, rows, None, None, PHILOX_SEED, step)
    check_flat(full_i, full_s, x, s, rows, what="unsharded")
    for G in (2, 4, 8):
        vs = V_HEAD // G
        best_s = np.full(B, -np.inf)
        best_i = np.full(B, -1, np.int64)
        z = np.empty((B, G), np.int64)
        Lg = np.empty((B, G), np.float64)
        for g in range(G):
            off = g * vs
            Ws = x_in.W[off:off + vs]
            ps = fs.params(B, D_HEAD, vs, v_offset=off, seed=PHILOX_SEED, step=step)
            idx = t.empty(B, dtype=t.int32, device="cuda")
            sc = t.empty(B, dtype=t.float32, device="cuda")
            ws = t.empty(fs.fs_workspace_bytes(ps, fs.FS_VARIANT_FLAT), dtype=t.uint8,
                         device="cuda")
            fs.check(fs.fs_sample(ps, x_in.H, Ws, None, None, idx, sc, ws), f"shard {g}/{G}")
            pg = fs.params(B, D_HEAD, vs, v_offset=off, tile_v=vs, seed=PHILOX_SEED, step=step)
            tm = t.empty((B, 1), dtype=t.float32, device="cuda")
            ti = t.empty((B, 1), dtype=t.int32, device="cuda")
            tl = t.empty((B, 1), dtype=t.float32, device="cuda")
            gws = t.empty(fs.fs_workspace_bytes(pg, fs.FS_VARIANT_GROUPED), dtype=t.uint8,
                          device="cuda")
            fs.check(fs.fs_sample_grouped(pg, x_in.H, Ws, None, None, tm, ti, tl, None, gws),
                     f"grouped shard {g}/{G}")
            t.cuda.synchronize()
            si, ss = host(idx).astype(np.int64), host(sc).astype(np.float64)
            assert np.all((si >= off) & (si < off + vs))
            better = (ss > best_s) | ((ss == best_s) & (si < best_i))
            best_s = np.where(better, ss, best_s)
            best_i = np.where(better, si, best_i)
            z[:, g] = host(ti)[:, 0]
            Lg[:, g] = host(tl)[:, 0]
            assert np.array_equal(z[:, g], si)   # one tile per shard: the shard's winner
        assert np.array_equal(best_i, full_i), f"G={G}: shard winners differ from the call"
        assert np.array_equal(best_s.astype(np.float32).view(np.uint32),
                              full_s.astype(np.float32).view(np.uint32))
        gz, gA = run_merge(z, Lg, None, PHILOX_SEED, step)
        om, oidx, oL, sgap = O.tile_records(x, s, vs)
        check_values(Lg, oL, what=f"G={G} shard log-mass")
        oz, oA, omarg = O.online_merge(oidx, oL, None, PHILOX_SEED, step)
        check_values(gA, oA, what=f"G={G} merged log-mass")
        sel = np.where(oz >= 0, oz // vs, 0)
        pin = (omarg > 1e-2) & (sgap[rows, sel] > TOL_GAP)
        assert np.array_equal(gz[pin], oz[pin])
        assert_pinned(pin, f"G={G} shard merge")


def test_topk_topp_histogram():
    """Top-40 then top-p 0.9 at the d=5120, V=152064 shape: over 600 decode
    steps the draws of 8 rows follow softmax(x) renormalised over the kept
    prefix of the top-40 set (pooled chi-square)."""
    wl = WORKLOADS["topk_b32"]
    B, k, top_p, steps = 8, wl.k, 0.9, 600
    Hb = hidden_bf16(wl.B, wl.d)[:B].copy()
    Wb = weights(wl.V, wl.d)
    temp = wl.temps()[:B]
    x_in = Inputs(Hb, Wb, temp)
    t = torch()
    idx = t.empty((steps, B), dtype=t.int32, device="cuda")
    p = x_in.params(tile_v=wl.tile_v, seed=PHILOX_SEED)
    ws = t.empty(fs.fs_workspace_bytes(p, fs.FS_VARIANT_TOPK, k), dtype=t.uint8, device="cuda")
    for step in range(steps):
        p.step = step
        fs.check(fs.fs_sample_topk_topp(p, x_in.H, x_in.W, x_in.temp, None, k, top_p, idx[step],
                                        ws))
    draws = idx.cpu().numpy()
    x = O.tempered(O.logits_bf16(Hb, Wb), temp)
    _, _, margin, cut = O.topk_topp_sample(x, x, k, top_p)
    rows = [b for b in range(B) if margin[b] > 1e-3 and cut[b] > 1e-4]   # sets pinned
    assert len(rows) >= B // 2
    probs = []
    for b in rows:
        order = np.lexsort((np.arange(wl.V), -x[b]))[:k]
        q = softmax(x[b, order])
        excl = np.concatenate([[0.0], np.cumsum(q)[:-1]])
        kept = order[excl < top_p]
        pb = np.zeros(wl.V)
        pb[kept] = softmax(x[b, kept])
        probs.append(pb)
        assert np.all(np.isin(draws[:, b], kept))
    pv = chi_square_rows_p([draws[:, b] for b in rows], probs)
    log(f"top-{k} top-p {top_p}: pooled chi-square over {len(rows)} rows x {steps} steps: "
        f"p = {pv:.3f}")
    assert pv > 0.01
