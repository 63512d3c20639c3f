"""GPU tests of the graph-friendly form of the calls: one Philox seed per batch
row (per-request seeds) and the decode step read from device memory, so that a
captured HIP graph replays with fresh noise.  Results are compared with the
oracle (per-row seeds), with the same calls given the step on the host
(bit-identical), and across graph replays that advance the step on the device.
"""
import numpy as np
import pytest

import lm_head_gumbel_amd as fs
from lm_head_gumbel_amd.inputs import hidden_bf16, weights_bf16
from oracle import fs_oracle as O
from gpu_util import (Inputs, TOL_CUT, TOL_GAP, check_index_rows, check_values, dev, host, log, run_flat,
                      run_grouped, run_logits, run_multinomial, run_topk, run_topp, torch,
                      workspace)

pytestmark = pytest.mark.gpu

SEEDS = np.array([3, 0xDEADBEEF12345678, 3, 77, 2 ** 63 + 5, 1], dtype=np.uint64)


def problem(B=6, d=256, V=3000, seed=0):
    rng = np.random.default_rng(50 + seed)
    Hb = hidden_bf16(B, d, seed=31 + seed)
    Wb = weights_bf16(V, d, std=0.05, seed=32 + seed)
    temp = rng.uniform(0.4, 1.4, B).astype(np.float32)
    temp[-1] = 0.0   # one greedy row
    return Hb, Wb, temp


def seeds_dev(B):
    return dev(SEEDS[:B].view(np.int64))


def test_per_row_seeds_match_oracle():
    Hb, Wb, temp = problem()
    B = Hb.shape[0]
    x_in = Inputs(Hb, Wb, temp)
    sd = seeds_dev(B)
    step = 9
    p = x_in.params(seed=1234, step=step, tile_v=128, seeds=sd)
    l = O.logits_bf16(Hb, Wb)
    r = O.run_call(l, temp, None, None, SEEDS[:B], step, 0, 128)
    log("per-row seeds: flat, grouped, top-k, multinomial, online merge")
    gi, gs = run_flat(x_in, p)
    check_index_rows(gi, r["flat_idx"], r["flat_gap"], r["s"], what="flat")
    m, ti, L, go = run_grouped(x_in, p)
    check_values(m, r["tile_m"], what="tile max")
    check_values(L, r["tile_L"], what="tile log-mass")
    gt = r["grp_tile"]
    pin = (r["grp_gap"] > TOL_GAP) & np.array([gt[b] < 0 or r["tile_gap"][b, gt[b]] > TOL_GAP
                                               for b in range(B)])
    assert np.array_equal(go[pin], r["grp_idx"][pin])
    for k in (1, 7, 40):
        tk = run_topk(x_in, p, k)
        oi, ogap, omarg = O.topk_sample(r["x"], r["s"], k)
        pin = (ogap > TOL_GAP) & (omarg > 1e-3)
        assert np.array_equal(tk[pin], oi[pin])
    gl, gl_dev = run_logits(x_in, p)
    mi = run_multinomial(x_in, p, gl_dev)
    oi, omarg = O.multinomial(r["x"], temp, SEEDS[:B], step)
    pin = omarg > 1e-4
    assert np.array_equal(mi[pin], oi[pin])
    # the online merge keyed per row, on the GPU's own chunk records
    t = torch()
    out = t.full((B,), -7, dtype=t.int32, device="cuda")
    A = t.zeros(B, dtype=t.float32, device="cuda")
    fs.check(fs.fs_merge_online_dev(B, ti.shape[1], dev(ti.astype(np.int32)),
                                    dev(L.astype(np.float32)), x_in.temp, 1234, sd, step, None,
                                    0, out, A), "merge")
    t.cuda.synchronize()
    oz, oA, omarg = O.online_merge(ti, L, temp, SEEDS[:B], step)
    pin = omarg > 1e-2
    assert np.array_equal(host(out)[pin], oz[pin])
    # rows 0 and 2 share a seed: their noise is that seed's, not the call's
    r1 = O.run_call(l, temp, None, None, 1234, step, 0, 128)
    assert not np.array_equal(r["s"][1], r1["s"][1])


def test_device_step_is_the_host_step():
    Hb, Wb, temp = problem(B=5, seed=1)
    x_in = Inputs(Hb, Wb, temp)
    t = torch()
    for step in (0, 41, 0xFFFFFFFF):
        sp = dev(np.array([step], np.uint32).view(np.int32))
        ph = x_in.params(seed=99, step=step, tile_v=64)
        pd = x_in.params(seed=99, step=12345, tile_v=64, step_ptr=sp)   # the host value is ignored
        log(f"device step {step}")
        a, b = run_flat(x_in, ph), run_flat(x_in, pd)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        ga, gb = run_grouped(x_in, ph), run_grouped(x_in, pd)
        for u, v in zip(ga, gb):
            assert np.array_equal(u, v)
        assert np.array_equal(run_topk(x_in, ph, 7), run_topk(x_in, pd, 7))
        assert np.array_equal(run_topp(x_in, ph, 7, 0.8), run_topp(x_in, pd, 7, 0.8))


def test_graph_replay_advances_the_device_step():
    """fs_sample captured once into a graph together with an increment of the
    device step: every replay equals an eager call with the next step."""
    t = torch()
    Hb, Wb, temp = problem(B=8, d=512, V=4000, seed=2)
    x_in = Inputs(Hb, Wb, temp)
    step_t = t.zeros(1, dtype=t.int32, device="cuda")
    sd = seeds_dev(6)
    seeds8 = t.cat([sd, sd[:2]])
    p = x_in.params(seed=5, step=0, tile_v=128, step_ptr=step_t, seeds=seeds8)
    idx = t.full((x_in.B,), -7, dtype=t.int32, device="cuda")
    score = t.zeros(x_in.B, dtype=t.float32, device="cuda")
    ws = workspace(p, fs.FS_VARIANT_FLAT)
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):   # warm-up outside the capture
        fs.check(fs.fs_sample(p, x_in.H, x_in.W, x_in.temp, None, idx, score, ws), "warm-up")
    t.cuda.current_stream().wait_stream(s)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        fs.check(fs.fs_sample(p, x_in.H, x_in.W, x_in.temp, None, idx, score, ws), "capture")
        step_t.add_(1)
    t.cuda.synchronize()
    step_t.zero_()
    t.cuda.synchronize()
    seeds_h = host(seeds8).view(np.uint64)
    for rep in range(5):
        g.replay()
        t.cuda.synchronize()
        got_i, got_s = host(idx).copy(), host(score).copy()
        assert int(host(step_t)[0]) == rep + 1
        # eager reference with the host step and the same per-row seeds
        pe = x_in.params(seed=5, step=rep, tile_v=128, seeds=seeds8)
        want_i, want_s = run_flat(x_in, pe)
        log(f"replay {rep}: {np.count_nonzero(got_i == want_i)}/{x_in.B} equal")
        assert np.array_equal(got_i, want_i) and np.array_equal(got_s, want_s)
        # and against the oracle
        r = O.run_call(O.logits_bf16(Hb, Wb), temp, None, None, seeds_h, rep, 0, 128)
        check_index_rows(got_i, r["flat_idx"], r["flat_gap"], r["s"], what=f"replay {rep}")


SCHED_TAG = 0x4C4D4847554D4231
SCHED_TAG32 = 0x53434844


def sched_block(ws):
    """The unit scheduler block at the end of a flat workspace: (tag, word)."""
    tail = host(ws[-256:-240]).view(np.uint64)
    return int(tail[0]), int(tail[1])


def test_flat_ticket_order_matches_fixed_order():
    """A flat workspace used again hands stage-1 units out by ticket (the first
    call, on a zeroed buffer, walks the fixed strided order and leaves the
    scheduler block initialised).  Every call, eager and replayed from a
    graph, equals the same call on a fresh zeroed workspace bit for bit and
    the oracle; after each call the ticket count is back at 0."""
    t = torch()
    B, d, V = 32, 512, 40000   # 1250 units of two blocks: the ticket order applies
    Hb = hidden_bf16(B, d, seed=71)
    Wb = weights_bf16(V, d, std=0.05, seed=72)
    temp = np.random.default_rng(73).uniform(0.5, 1.3, B).astype(np.float32)
    x_in = Inputs(Hb, Wb, temp)
    l = O.logits_bf16(Hb, Wb)

    def fresh(step):
        p = x_in.params(seed=11, step=step)
        idx = t.full((B,), -7, dtype=t.int32, device="cuda")
        score = t.zeros(B, dtype=t.float32, device="cuda")
        ws0 = t.zeros(fs.fs_workspace_bytes(p, fs.FS_VARIANT_FLAT), dtype=t.uint8, device="cuda")
        fs.check(fs.fs_sample(p, x_in.H, x_in.W, x_in.temp, None, idx, score, ws0), "fresh")
        t.cuda.synchronize()
        return host(idx).copy(), host(score).copy()

    p = x_in.params(seed=11, step=0)
    ws = t.zeros(fs.fs_workspace_bytes(p, fs.FS_VARIANT_FLAT), dtype=t.uint8, device="cuda")
    assert sched_block(ws) == (0, 0)
    idx = t.full((B,), -7, dtype=t.int32, device="cuda")
    score = t.zeros(B, dtype=t.float32, device="cuda")
    for step in range(4):
        p.step = step
        fs.check(fs.fs_sample(p, x_in.H, x_in.W, x_in.temp, None, idx, score, ws), "reused")
        t.cuda.synchronize()
        assert sched_block(ws) == (SCHED_TAG, SCHED_TAG32 << 32), "scheduler block after a call"
        gi, gs = host(idx).copy(), host(score).copy()
        wi, wsc = fresh(step)
        log(f"step {step}: {np.count_nonzero(gi == wi)}/{B} equal to the fixed order")
        assert np.array_equal(gi, wi) and np.array_equal(gs, wsc)
        r = O.run_call(l, temp, None, None, 11, step, 0, 128)
        check_index_rows(gi, r["flat_idx"], r["flat_gap"], r["s"], what=f"step {step}")

    # a workspace full of arbitrary bytes (a fresh allocation's content):
    # that call walks the fixed order and sets the block up
    g = t.Generator(device="cuda")
    g.manual_seed(5)
    ws_r = t.randint(0, 256, (ws.numel(),), generator=g, device="cuda", dtype=t.int32).to(t.uint8)
    p.step = 7
    fs.check(fs.fs_sample(p, x_in.H, x_in.W, x_in.temp, None, idx, score, ws_r), "random ws")
    t.cuda.synchronize()
    wi, wsc = fresh(7)
    assert np.array_equal(host(idx), wi) and np.array_equal(host(score), wsc)
    assert sched_block(ws_r) == (SCHED_TAG, SCHED_TAG32 << 32)

    # graph replays with the device step advancing
    step_t = t.zeros(1, dtype=t.int32, device="cuda")
    pg = x_in.params(seed=11, step=0, step_ptr=step_t)
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        fs.check(fs.fs_sample(pg, x_in.H, x_in.W, x_in.temp, None, idx, score, ws), "warm-up")
    t.cuda.current_stream().wait_stream(s)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        fs.check(fs.fs_sample(pg, x_in.H, x_in.W, x_in.temp, None, idx, score, ws), "capture")
        step_t.add_(1)
    t.cuda.synchronize()
    step_t.zero_()
    t.cuda.synchronize()
    for rep in range(4):
        g.replay()
        t.cuda.synchronize()
        assert sched_block(ws) == (SCHED_TAG, SCHED_TAG32 << 32), "scheduler block after a replay"
        gi, gs = host(idx).copy(), host(score).copy()
        wi, wsc = fresh(rep)
        log(f"replay {rep}: {np.count_nonzero(gi == wi)}/{B} equal to the fixed order")
        assert np.array_equal(gi, wi) and np.array_equal(gs, wsc)


def test_topk_ticket_order_matches_fixed_order():
    """The same for fs_sample_topk (k <= 64, where one stage-2 kernel follows
    and sets the block up; its scheduler block is the last 256 bytes of the
    top-k workspace): calls on a reused workspace, and top-p after top-k, equal
    fresh-workspace calls bit for bit and the oracle."""
    t = torch()
    B, d, V, k = 32, 512, 40000, 40
    Hb = hidden_bf16(B, d, seed=81)
    Wb = weights_bf16(V, d, std=0.05, seed=82)
    temp = np.random.default_rng(83).uniform(0.5, 1.3, B).astype(np.float32)
    x_in = Inputs(Hb, Wb, temp)
    l = O.logits_bf16(Hb, Wb)

    def call(p, ws, top_p):
        idx = t.full((B,), -7, dtype=t.int32, device="cuda")
        if top_p < 1:
            fs.check(fs.fs_sample_topk_topp(p, x_in.H, x_in.W, x_in.temp, None, k, top_p, idx, ws))
        else:
            fs.check(fs.fs_sample_topk(p, x_in.H, x_in.W, x_in.temp, None, k, idx, ws))
        t.cuda.synchronize()
        return host(idx).astype(np.int64)

    p = x_in.params(seed=13, step=0)
    n = fs.fs_workspace_bytes(p, fs.FS_VARIANT_TOPK, k)
    ws = t.zeros(n, dtype=t.uint8, device="cuda")
    for step in range(4):
        for top_p in (1.0, 0.8):
            p.step = step
            got = call(p, ws, top_p)
            assert sched_block(ws) == (SCHED_TAG, SCHED_TAG32 << 32), "scheduler block after a call"
            want = call(p, t.zeros(n, dtype=t.uint8, device="cuda"), top_p)
            log(f"step {step} top_p {top_p}: {np.count_nonzero(got == want)}/{B} equal to the fixed order")
            assert np.array_equal(got, want)
            r = O.run_call(l, temp, None, None, 13, step, 0, 128)
            if top_p < 1:
                oi, ogap, omarg, ocut = O.topk_topp_sample(r["x"], r["s"], k, top_p)
                pin = (ogap > TOL_GAP) & (omarg > 1e-3) & (ocut > TOL_CUT)
            else:
                oi, ogap, omarg = O.topk_sample(r["x"], r["s"], k)
                pin = (ogap > TOL_GAP) & (omarg > 1e-3)
            assert pin.sum() >= B // 4
            assert np.array_equal(got[pin], oi[pin])
