#!/usr/bin/env python3
"""Benchmark of fused LM-head Gumbel sampling (libfs) on one MI355X.

Workload: the LM-head shape d=4096, V=151936 with synthetic bf16 inputs
(H ~ N(0,1), W ~ N(0, 0.02^2), drawn on the device from fixed seeds), Philox
seed 1234, the decode step incremented every call.  A step is one fs_sample
call: the fused stage-1 kernel (stream W once, logits on chip, temperature,
mask, Philox-Gumbel noise, per-workgroup winners) plus the stage-2 reduction.

Prints ONE JSON line.  `value` is fused calls/s at the headline batch;
`roofline` rates the stage-1 kernel (timed alone with HIP events on the
launch stream) against MI355X's 8 TB/s HBM peak from the algorithmic bytes
2*V*d + 2*B*d + 4*B (W, H and temperatures read once); `sweep` repeats the
measurement over B = 1..256 with the unfused fs_logits + fs_multinomial
baseline beside it; `cpu_baseline` times the CPU oracle on a bounded slice of
the vocabulary and scales it to one full call.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused sample calls/s + HBM GB/s (% peak), d=4096 V=151936, B=1..256"
PEAK_HBM = 8.0e12          # bytes/s, MI355X HBM3E
PEAK_BF16 = 2.5e15         # dense bf16 MFMA flop/s
D, V = 4096, 151936
SEED = 1234


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def alg_bytes(B, d=D, v=V):
    return 2.0 * v * d + 2.0 * B * d + 4.0 * B


class Timer:
    """HIP events on the current (library launch) stream.  The mean per call
    comes from n back-to-back calls between two events (the timed region);
    the per-call distribution from a second pass of n calls with an event
    after each call (an event costs the stream about 3 us, so recording one
    per call would inflate the mean)."""

    def __init__(self, torch):
        self.t = torch

    def run(self, fn, n):
        """Mean seconds per call, wall seconds of the timed region, and the
        per-call seconds of the second pass."""
        t = self.t
        s = t.cuda.current_stream()
        e0 = t.cuda.Event(enable_timing=True)
        e1 = t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record(s)
        for i in range(n):
            fn(i)
        e1.record(s)
        t.cuda.synchronize()
        wall = time.perf_counter() - w0
        mean = e0.elapsed_time(e1) / 1e3 / n
        ev = [t.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        ev[0].record(s)
        for i in range(n):
            fn(i)
            ev[i + 1].record(s)
        t.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) / 1e3 for i in range(n)]
        return mean, wall, per


def pct(per, q):
    """q-th percentile of per-call seconds, in microseconds."""
    import numpy as np
    return float(np.percentile(np.asarray(per) * 1e6, q))


def dist(per):
    return {"p10_us": pct(per, 10), "p50_us": pct(per, 50), "p90_us": pct(per, 90)}


def make_inputs(torch, B, d=D, v=V):
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    W = (torch.randn((v, d), generator=g, device="cuda", dtype=torch.float32) * 0.02
         ).to(torch.bfloat16)
    g.manual_seed(1)
    H = torch.randn((B, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    return H, W


def bench_batch(torch, fs, H_all, W, B, steps, warmup, unfused=True, variants=False):
    H = H_all[:B].contiguous()
    timer = Timer(torch)
    p = fs.params(B, D, V, seed=SEED)
    idx = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(fs.fs_workspace_bytes(p, fs.FS_VARIANT_FLAT), dtype=torch.uint8,
                     device="cuda")

    def call(i):
        p.step = i
        fs.check(fs.fs_sample(p, H, W, None, None, idx, None, ws), "fs_sample")

    def stage1(i):
        p.step = i
        fs.check(fs.fs_sample_stage1(p, H, W, None, None, ws), "fs_sample_stage1")

    for i in range(warmup):
        call(i)
    t_call, wall, per_call = timer.run(call, steps)
    for i in range(max(2, warmup // 2)):
        stage1(i)
    t_k1, _, per_k1 = timer.run(stage1, steps)
    res = {"B": B, "calls_per_s": 1.0 / t_call, "tokens_per_s": B / t_call,
           "us_per_call": t_call * 1e6, "call": dist(per_call),
           "stage1_us": t_k1 * 1e6, "stage1": dist(per_k1),
           "hbm_GBps": alg_bytes(B) / t_k1 / 1e9,
           "hbm_frac": alg_bytes(B) / t_k1 / PEAK_HBM,
           "mfma_frac": 2.0 * B * D * V / t_k1 / PEAK_BF16,
           "wall_s": wall}
    if unfused:
        logits = torch.empty((B, V), dtype=torch.float32, device="cuda")
        mws = torch.empty(fs.fs_workspace_bytes(p, fs.FS_VARIANT_MULTINOMIAL),
                          dtype=torch.uint8, device="cuda")
        lws = torch.empty(fs.fs_workspace_bytes(p, fs.FS_VARIANT_LOGITS),
                          dtype=torch.uint8, device="cuda")

        def base(i):
            p.step = i
            fs.check(fs.fs_logits(p, H, W, logits, lws), "fs_logits")
            fs.check(fs.fs_multinomial(p, logits, None, None, idx, mws), "fs_multinomial")

        for i in range(max(2, warmup // 2)):
            base(i)
        t_base = timer.run(base, max(10, steps // 4))[0]
        res["unfused_calls_per_s"] = 1.0 / t_base
        res["fused_speedup"] = t_base / t_call
        del logits
        # for scale: the library GEMM alone (W times H^T into bf16 logits, no
        # sampling; a plain 2-D product of contiguous operands)
        Ht = H.t().contiguous()
        out = torch.empty((V, B), dtype=torch.bfloat16, device="cuda")
        for i in range(3):
            torch.mm(W, Ht, out=out)
        res["library_gemm_us"] = timer.run(lambda i: torch.mm(W, Ht, out=out),
                                           max(10, steps // 4))[0] * 1e6
        del out, Ht
    if variants:
        # the same call replayed from a HIP graph: the step lives on the device
        # and the graph advances it, so every replay draws fresh noise
        step_t = torch.zeros(1, dtype=torch.int32, device="cuda")
        pg = fs.params(B, D, V, seed=SEED, step_ptr=step_t)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fs.check(fs.fs_sample(pg, H, W, None, None, idx, None, ws), "graph warm-up")
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fs.check(fs.fs_sample(pg, H, W, None, None, idx, None, ws), "graph capture")
            step_t.add_(1)
        for i in range(3):
            graph.replay()
        res["graph_calls_per_s"] = 1.0 / timer.run(lambda i: graph.replay(), steps)[0]
        del graph

        T = fs.fs_num_tiles(p)
        tm = torch.empty((B, T), dtype=torch.float32, device="cuda")
        ti = torch.empty((B, T), dtype=torch.int32, device="cuda")
        tl = torch.empty((B, T), dtype=torch.float32, device="cuda")
        gws = torch.empty(fs.fs_workspace_bytes(p, fs.FS_VARIANT_GROUPED), dtype=torch.uint8,
                          device="cuda")

        def grouped(i):
            p.step = i
            fs.check(fs.fs_sample_grouped(p, H, W, None, None, tm, ti, tl, idx, gws), "grouped")

        for i in range(max(3, warmup // 2)):
            grouped(i)
        res["grouped_calls_per_s"] = 1.0 / timer.run(grouped, steps)[0]
        k = 40
        kws = torch.empty(fs.fs_workspace_bytes(p, fs.FS_VARIANT_TOPK, k), dtype=torch.uint8,
                          device="cuda")

        def topk(i):
            p.step = i
            fs.check(fs.fs_sample_topk(p, H, W, None, None, k, idx, kws), "topk")

        for i in range(max(3, warmup // 2)):
            topk(i)
        res["topk40_calls_per_s"] = 1.0 / timer.run(topk, steps)[0]

        def topp(i):
            p.step = i
            fs.check(fs.fs_sample_topk_topp(p, H, W, None, None, k, 0.9, idx, kws), "topp")

        for i in range(max(3, warmup // 2)):
            topp(i)
        res["topk40_topp0.9_calls_per_s"] = 1.0 / timer.run(topp, steps)[0]
    return res


def _gpu_weights(torch, v, d, std=0.02, seed=0):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return (torch.randn((v, d), generator=g, device="cuda", dtype=torch.float32) * std
            ).to(torch.bfloat16)


def _gpu_hidden(torch, B, d, seed=1):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn((B, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def bench_workloads(torch, fs, steps, W_head):
    """The other configured workloads at their own shapes (secondary lines):
    small-model flat, mid-size masked grouped, compute-leaning flat with
    per-row temperatures, top-k and online merge at d=5120, and the stage-1
    kernel on one vocabulary shard (V/G rows, v_offset = the shard start) as
    a rank of a G-way vocabulary split would run it."""
    from lm_head_gumbel_amd.inputs import WORKLOADS
    timer = Timer(torch)
    out = []
    n = max(10, steps // 2)

    def timed(fn):
        for i in range(5):
            fn(i)
        t, _, per = timer.run(fn, n)
        return t, per

    def line(name, wl, what, tp, extra=None):
        t, per = tp
        r = {"workload": name, "B": wl.B, "d": wl.d, "V": wl.V, "what": what,
             "calls_per_s": 1.0 / t, "us_per_call": t * 1e6, "p50_us": pct(per, 50),
             "hbm_GBps": alg_bytes(wl.B, wl.d, wl.V) / t / 1e9,
             "hbm_frac": alg_bytes(wl.B, wl.d, wl.V) / t / PEAK_HBM,
             "mfma_frac": 2.0 * wl.B * wl.d * wl.V / t / PEAK_BF16}
        if extra:
            r.update(extra)
        log(json.dumps({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}))
        out.append(r)

    cache = {}

    def weights(v, d):
        if (v, d) not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            cache[(v, d)] = _gpu_weights(torch, v, d)
        return cache[(v, d)]

    for name in ("small_b1", "small_b8", "small_b32", "mid_b1", "mid_b4", "mid_b16", "mid_b64",
                 "large_b128", "large_b256", "topk_b32"):
        wl = WORKLOADS[name]
        W = weights(wl.V, wl.d)
        H = _gpu_hidden(torch, wl.B, wl.d)
        temp = torch.from_numpy(wl.temps()).cuda()
        p = fs.params(wl.B, wl.d, wl.V, n_valid=wl.n_valid, tile_v=wl.tile_v, seed=SEED)
        idx = torch.empty(wl.B, dtype=torch.int32, device="cuda")
        ws = torch.empty(fs.fs_workspace_bytes(p, fs.FS_VARIANT_FLAT), dtype=torch.uint8,
                         device="cuda")

        def flat(i):
            p.step = i
            fs.check(fs.fs_sample(p, H, W, temp, None, idx, None, ws), name)

        line(name, wl, "flat fs_sample", timed(flat))

        def flat_stage1(i):
            p.step = i
            fs.check(fs.fs_sample_stage1(p, H, W, temp, None, ws), name)

        line(name, wl, "flat stage 1 alone (fs_sample_stage1)", timed(flat_stage1))

        # the unfused baseline at this shape: logits written to HBM, then the
        # two-pass inverse-CDF draw
        logits = torch.empty((wl.B, wl.V), dtype=torch.float32, device="cuda")
        lws = torch.empty(fs.fs_workspace_bytes(p, fs.FS_VARIANT_LOGITS), dtype=torch.uint8,
                          device="cuda")
        mws = torch.empty(fs.fs_workspace_bytes(p, fs.FS_VARIANT_MULTINOMIAL), dtype=torch.uint8,
                          device="cuda")

        def unfused(i):
            p.step = i
            fs.check(fs.fs_logits(p, H, W, logits, lws), name)
            fs.check(fs.fs_multinomial(p, logits, temp, None, idx, mws), name)

        line(name, wl, "unfused fs_logits + fs_multinomial", timed(unfused))
        del logits, lws, mws
        if name.startswith("mid_"):
            T = fs.fs_num_tiles(p)
            tm = torch.empty((wl.B, T), dtype=torch.float32, device="cuda")
            ti = torch.empty((wl.B, T), dtype=torch.int32, device="cuda")
            tl = torch.empty((wl.B, T), dtype=torch.float32, device="cuda")
            gws = torch.empty(fs.fs_workspace_bytes(p, fs.FS_VARIANT_GROUPED), dtype=torch.uint8,
                              device="cuda")

            def grouped(i):
                p.step = i
                fs.check(fs.fs_sample_grouped(p, H, W, temp, None, tm, ti, tl, idx, gws), name)

            line(name, wl, "grouped fs_sample_grouped (masked tail, hierarchical resample)",
                 timed(grouped))
        if name == "topk_b32":
            kws = torch.empty(fs.fs_workspace_bytes(p, fs.FS_VARIANT_TOPK, wl.k),
                              dtype=torch.uint8, device="cuda")

            def topk(i):
                p.step = i
                fs.check(fs.fs_sample_topk(p, H, W, temp, None, wl.k, idx, kws), name)

            line(name, wl, f"top-{wl.k} fs_sample_topk", timed(topk))

            def topp(i):
                p.step = i
                fs.check(fs.fs_sample_topk_topp(p, H, W, temp, None, wl.k, 0.9, idx, kws), name)

            line(name, wl, f"top-{wl.k} then top-p 0.9 fs_sample_topk_topp", timed(topp))
            # the pages' largest benchmarked k
            kl = 1000
            lws = torch.empty(fs.fs_workspace_bytes(p, fs.FS_VARIANT_TOPK, kl),
                              dtype=torch.uint8, device="cuda")

            def topk_l(i):
                p.step = i
                fs.check(fs.fs_sample_topk(p, H, W, temp, None, kl, idx, lws), name)

            line(name, wl, f"top-{kl} fs_sample_topk", timed(topk_l))

            def topp_l(i):
                p.step = i
                fs.check(fs.fs_sample_topk_topp(p, H, W, temp, None, kl, 0.9, idx, lws), name)

            line(name, wl, f"top-{kl} then top-p 0.9 fs_sample_topk_topp", timed(topp_l))
            del lws
            chunk = wl.V // wl.chunks
            pc = fs.params(wl.B, wl.d, wl.V, tile_v=chunk, seed=SEED)
            C = fs.fs_num_tiles(pc)
            tm = torch.empty((wl.B, C), dtype=torch.float32, device="cuda")
            ti = torch.empty((wl.B, C), dtype=torch.int32, device="cuda")
            tl = torch.empty((wl.B, C), dtype=torch.float32, device="cuda")
            oL = torch.empty(wl.B, dtype=torch.float32, device="cuda")
            gws = torch.empty(fs.fs_workspace_bytes(pc, fs.FS_VARIANT_GROUPED), dtype=torch.uint8,
                              device="cuda")

            def online(i):
                pc.step = i
                fs.check(fs.fs_sample_grouped(pc, H, W, temp, None, tm, ti, tl, None, gws), name)
                fs.check(fs.fs_merge_online(wl.B, C, ti, tl, temp, SEED, i, 0, idx, oL), name)

            line(name, wl, f"online merge over {C} chunks of {chunk} ids "
                 "(fs_sample_grouped + fs_merge_online)", timed(online))
        del H, temp, ws

    # the tiny reference configuration (B=4, d=256, V=4096, tiles of 512, W ~
    # N(0, 1/d)): a latency line
    cache.clear()
    torch.cuda.empty_cache()
    Wt = _gpu_weights(torch, 4096, 256, std=(1.0 / 256) ** 0.5)
    Ht = _gpu_hidden(torch, 4, 256)
    pt = fs.params(4, 256, 4096, tile_v=512, seed=SEED)
    it = torch.empty(4, dtype=torch.int32, device="cuda")
    wst = torch.empty(fs.fs_workspace_bytes(pt, fs.FS_VARIANT_FLAT), dtype=torch.uint8,
                      device="cuda")

    def tiny(i):
        pt.step = i
        fs.check(fs.fs_sample(pt, Ht, Wt, None, None, it, None, wst), "tiny")

    wl_t = type("S", (), {"B": 4, "d": 256, "V": 4096})()
    line("tiny_b4", wl_t, "flat fs_sample (latency)", timed(tiny))
    del Wt, Ht, wst

    # one rank's shard of a G-way vocabulary split (the stage-1 kernel alone)
    cache.clear()
    W = W_head
    H = _gpu_hidden(torch, 32, D)
    for G in (2, 4, 8):
        vs = V // G
        start = (G - 1) * vs     # the last shard: its ids are offset by the shard start
        p = fs.params(32, D, vs, v_offset=start, n_valid=start + vs, seed=SEED)
        ws = torch.empty(fs.fs_workspace_bytes(p, fs.FS_VARIANT_FLAT), dtype=torch.uint8,
                         device="cuda")
        Ws = W[start:start + vs]

        def shard(i):
            p.step = i
            fs.check(fs.fs_sample_stage1(p, H, Ws, None, None, ws), "shard")

        t = timed(shard)
        wl = type("S", (), {"B": 32, "d": D, "V": vs})()
        line(f"shard_{G}", wl, f"stage 1 on one of {G} vocabulary shards ({vs} rows)", t)
    cache.clear()
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(torch, H_all, W, B, seconds):
    """The CPU oracle (numpy float64: logits, Philox-Gumbel noise, argmax) on
    the headline batch, timed twice: with every BLAS thread the host offers
    and with one.  Whole calls are repeated (steps 0, 1, ...) until about
    `seconds` of CPU time is spent in each mode; if one call is longer than
    that, a prefix of the vocabulary is timed and scaled to the full call."""
    import numpy as np
    from oracle import fs_oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    Hb = H_all[:B].view(torch.int16).cpu().numpy().view(np.uint16)
    W_host = W.view(torch.int16).cpu().numpy().view(np.uint16)

    def call(Wb, step):
        l = O.logits_bf16(Hb, Wb)
        x = O.tempered(l, None, None, None, 0, 0)
        s = O.scores(x, None, SEED, step, 0, 0)
        return O.sample_flat(s)[0]

    def timed():
        t0 = time.perf_counter()
        call(W_host[:4096], 0)
        est = (time.perf_counter() - t0) * V / 4096          # seconds per full call, estimated
        if est <= seconds:
            n, t0 = 0, time.perf_counter()
            while n == 0 or time.perf_counter() - t0 < seconds:
                call(W_host, n)
                n += 1
            t = time.perf_counter() - t0
            return t / n, (f"{n} full oracle calls (float64 logits + Philox-Gumbel + argmax), "
                           f"B={B}, d={D}, V={V}, steps 0..{n - 1}: {t:.1f} s")
        nv = int(min(V, max(4096, 4096 * seconds / est * V / 4096)) // 16 * 16)
        t0 = time.perf_counter()
        call(W_host[:nv], 0)
        t = time.perf_counter() - t0
        return t * V / nv, (f"one oracle call over the first {nv} of {V} ids (B={B}, d={D}): "
                            f"{t:.1f} s, scaled by {V}/{nv}")

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    per_all, sample_all = timed()
    with threadpool_limits(limits=1):
        per_one, sample_one = timed()
    return {"value": 1.0 / per_all, "unit": "calls/s", "cores": int(threads), "kind": "oracle",
            "sample": sample_all, "seconds_per_call": per_all,
            "single_thread": {"value": 1.0 / per_one, "unit": "calls/s", "cores": 1,
                              "sample": sample_one, "seconds_per_call": per_one},
            "nproc": os.cpu_count(), "cpu_model": cpu_model()}


def hbm_probe(torch, fs, W):
    """Practical HBM ceiling: a streaming read of the W buffer (plain loads, and
    nontemporal loads, whose streaming policy reads faster) and a copy of 1 GiB,
    each timed with HIP events (GB/s of bytes moved)."""
    nbytes = W.numel() * 2
    sink = torch.empty(256 * 256, dtype=torch.int32, device="cuda")
    timer = Timer(torch)
    for i in range(3):
        fs.check(fs.fs_debug_read_probe(W, nbytes, sink, 256), "read probe")
    t_read = timer.run(lambda i: fs.check(fs.fs_debug_read_probe(W, nbytes, sink, 256)), 20)[0]
    for i in range(3):
        fs.check(fs.fs_debug_read_probe_nt(W, nbytes, sink, 256), "read probe (nt)")
    t_read_nt = timer.run(lambda i: fs.check(fs.fs_debug_read_probe_nt(W, nbytes, sink, 256)),
                          20)[0]
    n = 1 << 30
    a = torch.empty(n // 4, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    for i in range(3):
        fs.check(fs.fs_debug_copy(b, a, n, 1024), "copy")
    t_copy = timer.run(lambda i: fs.check(fs.fs_debug_copy(b, a, n, 1024)), 10)[0]
    del a, b
    # L2 -> compute unit rate: every workgroup reads the same 2 MiB (the H of
    # B = 256, d = 4096; it fits one XCD's L2) four times
    l2b, reps = 2 << 20, 4
    l2 = {}
    for grid in (256, 512):
        sink2 = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
        for i in range(3):
            fs.check(fs.fs_debug_shared_read_probe(W, l2b, reps, sink2, grid), "L2 probe")
        t_l2 = timer.run(lambda i: fs.check(
            fs.fs_debug_shared_read_probe(W, l2b, reps, sink2, grid)), 20)[0]
        l2[f"grid{grid}_GBps"] = grid * reps * l2b / t_l2 / 1e9
    return {"read_GBps": nbytes / t_read / 1e9, "read_nt_GBps": nbytes / t_read_nt / 1e9,
            "copy_GBps": 2 * n / t_copy / 1e9,
            "read_grid": 256, "copy_grid": 1024, "copy_bytes": n,
            "l2_shared_read": dict(l2, bytes=l2b, reps=reps,
                                   per_cu_bytes_per_clk_at_2_4GHz=max(l2.values()) * 1e9 / 256 / 2.4e9)}


# The sources the headline stage-1 kernel (resident_kernel) and its launch
# plan are built from.
DIGEST_SOURCES = ("fs_api.hip", "fs_device.h", "fs_epilogue.h", "fs_internal.h", "fs_mfma.h",
                  "fs_plan.cpp", "fs_plan.h",
                  "fs_resident.hip", "fs_topk.h")


def source_digest():
    """sha256 over the headline stage-1 kernel's sources, to tell whether a
    stored counter summary still describes the kernel being timed."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "lm_head_gumbel_amd", "csrc")
    for f in DIGEST_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def stored_traffic(B):
    """HBM bytes per stage-1 launch from the committed counter summary for
    batch B, or None when there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"stage1_d4096_v151936_b{B}_counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != source_digest():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=32, help="headline batch")
    ap.add_argument("--sweep", default="1,2,4,8,16,32,64,128,256",
                    help="comma-separated batches for the sweep ('' to skip)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other configured workloads and the shard shapes")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the fused sampler is a single-GPU kernel "
              f"here (requested --gpus {args.gpus}, WORLD_SIZE={world}); vocab-parallel "
              f"sharding is a design note, not a measured path", file=sys.stderr)
        sys.exit(2)

    import torch
    import lm_head_gumbel_amd as fs
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    fs.lib()
    sweep = [int(b) for b in args.sweep.split(",") if b.strip()]
    bmax = max(sweep + [args.batch])
    log(f"generating inputs d={D} V={V} (W {2 * V * D / 1e9:.2f} GB bf16)")
    H_all, W = make_inputs(torch, bmax)

    # the HBM ceilings first: a measurement of its own, and the device's clocks
    # have settled by the time the headline is timed
    probe = None
    if not args.no_probe:
        probe = hbm_probe(torch, fs, W)
        log(json.dumps(probe))

    log(f"headline B={args.batch}: {args.warmup} warmup + {args.steps} timed calls")
    head = bench_batch(torch, fs, H_all, W, args.batch, args.steps, args.warmup,
                       unfused=True, variants=not args.no_variants)
    log(json.dumps(head))
    rows = []
    for B in sweep:
        if B == args.batch:
            rows.append(head)
            continue
        r = bench_batch(torch, fs, H_all, W, B, max(20, args.steps // 2), max(5, args.warmup // 2))
        log(json.dumps(r))
        rows.append(r)

    workloads = None
    if not args.no_workloads:
        log("other workloads and shard shapes")
        workloads = bench_workloads(torch, fs, args.steps, W)

    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(torch, H_all, W, args.batch, args.cpu_seconds)
        log(json.dumps(cpu))

    t_k1 = head["stage1_us"] * 1e-6
    out = {
        "metric": METRIC,
        "value": head["calls_per_s"],
        "unit": "calls/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["us_per_call"] / 1e3,
        "per_call_us": head["call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"fused LM-head Gumbel sample, d={D} V={V} B={args.batch}",
                   "d": D, "V": V, "B": args.batch, "temperature": 1.0, "seed": SEED,
                   "tokens_per_s": head["tokens_per_s"]},
        "roofline": {"bound": "hbm", "achieved": alg_bytes(args.batch) / t_k1 / 1e9,
                     "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": alg_bytes(args.batch) / t_k1 / PEAK_HBM,
                     "traffic": stored_traffic(args.batch),
                     "kernel": ("fs::resident_kernel" if args.batch <= 32 else "fs::rows_kernel")
                               + " (flat stage 1)",
                     "kernel_us": head["stage1_us"], "kernel_per_launch_us": head["stage1"],
                     "bytes_per_launch": alg_bytes(args.batch),
                     "frac_of_read_probe": (alg_bytes(args.batch) / t_k1 / 1e9 / probe["read_GBps"]
                                            if probe else None),
                     "frac_of_read_probe_nt": (alg_bytes(args.batch) / t_k1 / 1e9
                                               / probe["read_nt_GBps"] if probe else None)},
        "hbm_probe": probe,
        "cpu_baseline": cpu,
        "unfused_calls_per_s": head.get("unfused_calls_per_s"),
        "variants": {k: head[k] for k in ("graph_calls_per_s", "grouped_calls_per_s",
                                          "topk40_calls_per_s", "topk40_topp0.9_calls_per_s")
                     if k in head},
        "sweep": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
                  for r in rows],
        "workloads": ([{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}
                       for r in workloads] if workloads is not None else None),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
