"""Pins for the oracle helpers that decide which rows a parity test compares
(CPU only), and for its bf16 conversion.

A GPU result is compared index for index only on rows where the oracle's
answer is robust: the top-two noisy scores differ by more than 1e-2 (the
tolerance the FlashSampling pages' correctness check implies for FP32 noise
and accumulation), the top-k membership and top-p cut are not on a boundary,
the online merge's Bernoulli decisions are not on a boundary, and the
multinomial uniform is not on a CDF boundary.  A mistake in one of these
helpers would silently empty or corrupt those comparisons, so each is pinned
here twice: by values worked out by hand, and by its meaning -- the margin
must equal the distance to the point where the oracle's own decision flips,
found by bisection on the decision alone.  Planted mistakes at the end must
each be caught by a named pin.
"""
import math

import numpy as np
import pytest

from oracle import fs_oracle as O

INF = math.inf


# ----------------------------------------------------------------------------
# bf16 conversion: fixed bit patterns of the bfloat16 format
# ----------------------------------------------------------------------------
BF16_PATTERNS = [
    (0x3F80, 1.0),
    (0xC000, -2.0),
    (0x3F81, 1.0 + 2.0 ** -7),          # one ulp above 1 (7 stored fraction bits)
    (0x4049, 3.140625),                 # 2 * (1 + 73/128)
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),   # largest finite
    (0x0080, 2.0 ** -126),              # smallest normal
    (0x0001, 2.0 ** -133),              # smallest subnormal
    (0x8001, -(2.0 ** -133)),
    (0x7F80, INF),
    (0xFF80, -INF),
    (0x0000, 0.0),
]


def check_bf16_patterns(o):
    bits = np.array([b for b, _ in BF16_PATTERNS], np.uint16)
    got = o.bf16_bits_to_f64(bits)
    for (b, want), g in zip(BF16_PATTERNS, got):
        assert g == want, f"bf16 {b:#06x}: got {g!r} want {want!r}"
    neg0 = o.bf16_bits_to_f64(np.array([0x8000], np.uint16))[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) < 0
    assert np.isnan(o.bf16_bits_to_f64(np.array([0x7FC0], np.uint16))[0])


def check_logits_chunking(o):
    """The chunked bf16 logits equal the unchunked product exactly: small
    integer values make every product and sum exact in float64, so any chunk
    boundary or offset mistake shows as a mismatch (V not a multiple of 8192,
    and odd chunk sizes)."""
    rng = np.random.default_rng(5)
    B, d, V = 3, 24, 2 * 8192 + 37
    # bit patterns of 0, 1, -1, 2, -2, 3 and their integer values
    vals = np.array([0x0000, 0x3F80, 0xBF80, 0x4000, 0xC000, 0x4040], np.uint16)
    ints = np.array([0, 1, -1, 2, -2, 3], np.int64)
    hi = rng.integers(0, vals.size, size=(B, d))
    wi = rng.integers(0, vals.size, size=(V, d))
    Hb, Wb = vals[hi], vals[wi]
    Hi, Wi = ints[hi], ints[wi]
    exact = (Hi @ Wi.T).astype(np.float64)          # integer arithmetic, then exact float
    for chunk in (8192, 7, 1000, V + 5):
        got = o.logits_bf16(Hb, Wb, chunk=chunk)
        assert got.shape == (B, V)
        assert np.array_equal(got, exact), f"chunk {chunk}"


# ----------------------------------------------------------------------------
# top-two gap (flat, tile and group pinning)
# ----------------------------------------------------------------------------
GAP_CASES = [
    ([3.0, 1.0, 2.0], 1.0),
    ([5.0, 5.0, 1.0], 0.0),             # exact tie at the top
    ([-INF, 2.0, -INF, 7.5], 5.5),      # masked entries ignored
    ([10.0, -INF, 9.25, 9.25], 0.75),
    ([-1.0, -3.5], 2.5),
    ([4.0], INF),                       # one finite entry: nothing to confuse it with
    ([-INF, -INF, 1.0], INF),
    ([-INF, -INF], INF),
    ([], INF),
]


def check_top_two_gap(o):
    for a, want in GAP_CASES:
        got = o.top_two_gap(np.array(a, np.float64))
        assert got == want, f"top_two_gap({a}) = {got}, want {want}"
    # meaning: lowering the winner by less than the gap keeps it the argmax,
    # by more than the gap hands the argmax to the runner-up
    rng = np.random.default_rng(7)
    for _ in range(200):
        a = rng.normal(size=rng.integers(2, 30))
        a[rng.random(a.size) < 0.2] = -INF
        g = o.top_two_gap(a)
        fin = np.isfinite(a)
        if fin.sum() < 2:
            assert g == INF
            continue
        w, _ = o.first_argmax(a)
        for frac, same in ((0.999, True), (1.001, False)):
            b = a.copy()
            b[w] -= frac * g
            if g == 0.0:
                continue
            assert (o.first_argmax(b)[0] == w) == same


# ----------------------------------------------------------------------------
# top-k membership margin and top-p cut margin
# ----------------------------------------------------------------------------
def check_topk_margin(o):
    x = np.array([[1.0, 5.0, 3.0, 3.0, -INF, 2.0]])
    s = x + np.array([[0.0, 0.0, 0.5, 0.0, 0.0, 0.0]])
    # order by x descending then id: 1 (5), 2 (3), 3 (3), 5 (2), 0 (1)
    want = {1: (1, INF, 2.0), 2: (1, 1.5, 0.0), 3: (1, 1.5, 1.0), 4: (1, 1.5, 1.0),
            5: (1, 1.5, INF), 6: (1, 1.5, INF)}
    for k, (wi, wg, wm) in want.items():
        idx, gap, margin = o.topk_sample(x, s, k)
        assert (idx[0], gap[0], margin[0]) == (wi, wg, wm), (k, idx, gap, margin)
    # the winner inside the set follows s: raising id 3 above id 1 in s
    s2 = s.copy()
    s2[0, 3] = 6.0
    assert o.topk_sample(x, s2, 3)[0][0] == 3 and o.topk_sample(x, s2, 2)[0][0] == 1
    # meaning: raising the (k+1)-th x by less than the margin leaves the set
    # unchanged, by more than it changes the set
    rng = np.random.default_rng(9)
    for _ in range(100):
        V = int(rng.integers(3, 40))
        xr = np.round(rng.normal(size=(1, V)) * 4, 1)
        k = int(rng.integers(1, V))
        _, _, m = o.topk_sample(xr, xr, k)
        if not (0 < m[0] < INF):
            continue
        order = np.lexsort((np.arange(V), -xr[0]))
        nxt = order[k]
        for frac, same in ((0.999, True), (1.001, False)):
            x2 = xr.copy()
            x2[0, nxt] += frac * m[0]
            S2 = set(np.lexsort((np.arange(V), -x2[0]))[:k])
            assert (S2 == set(order[:k])) == same


def check_topp_cut(o):
    q = np.array([0.5, 0.3, 0.2])
    x = np.log(q)[None, :]
    # exclusive masses in x order: 0, 0.5, 0.8
    want = {0.75: 0.05, 0.4: 0.1, 1.0: 0.2, 0.5: 0.0, 0.85: 0.05, 0.9: 0.1}
    for top_p, wc in want.items():
        _, _, _, cut = o.topk_topp_sample(x, x, 3, top_p)
        assert abs(cut[0] - wc) < 1e-12, (top_p, cut[0], wc)
    # meaning: moving top_p by less than the cut keeps the kept set, crossing
    # it changes the set
    rng = np.random.default_rng(13)
    for _ in range(100):
        V = int(rng.integers(2, 25))
        xr = rng.normal(size=(1, V)) * 2
        k = int(rng.integers(1, V + 1))
        top_p = float(rng.uniform(0.05, 0.999))

        def kept(tp):
            # the kept prefix's size from the sample of a score vector that
            # favours later (less likely) ids: the draw is the last kept id
            order = np.lexsort((np.arange(V), -xr[0]))
            s = np.full((1, V), -INF)
            s[0, order[:k]] = np.arange(k, dtype=np.float64)
            return int(np.nonzero(order == o.topk_topp_sample(xr, s, k, tp)[0][0])[0][0]) + 1

        _, _, _, cut = o.topk_topp_sample(xr, xr, k, top_p)
        c = cut[0]
        if not (1e-9 < c < INF):
            continue
        n0 = kept(top_p)
        for tp in (top_p - 0.999 * c, top_p + 0.999 * c):
            if 0 < tp <= 1:
                assert kept(tp) == n0
        flips = [tp for tp in (top_p - 1.001 * c, top_p + 1.001 * c) if 0 < tp <= 1]
        assert any(kept(tp) != n0 for tp in flips) or not flips


# ----------------------------------------------------------------------------
# online-merge decision margin and multinomial CDF margin
# ----------------------------------------------------------------------------
def _boundary(decide, lo, hi, iters=200):
    """Bisection for the flip point of a monotone boolean decision on [lo, hi]."""
    d_lo = decide(lo)
    assert decide(hi) != d_lo
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if decide(mid) == d_lo:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def check_merge_margin(o):
    # one chunk: no decision at all
    _, _, m = o.online_merge(np.array([[4]]), np.array([[0.3]]), None, 1, 0)
    assert m[0] == INF
    # a masked chunk takes no decision either
    _, _, m = o.online_merge(np.array([[4, 9]]), np.array([[0.3, -INF]]), None, 1, 0)
    assert m[0] == INF
    # greedy rows: margin 0 exactly on a tie of the log-masses, else none
    g = o.online_merge(np.array([[4, 9]]), np.array([[0.3, 0.3]]), np.array([0.0]), 1, 0)
    assert (g[0][0], g[2][0]) == (4, 0.0)
    g = o.online_merge(np.array([[4, 9]]), np.array([[0.3, 0.7]]), np.array([0.0]), 1, 0)
    assert (g[0][0], g[2][0]) == (9, INF)
    # meaning (two chunks, one decision): the chunk-1 probability is
    # p(t) = sigmoid(t), t = L_1 - L_0; the oracle replaces the sample when its
    # uniform u is below p.  The flip point t* of that decision, found by
    # bisection on the returned index alone, gives u = sigmoid(t*), and the
    # margin must be |log u - log p(t)|.
    for seed, step in ((1, 0), (1234, 7), (99, 3)):
        def decide(t):
            return o.online_merge(np.array([[0, 1]]), np.array([[0.0, t]]), None, seed, step)[0][0]
        ts = _boundary(decide, -40.0, 40.0)
        log_u = -math.log1p(math.exp(-ts)) if ts > -30 else ts
        for t in (ts - 2.0, ts - 0.1, ts + 0.05, ts + 1.5):
            _, _, m = o.online_merge(np.array([[0, 1]]), np.array([[0.0, t]]), None, seed, step)
            log_p = -math.log1p(math.exp(-t))
            assert abs(m[0] - abs(log_u - log_p)) < 1e-9, (seed, step, t, m[0])
    # several chunks: the margin is the smallest over the decisions
    L = np.array([[0.0, 0.1, -0.3, 0.2]])
    z = np.array([[10, 11, 12, 13]])
    _, _, m4 = o.online_merge(z, L, None, 5, 2)
    prefix = [o.online_merge(z[:, :c], L[:, :c], None, 5, 2)[2][0] for c in range(2, 5)]
    assert m4[0] == min(prefix) and prefix == sorted(prefix, reverse=True)


def check_multinomial_margin(o):
    # two ids with masses a and 1 - a: id 0 is drawn exactly when u < a.  The
    # flip point a* (bisection on the drawn id) is the uniform u itself, and
    # the margin must be min(u, a - u) below a and min(u - a, 1 - u) above.
    for seed, step in ((55, 0), (1, 9), (777, 4)):
        def decide(a):
            x = np.log(np.array([[a, 1.0 - a]]))
            return o.multinomial(x, np.array([1.0]), seed, step)[0][0]
        u = _boundary(decide, 1e-12, 1.0 - 1e-12)
        for a in (u * 0.5, u - 1e-3, min(u + 1e-3, 1 - 1e-9), u + 0.5 * (1 - u)):
            x = np.log(np.array([[a, 1.0 - a]]))
            j, m = o.multinomial(x, np.array([1.0]), seed, step)
            want = min(u, a - u) if j[0] == 0 else min(u - a, 1.0 - u)
            assert (j[0] == 0) == (u < a)
            assert abs(m[0] - want) < 1e-9, (seed, step, a, m[0], want)
    # greedy rows carry no margin
    _, m = o.multinomial(np.array([[0.0, 1.0]]), np.array([0.0]), 1, 0)
    assert m[0] == INF


def check_topk_pick_margin(o):
    tol = 1e-3
    x = np.array([[1.0, 5.0, 3.0, 3.0, -INF, 2.0]])
    s = x + np.array([[0.0, 0.0, 0.5, 0.0, 0.0, 0.0]])
    # k = 2: ids 2 and 3 tie for the second place, but the pick (id 1) is
    # certainly in every admissible set and beats both by 1.5 in s
    for k, want in ((1, INF), (2, 1.5), (3, 1.5), (5, 1.5)):
        assert o.topk_pick_margin(x, s, k, tol)[0] == want, k
    # id 1 sits 5e-4 below the second place: a set with it is admissible and
    # then it wins on s, so the pick is not robust
    x = np.array([[4.0, 3.0, 3.0005, 1.0]])
    assert o.topk_pick_margin(x, x + np.array([[0.0, 2.0, 0.0, 0.0]]), 2, tol)[0] == 0.0
    # with that id far behind in s the pick (id 0) holds: gap over {0, 1, 2}
    assert abs(o.topk_pick_margin(x, x, 2, tol)[0] - 0.9995) < 1e-12
    assert o.topk_pick_margin(np.full((1, 3), -INF), np.full((1, 3), -INF), 2, tol)[0] == INF
    # meaning: where the margin exceeds tol_s, no perturbation of x by tol/2
    # per id (s moving with it) and of s by tol_s/2 changes the sample
    rng = np.random.default_rng(17)
    tol_s, checked = 1e-2, 0
    for _ in range(300):
        V = int(rng.integers(3, 30))
        xr = np.round(rng.normal(size=(1, V)) * 2, 3)          # near-ties on purpose
        g = rng.gumbel(size=(1, V))
        k = int(rng.integers(1, V))
        m = o.topk_pick_margin(xr, xr + g, k, tol)[0]
        base = o.topk_sample(xr, xr + g, k)[0][0]
        if not m > tol_s:
            continue
        checked += 1
        for _ in range(40):
            dx = rng.choice([-0.5, 0.5], size=(1, V)) * tol * rng.uniform(0.0, 1.0, size=(1, V))
            ds = rng.uniform(-0.5, 0.5, size=(1, V)) * tol_s
            assert o.topk_sample(xr + dx, xr + dx + g + ds, k)[0][0] == base
    assert checked > 100


def check_topp_pick_margin(o):
    tol, tm = 1e-3, 1e-4
    q = np.array([0.5, 0.3, 0.2])
    x = np.log(q)[None, :]
    # kept {0, 1} (exclusive masses 0, 0.5; the next one 0.8): robust, gap of s
    assert abs(o.topp_pick_margin(x, x, 3, 0.75, tol, tm)[0] - math.log(5 / 3)) < 1e-12
    # id 2's exclusive mass 0.8 can shrink to 0.8 (1 - rho) / (1 + rho) ~ 0.7992:
    # with top_p = 0.79 it stays out, with 0.7995 it may be kept -- which
    # matters only when it would win on s
    s2 = x + np.array([[0.0, 0.0, 2.0]])
    assert abs(o.topp_pick_margin(x, s2, 3, 0.79, tol, tm)[0] - math.log(5 / 3)) < 1e-12
    assert o.topp_pick_margin(x, s2, 3, 0.7995, tol, tm)[0] == 0.0
    assert abs(o.topp_pick_margin(x, x, 3, 0.7995, tol, tm)[0] - math.log(5 / 3)) < 1e-12
    # two ids 5e-4 apart in x straddle the cut: either may be the kept one
    x3 = np.log(np.array([[0.6, 0.2, 0.2 * math.exp(-5e-4), 0.0001]]))
    s3 = x3 + np.array([[0.0, 0.0, 3.0, 0.0]])
    assert o.topp_pick_margin(x3, s3, 4, 0.7, tol, tm)[0] == 0.0
    assert o.topp_pick_margin(x3, x3, 4, 0.7, tol, tm)[0] > 0.5
    # everything kept: the top-k question (one id in the set: inf)
    assert o.topp_pick_margin(x, x, 1, 1.0, tol, tm)[0] == INF
    assert abs(o.topp_pick_margin(x, x, 3, 1.0, tol, tm)[0] - math.log(5 / 3)) < 1e-12
    # meaning: where the margin exceeds tol_s, perturbations of x by tol/2
    # per id and of s by tol_s/2 never change the sample
    rng = np.random.default_rng(23)
    tol_s, checked = 1e-2, 0
    for _ in range(300):
        V = int(rng.integers(3, 30))
        xr = np.round(rng.normal(size=(1, V)) * 1.5, 3)
        g = rng.gumbel(size=(1, V))
        k = int(rng.integers(1, V + 1))
        top_p = float(rng.uniform(0.2, 1.0))
        m = o.topp_pick_margin(xr, xr + g, k, top_p, tol, 0.0)[0]
        if not m > tol_s:
            continue
        checked += 1
        base = o.topk_topp_sample(xr, xr + g, k, top_p)[0][0]
        for _ in range(40):
            dx = rng.choice([-0.5, 0.5], size=(1, V)) * tol * rng.uniform(0.0, 1.0, size=(1, V))
            ds = rng.uniform(-0.5, 0.5, size=(1, V)) * tol_s
            assert o.topk_topp_sample(xr + dx, xr + dx + g + ds, k, top_p)[0][0] == base
    assert checked > 100


PINS = [check_bf16_patterns, check_logits_chunking, check_top_two_gap, check_topk_margin,
        check_topp_cut, check_merge_margin, check_multinomial_margin, check_topk_pick_margin,
        check_topp_pick_margin]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_selection_pin(pin):
    pin(O)


# ----------------------------------------------------------------------------
# planted mistakes in the selection helpers: each caught by its named pin
# ----------------------------------------------------------------------------
# (function, line as the oracle writes it, the mistake planted in its place)
SOURCE_MUTANTS = {
    "gap_always_zero": ("top_two_gap", "return float(top[1] - top[0])", "return 0.0"),
    "gap_max_minus_min": ("top_two_gap", "return float(top[1] - top[0])",
                          "return float(f.max() - f.min())"),
    "topk_margin_wrong_sign": ("topk_sample",
                               "margin[b] = float(x[b, order[k - 1]] - x[b, order[k]])",
                               "margin[b] = float(x[b, order[k]] - x[b, order[k - 1]])"),
    "topp_cut_inside_only": ("topk_topp_sample", "cut[b] = min(d_in, d_out)", "cut[b] = d_in"),
    "merge_margin_signed": ("online_merge", "abs(math.log(u) - math.log(p))",
                            "(math.log(u) - math.log(p))"),
    "merge_margin_linear": ("online_merge", "abs(math.log(u) - math.log(p))", "abs(u - p)"),
    "multinomial_margin_upper_only": ("multinomial", "margin[b] = min(u - lo, cdf[j] - u)",
                                      "margin[b] = cdf[j] - u"),
    "bf16_drops_sign": ("bf16_bits_to_f64", "np.asarray(bits, dtype=np.uint16).astype(np.uint32)",
                        "(np.asarray(bits, dtype=np.uint16).astype(np.uint32) & np.uint32(0x7FFF))"),
    "logits_chunk_offset": ("logits_bf16", "bf16_bits_to_f64(W_bits[i0:i1])",
                            "bf16_bits_to_f64(W_bits[max(0, i0 - 1):i1 - min(i0, 1)])"),
    "pick_ignores_zone": ("topk_pick_margin",
                          "top_two_gap(s[b, s_plus]) if w in set(s_minus.tolist()) else 0.0",
                          "top_two_gap(s[b, s_plus])"),
    "bounds_minus_too_wide": ("_topk_bounds", "xb[valid] > xk1 + tol_x", "xb[valid] > xk - tol_x"),
    "topp_pick_possible_is_certain": ("topp_pick_margin",
                                      "possible = p_min / z_hi < top_p + tol_mass",
                                      "possible = certain"),
}


def _mutant(name):
    """A copy of the oracle module with one mistake planted in the source of
    one function (the edited line must exist, so no mutant is a no-op)."""
    import inspect
    import textwrap
    import types
    mod = types.ModuleType("oracle_selection_mutant")
    mod.__dict__.update(O.__dict__)
    for fname, f in list(O.__dict__.items()):
        if isinstance(f, types.FunctionType) and f.__module__ == O.__name__:
            setattr(mod, fname, types.FunctionType(f.__code__, mod.__dict__, f.__name__,
                                                   f.__defaults__, f.__closure__))
    if name == "bf16_as_fp16":
        mod.bf16_bits_to_f64 = lambda bits: np.asarray(bits, np.uint16).view(np.float16).astype(
            np.float64)
        return mod
    fname, line, planted = SOURCE_MUTANTS[name]
    src = textwrap.dedent(inspect.getsource(getattr(O, fname)))
    assert src.count(line) == 1, f"{fname} no longer holds the line to mutate"
    exec(compile(src.replace(line, planted), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


MUTANTS = {
    "gap_always_zero": check_top_two_gap,
    "gap_max_minus_min": check_top_two_gap,
    "topk_margin_wrong_sign": check_topk_margin,
    "topp_cut_inside_only": check_topp_cut,
    "merge_margin_signed": check_merge_margin,
    "merge_margin_linear": check_merge_margin,
    "multinomial_margin_upper_only": check_multinomial_margin,
    "bf16_drops_sign": check_bf16_patterns,
    "bf16_as_fp16": check_bf16_patterns,
    "logits_chunk_offset": check_logits_chunking,
    "pick_ignores_zone": check_topk_pick_margin,
    "bounds_minus_too_wide": check_topk_pick_margin,
    "topp_pick_possible_is_certain": check_topp_pick_margin,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_selection_mistake_is_caught(name):
    mod = _mutant(name)
    with np.errstate(all="ignore"):
        with pytest.raises((AssertionError, ValueError, IndexError)):
            MUTANTS[name](mod)
