"""Pins for the CPU oracle's sampling definitions (CPU only).

Each check ties the oracle to something outside itself: exact rational
arithmetic, brute force over tiny inputs, the closed forms of the Gumbel law,
the softmax distribution the method must reproduce exactly (chi-square, as
the FlashSampling pages validate their kernel with 5000 samples), partition
invariance of argmax, and the reductions of every variant to the flat or
greedy case.  The last test plants plausible mistakes in a copy of the oracle
and checks that some pin catches each one.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy import special, stats

from oracle import fs_oracle as O
from oracle import philox as px
from lm_head_gumbel_amd.inputs import f32_to_bf16_bits
from stats_util import chi_square_p, softmax

EULER_GAMMA = 0.5772156649015329
N_DRAWS = 5000


# ----------------------------------------------------------------------------
# helpers: many independent draws of one row, one per decode step
# ----------------------------------------------------------------------------
def small_row(V=16, T=0.8, masked=(3, 11), seed=5):
    rng = np.random.default_rng(seed)
    l = rng.normal(0.0, 1.5, size=V)
    x = l / T
    for j in masked:
        x[j] = -np.inf
    return l, x


def scores_over_steps(o, x, seed, steps, b=0, id0=0):
    """s[step, j] = x_j + g(seed, b, id0 + j, step) for many steps at once."""
    V = x.size
    ids = id0 + np.arange(V)
    w = px.noise_words(seed, b, ids[None, :], np.asarray(steps)[:, None], px.STREAM_TOKEN)
    s = x[None, :] + o.gumbel_from_word(w)
    s[:, np.isneginf(x)] = -np.inf
    return s


def flat_draws(o, x, seed=1234, n=N_DRAWS):
    s = scores_over_steps(o, x, seed, np.arange(n))
    return np.array([o.sample_flat(s[i:i + 1])[0][0] for i in range(n)])


# ----------------------------------------------------------------------------
# pin functions (take the oracle module so planted mistakes can be re-checked)
# ----------------------------------------------------------------------------
def check_logits_exact(o):
    """l = H W^T equals the exact rational sum of the bf16 products."""
    rng = np.random.default_rng(3)
    Hb = f32_to_bf16_bits(rng.normal(size=(2, 8)).astype(np.float32))
    Wb = f32_to_bf16_bits(rng.normal(size=(5, 8)).astype(np.float32))
    H, W = o.bf16_bits_to_f64(Hb), o.bf16_bits_to_f64(Wb)
    l = o.logits(H, W)
    assert l.shape == (2, 5)
    for b in range(2):
        for i in range(5):
            exact = sum(Fraction(float(H[b, k])) * Fraction(float(W[i, k])) for k in range(8))
            assert abs(float(l[b, i]) - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))


def check_softmax_exact(o):
    """Flat Gumbel-max draws follow softmax(l/T) over the unmasked ids."""
    l, x = small_row()
    T = 0.8
    xt = o.tempered(l[None, :], np.array([T]), allow=None)[0]
    xt[[3, 11]] = -np.inf
    draws = flat_draws(o, xt)
    assert chi_square_p(draws, softmax(x)) > 0.01


def check_greedy(o):
    """NO_NOISE and T <= 0 rows return the first maximiser of x (brute force)."""
    rng = np.random.default_rng(11)
    l = rng.normal(size=(3, 50))
    l[1, 7] = l[1, 30] = l[1].max() + 1.0       # exact tie: the lower id must win
    temp = np.array([0.9, -1.0, 0.0])
    for flags, tmp in ((O.NO_NOISE, np.array([0.9, 0.9, 0.9])), (0, temp)):
        r = o.run_call(l, tmp, n_valid=45, seed=1, step=2, flags=flags, tile_v=8)
        for b in range(3):
            if flags == 0 and b == 0:
                continue                           # the sampled row
            xb = r["x"][b]
            best, bi = -np.inf, -1
            for i in range(xb.size):
                if xb[i] > best:
                    best, bi = xb[i], i
            assert r["flat_idx"][b] == bi
            assert r["grp_idx"][b] == bi
            assert o.topk_sample(r["x"][b:b + 1], r["s"][b:b + 1], 4)[0][0] == bi
            mn = o.multinomial(r["x"][b:b + 1], tmp[b:b + 1], 1, 2, flags)[0][0]
            assert mn == bi
    assert r["flat_idx"][1] == 7


def check_partition_invariance(o):
    """The max over per-tile winners equals the flat winner for every tiling and
    for random non-contiguous partitions (argmax decomposes over partitions)."""
    rng = np.random.default_rng(21)
    B, V = 3, 1000
    l = rng.normal(size=(B, V)) * 2
    temp = np.array([1.0, 0.6, 1.7])
    x = o.tempered(l, temp, n_valid=990)
    s = o.scores(x, temp, seed=77, step=3)
    flat, _, _ = o.sample_flat(s)
    for tv in (1, 7, 128, 256, 512, V):
        m, idx, L, _ = o.tile_records(x, s, tv)
        for b in range(B):
            t, _ = o.first_argmax(m[b])
            assert idx[b, t] == flat[b]
    for b in range(B):
        perm = rng.permutation(V)
        groups = np.array_split(perm, 37)
        best = (-np.inf, -1)
        for gidx in groups:
            gidx = np.sort(gidx)
            j, mv = o.first_argmax(s[b, gidx])
            cand = (mv, int(gidx[j]))
            if cand[0] > best[0] or (cand[0] == best[0] and cand[1] < best[1]):
                best = cand
        assert best[1] == flat[b]


def check_logmass(o):
    """Tile log-mass equals scipy's logsumexp; a fully masked tile gives -inf."""
    rng = np.random.default_rng(4)
    l = rng.normal(size=(2, 300)) * 3
    x = o.tempered(l, np.array([1.0, 0.5]), n_valid=250)
    s = o.scores(x, np.array([1.0, 0.5]), seed=9, step=0)
    m, idx, L, _ = o.tile_records(x, s, 64)
    for b in range(2):
        for t in range(L.shape[1]):
            seg = x[b, t * 64:(t + 1) * 64]
            ref = special.logsumexp(seg) if np.isfinite(seg).any() else -np.inf
            if np.isfinite(ref):
                assert abs(L[b, t] - ref) < 1e-12 * max(1, abs(ref))
            else:
                assert L[b, t] == -np.inf and idx[b, t] == -1 and m[b, t] == -np.inf
    # tile 3 covers ids 192..255 (ids >= 250 masked); tile 4 covers 256..299: all masked
    assert L[0, 4] == -np.inf


def check_max_stability(o):
    """m_t - L_t is standard Gumbel: mean gamma, variance pi^2/6, Gumbel CDF."""
    rng = np.random.default_rng(8)
    l = rng.normal(size=(1, 96)) * 2
    x = o.tempered(l, np.array([0.7]))
    steps = np.arange(N_DRAWS)
    s = scores_over_steps(o, x[0], 31, steps)
    L = o.tile_records(x, x, 96)[2][0, 0]
    d = s.max(axis=1) - L
    assert abs(d.mean() - EULER_GAMMA) < 4 * (math.pi / math.sqrt(6)) / math.sqrt(d.size)
    assert abs(d.var() - math.pi ** 2 / 6) < 0.15
    assert stats.kstest(d, lambda t: np.exp(-np.exp(-t))).pvalue > 0.01


def check_hierarchical(o):
    """Group-Gumbel-Max: the chosen group follows softmax(L) and the final
    sample follows softmax(x); one group reproduces the flat sample."""
    l, x = small_row(V=16, T=1.3, masked=(0, 9))
    tv = 4
    xg = x[None, :]
    groups, finals = [], []
    for step in range(N_DRAWS):
        s = o.scores(xg, np.array([1.3]), seed=1234, step=step)
        m, idx, L, _ = o.tile_records(xg, s, tv)
        gi, _, gt = o.sample_grouped(idx, L, np.array([1.3]), seed=1234, step=step)
        groups.append(gt[0])
        finals.append(gi[0])
        if step < 50:
            m1, idx1, L1, _ = o.tile_records(xg, s, 16)
            assert o.sample_grouped(idx1, L1, np.array([1.3]), 1234, step)[0][0] == \
                o.sample_flat(s)[0][0]
    Lt = np.array([special.logsumexp(x[t * tv:(t + 1) * tv]) for t in range(4)])
    assert chi_square_p(groups, softmax(Lt)) > 0.01
    assert chi_square_p(finals, softmax(x)) > 0.01


def check_online_merge(o):
    """Binary merge: final log-mass is the total logsumexp, one chunk is the
    flat sample, the chosen chunk follows exp(L_c - A) and the sample
    follows softmax(x)."""
    l, x = small_row(V=16, T=0.9, masked=(4, 5))
    tv, C = 4, 4
    xg = x[None, :]
    finals, chunk_of = [], []
    Lc = None
    for step in range(N_DRAWS):
        s = o.scores(xg, np.array([0.9]), seed=4321, step=step)
        m, idx, L, _ = o.tile_records(xg, s, tv)
        z, A, _ = o.online_merge(idx, L, np.array([0.9]), seed=4321, step=step)
        assert abs(A[0] - special.logsumexp(x)) < 1e-12
        finals.append(z[0])
        chunk_of.append(z[0] // tv)
        Lc = L[0]
        if step < 50:
            m1, idx1, L1, _ = o.tile_records(xg, s, 16)
            assert o.online_merge(idx1, L1, np.array([0.9]), 4321, step)[0][0] == \
                o.sample_flat(s)[0][0]
    A = special.logsumexp(x)
    assert chi_square_p(chunk_of, np.exp(Lc - A)) > 0.01
    assert chi_square_p(finals, softmax(x)) > 0.01


def check_topk(o):
    """Top-k: k = 1 is greedy, k >= #valid is the flat sample, and draws
    follow the renormalised softmax over the k largest x."""
    l, x = small_row(V=16, T=1.0, masked=(2,))
    k = 5
    xg = x[None, :]
    draws = []
    for step in range(N_DRAWS):
        s = o.scores(xg, None, seed=777, step=step)
        draws.append(o.topk_sample(xg, s, k)[0][0])
        if step < 50:
            assert o.topk_sample(xg, s, 1)[0][0] == int(np.argmax(x))
            assert o.topk_sample(xg, s, 15)[0][0] == o.sample_flat(s)[0][0]
    keep = np.argsort(-x, kind="stable")[:k]
    p = np.zeros_like(x)
    p[keep] = softmax(x[keep])
    assert chi_square_p(draws, p) > 0.01


def _topp_golden():
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "topp_worked_example.txt")
    probs, cases = None, []
    with open(path) as fh:
        for line in fh:
            f = line.split()
            if not f or f[0].startswith("#"):
                continue
            if f[0] == "probs":
                probs = np.array([float(v) for v in f[1:]])
            elif f[0] == "case":
                cases.append((int(f[1]), float(f[2]), [int(v) for v in f[3:]]))
    return probs, cases


def check_topk_topp(o):
    """Top-p after top-k: the hand-worked cuts of tests/golden (kept ids are
    exactly the support of the draws, with the renormalised probabilities),
    top_p = 1 is the top-k sample, and a tiny top_p keeps only argmax x."""
    probs, cases = _topp_golden()
    with np.errstate(divide="ignore"):
        x = np.log(probs)[None, :]
    for k, top_p, kept in cases:
        draws = []
        for step in range(1500):
            s = o.scores(x, None, seed=4242, step=step)
            draws.append(o.topk_topp_sample(x, s, k, top_p)[0][0])
        draws = np.array(draws)
        assert set(np.unique(draws)) == set(kept), (k, top_p, kept, np.unique(draws))
        p = np.zeros(probs.size)
        p[kept] = probs[kept] / probs[kept].sum()
        if len(kept) > 1:
            assert chi_square_p(draws, p) > 0.01
    rng = np.random.default_rng(31)
    xr = rng.normal(0.0, 2.0, size=(6, 40))
    xr[0, 5] = -np.inf
    s = o.scores(xr, None, seed=9, step=4)
    for k in (1, 7, 40):
        assert np.array_equal(o.topk_topp_sample(xr, s, k, 1.0)[0], o.topk_sample(xr, s, k)[0])
        assert np.array_equal(o.topk_topp_sample(xr, s, k, 1e-12)[0],
                              np.argmax(np.where(np.isfinite(xr), xr, -np.inf), axis=1))


def check_multinomial(o):
    """Inverse-CDF baseline follows softmax(x); a one-hot distribution returns its id."""
    l, x = small_row(V=16, T=0.7, masked=(1, 2))
    xg = x[None, :]
    draws = [o.multinomial(xg, np.array([0.7]), seed=55, step=st)[0][0] for st in range(N_DRAWS)]
    assert chi_square_p(draws, softmax(x)) > 0.01
    one = np.full((1, 16), -np.inf)
    one[0, 6] = 0.0
    assert o.multinomial(one, np.array([1.0]), seed=1, step=0)[0][0] == 6


def check_scaled_noise_form(o):
    """argmax(l + T g) picks the same id as argmax(l/T + g) for T > 0."""
    rng = np.random.default_rng(12)
    l = rng.normal(size=(4, 500))
    temp = np.array([0.3, 0.7, 1.0, 1.9])
    x = o.tempered(l, temp)
    s = o.scores(x, temp, seed=3, step=8)
    g = s - x
    idx, _, gap = o.sample_flat(s)
    idx2, _, _ = o.sample_flat(l + temp[:, None] * g)
    assert np.array_equal(idx[gap > 1e-9], idx2[gap > 1e-9])


PINS = [check_logits_exact, check_softmax_exact, check_greedy, check_partition_invariance,
        check_logmass, check_max_stability, check_hierarchical, check_online_merge,
        check_topk, check_topk_topp, check_multinomial, check_scaled_noise_form]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(O)


def test_softmax_calibration_across_seeds():
    """Chi-square p-values over many seeds are uniform, and the 1% failure rate
    stays within its binomial band (calibration of the statistic itself)."""
    l, x = small_row(V=8, T=1.0, masked=())
    p = softmax(x)
    pv = []
    for seed in range(120):
        s = scores_over_steps(O, x, seed, np.arange(2000))
        pv.append(chi_square_p(np.argmax(s, axis=1), p))
    pv = np.array(pv)
    assert stats.kstest(pv, "uniform").pvalue > 1e-3
    assert (pv < 0.01).sum() <= stats.binom.ppf(0.999, pv.size, 0.01)


def test_allow_mask_and_id_offset():
    """Masked ids never win; ids and noise follow the global id offset."""
    rng = np.random.default_rng(2)
    l = rng.normal(size=(2, 70)) * 5
    allow = np.full((2, 3), 0xFFFFFFFF, np.uint32)
    allow[0, 0] = 0                      # row 0: ids 0..31 disallowed
    allow[1, 1] = 0x0000FFFF             # row 1: columns 48..63 disallowed
    l[0, 5] = 100.0
    l[1, 50] = 100.0
    r = O.run_call(l, np.array([1.0, 1.0]), allow=allow, seed=5, step=0, tile_v=16, id0=1000)
    assert r["flat_idx"][0] >= 1032 and r["flat_idx"][1] != 1050
    # the same columns scored with id0 = 0 use different noise words
    s0 = O.scores(r["x"], np.array([1.0, 1.0]), seed=5, step=0, id0=0)
    fin = np.isfinite(r["x"])
    assert not np.allclose(s0[fin], r["s"][fin])


# ----------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin
# ----------------------------------------------------------------------------
def _mutant(name):
    """A copy of the oracle module with one plausible mistake planted in it."""
    import types
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__.update(O.__dict__)
    # rebind every oracle function to the copy's globals, so that helpers
    # replaced below are the ones the other functions call
    for fname, f in list(O.__dict__.items()):
        if isinstance(f, types.FunctionType) and f.__module__ == O.__name__:
            setattr(mod, fname, types.FunctionType(f.__code__, mod.__dict__, f.__name__,
                                                   f.__defaults__, f.__closure__))
    if name == "noise_sign":
        mod.gumbel_from_word = lambda r: np.log(-np.log1p(-O.uniform_from_word(r)))
    elif name == "temperature_multiplies":
        def tempered(l, temp=None, *a, **k):
            t = None if temp is None else 1.0 / np.asarray(temp, np.float64)
            return O.tempered(l, t, *a, **k)
        mod.tempered = tempered
    elif name == "tile_offset_off_by_one":
        def tile_records(x, s, tile_v, greedy=None, id0=0):
            return O.tile_records(x, s, tile_v, greedy, id0 + 1)
        mod.tile_records = tile_records
    elif name == "logsumexp_drops_shift":
        def log_sum_exp(a):
            a = np.asarray(a, np.float64)
            if a.size == 0 or np.max(a) == -np.inf:
                return -np.inf
            return float(math.log(np.sum(np.exp(a - np.max(a)))))
        mod.log_sum_exp = log_sum_exp
    elif name == "group_noise_ignored":
        mod.group_noise = lambda seed, step, B, T: np.zeros((B, T))
    elif name == "merge_weights_by_count":
        mod.online_merge = lambda z, L, *a, **k: O.online_merge(
            z, np.where(np.isneginf(L), L, 0.0), *a, **k)
    elif name == "noise_word_shared_by_block":
        def token_noise(seed, step, B, V, id0=0):
            g = O.token_noise(seed, step, B, V + 4, id0)
            return g[:, np.arange(V) & ~3]
        mod.token_noise = token_noise
    elif name == "transposed_operand":
        # W read as if stored [d, V] instead of row-major [V, d]
        mod.logits = lambda H, W: np.asarray(H, np.float64) @ np.asarray(W, np.float64).reshape(
            np.asarray(W).shape[1], np.asarray(W).shape[0])
    elif name == "topp_inclusive_mass":
        def topk_topp_sample(x, s, k, top_p, id0=0):
            # keeps j while the mass up to and including j is below top_p
            x = np.asarray(x, np.float64)
            out = np.full(x.shape[0], -1, np.int64)
            for b in range(x.shape[0]):
                valid = np.nonzero(np.isfinite(x[b]))[0]
                S = valid[np.lexsort((valid, -x[b, valid]))][:k]
                q = np.exp(x[b, S] - x[b, S[0]])
                q /= q.sum()
                kept = S[np.cumsum(q) < top_p]
                kept = kept if kept.size else S[:1]
                out[b] = id0 + int(kept[np.argmax(np.asarray(s)[b, kept])])
            return out, None, None, None
        mod.topk_topp_sample = topk_topp_sample
    elif name == "topp_in_id_order":
        def topk_topp_sample(x, s, k, top_p, id0=0):
            # cuts the top-k set in id order instead of probability order
            x = np.asarray(x, np.float64)
            out = np.full(x.shape[0], -1, np.int64)
            for b in range(x.shape[0]):
                valid = np.nonzero(np.isfinite(x[b]))[0]
                S = np.sort(valid[np.lexsort((valid, -x[b, valid]))][:k])
                q = np.exp(x[b, S] - x[b, S].max())
                q /= q.sum()
                excl = np.concatenate([[0.0], np.cumsum(q)[:-1]])
                kept = S[excl < top_p]
                out[b] = id0 + int(kept[np.argmax(np.asarray(s)[b, kept])])
            return out, None, None, None
        mod.topk_topp_sample = topk_topp_sample
    elif name == "topk_by_noisy_score":
        mod.topk_sample = lambda x, s, k, id0=0: O.topk_sample(s, s, k, id0)
    else:
        raise KeyError(name)
    return mod


# each planted mistake and the pin expected to catch it
MUTANTS = {
    "noise_sign": check_softmax_exact,
    "temperature_multiplies": check_softmax_exact,
    "tile_offset_off_by_one": check_partition_invariance,
    "logsumexp_drops_shift": check_logmass,
    "group_noise_ignored": check_hierarchical,
    "merge_weights_by_count": check_online_merge,
    "noise_word_shared_by_block": check_hierarchical,
    "transposed_operand": check_logits_exact,
    "topk_by_noisy_score": check_topk,
    "topp_inclusive_mass": check_topk_topp,
    "topp_in_id_order": check_topk_topp,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(name)
    with np.errstate(all="ignore"):
        with pytest.raises((AssertionError, ValueError, IndexError)):
            MUTANTS[name](mod)


def test_per_row_seeds_select_each_rows_key():
    """One seed per row: row b's noise in every stream is the noise that the
    single seed seeds[b] gives that row (keys are per row, counters unchanged)."""
    seeds = np.array([7, 2 ** 40 + 3, 7, 0], dtype=np.uint64)
    B, V, T = 4, 37, 6
    rng = np.random.default_rng(4)
    x = rng.normal(size=(B, V))
    g = O.token_noise(seeds, 5, B, V)
    G = O.group_noise(seeds, 5, B, T)
    s_rows = O.scores(x, None, seeds, 5)
    z = rng.integers(0, V, size=(B, T))
    L = rng.normal(size=(B, T))
    zm, Am, _ = O.online_merge(z, L, None, seeds, 5)
    mi, _ = O.multinomial(x, None, seeds, 5)
    for b in range(B):
        sb = int(seeds[b])
        assert np.array_equal(g[b], O.token_noise(sb, 5, B, V)[b])
        assert np.array_equal(G[b], O.group_noise(sb, 5, B, T)[b])
        assert np.array_equal(s_rows[b], O.scores(x, None, sb, 5)[b])
        assert zm[b] == O.online_merge(z, L, None, sb, 5)[0][b]
        assert mi[b] == O.multinomial(x, None, sb, 5)[0][b]
    assert not np.array_equal(g[0], g[1]) and np.array_equal(g[0][:0], g[2][:0])
