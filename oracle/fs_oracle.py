"""Plain, slow, obviously-correct CPU oracle for fused LM-head Gumbel sampling.

TEST INFRASTRUCTURE.  Only `tests/`, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` may import or call anything under `oracle/`.
The product library never imports it, and the two share no code: this file
writes every step out in numpy float64 from the definitions on the pages.

Pages cited (by title and the passage used):
  [FS-abs]   "FlashSampling: Fast and Memory-Efficient Exact Sampling"
             (tomesphere.com/paper/2603.15854), Abstract.
  [FS-kr]    "FlashSampling: 빠르고 메모리 효율적인 정확한 샘플링 기법"
             (aitrends.kr/articles/26667); paragraphs named by subject:
             "Gumbel-Max", "Stage 1", "Stage 2", "tensor parallel",
             "max-stability", "Group-Gumbel-Max", "implementation", "top-p".
  [CAKE]     "flashinfer.cake_sampling" (docs.flashinfer.ai), sections
             "Correctness contract" and "Launch forms".
  [GMX]      "On-Chip LLM: Sampling Without Asking" (mikeayles.com), the
             Gumbel-max identity paragraph.
  [PHILOX]   Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3",
             SC'11, section 3 (see oracle/philox.py).

What is computed (all in float64; every helper is a direct definition):
  logits        l[b,i] = sum_k H[b,k] W[i,k]                       [FS-kr Stage 1]
  temper/mask   x = l / T_b, or -inf where id >= n_valid or the
                row's allow bit is clear                          [FS-kr Stage 1]
  noise         r = Philox-4x32-10 word for (id, row, step, stream 0)
                v = (r + 1/2) 2^-32, u = 1 - v, g = -log(-log u)  [FS-kr Stage 1]
  score         s = x + g                                          [FS-kr Stage 1]
  tile records  m_t = max s, idx_t = lowest id attaining it,
                L_t = log sum exp x over the tile                  [FS-kr Stage 1, tensor parallel]
  flat sample   i* = argmax_i s (lowest id on ties)                [FS-kr Stage 2; FS-abs]
  hierarchical  t* = argmax_t (L_t + G_t), G from stream 1; i = idx_t*
                                                                   [FS-kr Group-Gumbel-Max; FS-abs]
  online merge  Bernoulli binary merge of (z_c, L_c) chunk summaries,
                uniforms from stream 2                             [FS-kr Group-Gumbel-Max]
  top-k         k largest x (lowest id on ties), then argmax s     [FS-kr implementation; GMX]
  top-p after   sort the top-k set, keep the shortest prefix whose
  top-k         exclusive softmax mass is below top_p times the
                set's mass, then argmax s over the kept prefix     [FS-kr top-p; CAKE]
  multinomial   inverse CDF of softmax(x) at a stream-3 uniform    [FS-kr problem statement]

Besides the results, the oracle reports how far each result is from changing
(top-two gaps, membership, cut and decision margins, and the robustness of
top-k and top-p picks to small logit errors): the parity tests compare an
index only where that distance exceeds the stated tolerance.

Every function taking `seed` also accepts one seed per batch row (a
length-B sequence): row b then draws all its noise under key seed[b].

Readings taken where the pages leave a step open (each is listed in the design doc):
  * Temperature divides the logit before the noise is added (x/T + g) as the
    Stage 1 paragraph orders it; the x + T*g form of [GMX] picks the same id.
  * The log-mass covers the tempered, masked logits x.
  * A row with T_b <= 0 (or NaN), or any row under the NO_NOISE flag, is
    greedy: no noise, and its log-mass is the tile maximum of x (the
    zero-temperature limit), so every variant returns argmax x.
  * Ties go to the lowest id everywhere [CAKE Correctness contract].
  * A NaN logit counts as masked; a tile or row with nothing valid gives
    m = L = -inf and index -1.
  * Top-p after top-k works on softmax(x) restricted to the top-k set (x is
    already tempered), orders the set by x descending with ties to the lower
    id, and keeps element j when the mass of the elements before it is below
    top_p times the set's mass [CAKE launch forms]; the draw is the Gumbel
    argmax over the kept elements, the same noise as every other variant.
"""
import math

import numpy as np

from . import philox as px

NO_NOISE = 1          # flag bit: seed-less operation, every row greedy [GMX]


def row_seed(seed, b):
    """The Philox seed of batch row b: `seed` itself, or seed[b] when one seed
    per row is given (per-request seeds, as a serving engine would pass)."""
    if np.ndim(seed) == 0:
        return int(seed)
    return int(np.asarray(seed, dtype=np.uint64)[b])
NEG_INF = -np.inf
TWO_M32 = 2.0 ** -32


# ----------------------------------------------------------------------------
# data conversion (exact)
# ----------------------------------------------------------------------------
def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# logits and the per-element definitions
# ----------------------------------------------------------------------------
def logits(H, W):
    """l = H W^T for float64 H [B,d], W [V,d]  ([FS-kr] Stage 1: the logits
    tile is the product of the hidden states with the weight sub-matrix).
    Each bf16 product is exact in float64; the sum rounds in float64."""
    return np.asarray(H, np.float64) @ np.asarray(W, np.float64).T


def logits_bf16(H_bits, W_bits, chunk=8192):
    """l for bf16 bit-pattern inputs, converting W to float64 one id-chunk at a
    time so the full-size weight matrix never exists in float64 at once."""
    Hd = bf16_bits_to_f64(H_bits)
    V = W_bits.shape[0]
    out = np.empty((Hd.shape[0], V), np.float64)
    for i0 in range(0, V, chunk):
        i1 = min(V, i0 + chunk)
        out[:, i0:i1] = logits(Hd, bf16_bits_to_f64(W_bits[i0:i1]))
    return out


def greedy_rows(temp, B, flags=0):
    """Boolean [B]: rows sampled greedily (T_b <= 0, NaN, or NO_NOISE)."""
    if flags & NO_NOISE:
        return np.ones(B, bool)
    if temp is None:
        return np.zeros(B, bool)
    t = np.asarray(temp, np.float64)
    return ~(t > 0)


def tempered(l, temp=None, n_valid=None, allow=None, flags=0, id0=0):
    """x = l / T_b (or l for greedy rows), -inf where masked.

    ids are global: column j of `l` is id id0 + j.  An id is masked when
    id >= n_valid or when bit j of the row's `allow` words is clear
    (allow is uint32 [B, ceil(V/32)], indexed by column).  NaN -> -inf.
    """
    l = np.asarray(l, np.float64)
    B, V = l.shape
    greedy = greedy_rows(temp, B, flags)
    T = np.ones(B) if temp is None else np.asarray(temp, np.float64).copy()
    T[greedy] = 1.0
    x = l / T[:, None]
    if n_valid is not None:
        ids = id0 + np.arange(V)
        x[:, ids >= n_valid] = NEG_INF
    if allow is not None:
        cols = np.arange(V)
        bits = (np.asarray(allow, np.uint32)[:, cols >> 5] >> (cols & 31).astype(np.uint32)) & 1
        x[bits == 0] = NEG_INF
    x[np.isnan(x)] = NEG_INF
    return x


def uniform_from_word(r):
    """v = (r + 1/2) 2^-32: a uniform on the open interval (0, 1), exact in float64."""
    return (np.asarray(r, np.float64) + 0.5) * TWO_M32


def gumbel_from_word(r):
    """Standard Gumbel variate from one 32-bit word ([FS-kr] Stage 1: g = -log(-log u)).

    u = 1 - v; -log u is evaluated as -log1p(-v) so that the region u -> 1,
    where the largest g (the likely winners) live, keeps full precision.
    """
    v = uniform_from_word(r)
    return -np.log(-np.log1p(-v))


def token_noise(seed, step, B, V, id0=0):
    """g[b, j] for ids id0 + j from stream 0."""
    ids = id0 + np.arange(V, dtype=np.int64)
    g = np.empty((B, V), np.float64)
    for b in range(B):
        g[b] = gumbel_from_word(px.noise_words(row_seed(seed, b), b, ids, step, px.STREAM_TOKEN))
    return g


def scores(x, temp=None, seed=0, step=0, flags=0, id0=0):
    """s = x + g; greedy rows take g = 0; masked ids stay -inf."""
    x = np.asarray(x, np.float64)
    B, V = x.shape
    greedy = greedy_rows(temp, B, flags)
    s = x.copy()
    if not greedy.all():
        g = token_noise(seed, step, B, V, id0)
        s[~greedy] += g[~greedy]
    s[np.isneginf(x)] = NEG_INF
    return s


# ----------------------------------------------------------------------------
# reductions
# ----------------------------------------------------------------------------
def first_argmax(a):
    """(index, value) of the maximum of a 1-D array, lowest index on ties;
    (-1, -inf) when every entry is -inf or the array is empty."""
    a = np.asarray(a, np.float64)
    if a.size == 0:
        return -1, NEG_INF
    j = int(np.argmax(a))   # numpy returns the first occurrence of the maximum
    if a[j] == NEG_INF:
        return -1, NEG_INF
    return j, float(a[j])


def top_two_gap(a):
    """Difference between the largest and second-largest entries (inf if < 2 finite)."""
    a = np.asarray(a, np.float64)
    f = a[np.isfinite(a)]
    if f.size < 2:
        return math.inf
    top = np.partition(f, f.size - 2)[-2:]
    return float(top[1] - top[0])


def log_sum_exp(a):
    """log sum exp, shifted by the maximum; -inf when nothing is finite."""
    a = np.asarray(a, np.float64)
    if a.size == 0:
        return NEG_INF
    mx = np.max(a)
    if mx == NEG_INF:
        return NEG_INF
    return float(mx + math.log(np.sum(np.exp(a - mx))))


def tile_records(x, s, tile_v, greedy=None, id0=0):
    """Per-(row, tile) winner records ([FS-kr] Stage 1 outputs m and idx;
    the tensor-parallel paragraph adds the log-mass L).

    Tile t covers columns [t*tile_v, min((t+1)*tile_v, V)).  Returns
    m, idx (global ids), L, gap, each [B, T].  Greedy rows take L = max x.
    """
    x = np.asarray(x, np.float64)
    s = np.asarray(s, np.float64)
    B, V = x.shape
    T = -(-V // tile_v)
    if greedy is None:
        greedy = np.zeros(B, bool)
    m = np.full((B, T), NEG_INF)
    idx = np.full((B, T), -1, np.int64)
    L = np.full((B, T), NEG_INF)
    gap = np.full((B, T), math.inf)
    for b in range(B):
        for t in range(T):
            c0, c1 = t * tile_v, min(V, (t + 1) * tile_v)
            j, mv = first_argmax(s[b, c0:c1])
            m[b, t] = mv
            idx[b, t] = -1 if j < 0 else id0 + c0 + j
            L[b, t] = float(np.max(x[b, c0:c1])) if greedy[b] else log_sum_exp(x[b, c0:c1])
            gap[b, t] = top_two_gap(s[b, c0:c1])
    return m, idx, L, gap


def sample_flat(s, id0=0):
    """Flat sample per row: i* = argmax_i s ([FS-kr] Stage 2: argmax over the
    tile maxima, which equals the argmax over all ids [FS-abs]).
    Returns (idx [B] global ids or -1, max score [B], top-two gap [B])."""
    s = np.asarray(s, np.float64)
    B = s.shape[0]
    out = np.full(B, -1, np.int64)
    mx = np.full(B, NEG_INF)
    gap = np.full(B, math.inf)
    for b in range(B):
        j, v = first_argmax(s[b])
        out[b] = -1 if j < 0 else id0 + j
        mx[b] = v
        gap[b] = top_two_gap(s[b])
    return out, mx, gap


def group_noise(seed, step, B, T):
    """G[b, t]: standard Gumbel per group from stream 1 (group index t)."""
    G = np.empty((B, T), np.float64)
    ts = np.arange(T, dtype=np.int64)
    for b in range(B):
        G[b] = gumbel_from_word(px.noise_words(row_seed(seed, b), b, ts, step, px.STREAM_GROUP))
    return G


def sample_grouped(idx, L, temp=None, seed=0, step=0, flags=0):
    """Hierarchical (Group-Gumbel-Max) sample from tile records
    ([FS-kr] tensor-parallel and Group-Gumbel-Max paragraphs; [FS-abs]):
    pick group t with probability softmax(L)_t via argmax_t (L_t + G_t),
    then return that group's own local sample idx_t.
    Greedy rows use G = 0 (their L is the tile maximum).
    Returns (idx [B], gap of the group scores [B], chosen group [B])."""
    idx = np.asarray(idx)
    L = np.asarray(L, np.float64)
    B, T = L.shape
    greedy = greedy_rows(temp, B, flags)
    G = group_noise(seed, step, B, T)
    out = np.full(B, -1, np.int64)
    gap = np.full(B, math.inf)
    chosen = np.full(B, -1, np.int64)
    for b in range(B):
        sc = L[b].copy() if greedy[b] else L[b] + G[b]
        sc[np.isneginf(L[b])] = NEG_INF
        t, _ = first_argmax(sc)
        chosen[b] = t
        out[b] = -1 if t < 0 else int(idx[b, t])
        gap[b] = top_two_gap(sc)
    return out, gap, chosen


def online_merge(z, L, temp=None, seed=0, step=0, flags=0):
    """Online binary merge of chunk summaries ([FS-kr] Group-Gumbel-Max
    paragraph: as each group arrives a Bernoulli choice decides whether it
    replaces the running sample, with O(1) state).

    State (z, A) starts at chunk 0.  For chunk c >= 1: A' = logaddexp(A, L_c),
    p = exp(L_c - A') (0 when L_c = -inf), u_c = (r + 1/2) 2^-32 with r the
    stream-2 word of group index c; replace z by z_c when u_c < p; A = A'.
    Greedy rows replace when L_c > A and keep A = max.
    Returns (z [B], A [B], min decision margin |log u - log p| [B])."""
    z = np.asarray(z)
    L = np.asarray(L, np.float64)
    B, C = L.shape
    greedy = greedy_rows(temp, B, flags)
    out = np.array(z[:, 0], np.int64)
    A = np.array(L[:, 0], np.float64)
    margin = np.full(B, math.inf)
    cs = np.arange(C, dtype=np.int64)
    for b in range(B):
        u_all = uniform_from_word(px.noise_words(row_seed(seed, b), b, cs, step, px.STREAM_MERGE))
        for c in range(1, C):
            Lc = L[b, c]
            if greedy[b]:
                if Lc > A[b]:
                    out[b], A[b] = z[b, c], Lc
                elif Lc == A[b] and Lc > NEG_INF:
                    margin[b] = 0.0
                continue
            if Lc == NEG_INF:
                continue
            A_new = float(np.logaddexp(A[b], Lc))
            p = math.exp(Lc - A_new)
            u = float(u_all[c])
            margin[b] = min(margin[b], abs(math.log(u) - math.log(p)))
            if u < p:
                out[b] = z[b, c]
            A[b] = A_new
    return out, A, margin


def topk_sample(x, s, k, id0=0):
    """Top-k restricted sample ([FS-kr] implementation paragraph: the tile
    scheme extends to top-k; [GMX]: only the k most likely tokens may be
    drawn).  S = the k valid ids with the largest x (lowest id on ties; all
    valid ids when fewer than k), then i = argmax over S of s.
    Returns (idx [B], s-gap within S [B], membership margin x(k)-x(k+1) [B])."""
    x = np.asarray(x, np.float64)
    s = np.asarray(s, np.float64)
    B, V = x.shape
    out = np.full(B, -1, np.int64)
    gap = np.full(B, math.inf)
    margin = np.full(B, math.inf)
    for b in range(B):
        valid = np.nonzero(np.isfinite(x[b]))[0]
        if valid.size == 0:
            continue
        order = valid[np.lexsort((valid, -x[b, valid]))]   # by x descending, then id
        S = order[:k]
        if order.size > k:
            margin[b] = float(x[b, order[k - 1]] - x[b, order[k]])
        j, _ = first_argmax(s[b, S])
        out[b] = id0 + int(S[j])
        gap[b] = top_two_gap(s[b, S])
    return out, gap, margin


def topk_topp_sample(x, s, k, top_p, id0=0):
    """Top-p after top-k ([FS-kr] top-p paragraph: top-k first, then top-p
    on the few candidates; [CAKE] launch forms: keep the shortest prefix
    whose exclusive mass is below top_p times the top-k mass).

    Per row: S = the k valid ids with the largest x (lowest id on ties),
    ordered by x descending and then id; q = softmax of x over S; element j
    of that order is kept when sum_{i<j} q_i < top_p (the q sum to 1 over S);
    the sample is argmax over the kept ids of s (lowest id on ties).

    Returns (idx [B], s-gap within the kept set [B], top-k membership margin
    x(k) - x(k+1) [B], cut margin [B]: the distance of the exclusive masses
    on both sides of the cut from top_p)."""
    x = np.asarray(x, np.float64)
    s = np.asarray(s, np.float64)
    B, V = x.shape
    out = np.full(B, -1, np.int64)
    gap = np.full(B, math.inf)
    margin = np.full(B, math.inf)
    cut = np.full(B, math.inf)
    for b in range(B):
        valid = np.nonzero(np.isfinite(x[b]))[0]
        if valid.size == 0:
            continue
        order = valid[np.lexsort((valid, -x[b, valid]))]   # by x descending, then id
        S = order[:k]
        if order.size > k:
            margin[b] = float(x[b, order[k - 1]] - x[b, order[k]])
        w = np.exp(x[b, S] - x[b, S[0]])
        q = w / w.sum()
        excl = np.concatenate([[0.0], np.cumsum(q)[:-1]])
        keep = excl < top_p
        kept = S[keep]
        # the kept ones are a prefix: the first dropped element (if any) and
        # the last kept one bound the cut; the first element has no mass
        # before it and is kept for every top_p > 0, so it bounds nothing
        nk = kept.size
        d_in = abs(top_p - excl[nk - 1]) if nk > 1 else math.inf
        d_out = abs(excl[nk] - top_p) if nk < S.size else math.inf
        cut[b] = min(d_in, d_out)
        j, _ = first_argmax(s[b, kept])
        out[b] = id0 + int(kept[j])
        gap[b] = top_two_gap(s[b, kept])
    return out, gap, margin, cut


def _topk_bounds(xb, k, tol_x):
    """For one row of x: the ids ordered by x descending then id, and the ids
    certainly in the top-k set and possibly in it when every x may be off by
    up to tol_x / 2 (S- = x above x(k+1) + tol_x, S+ = x at least x(k) - tol_x;
    every valid id when there are at most k)."""
    valid = np.nonzero(np.isfinite(xb))[0]
    order = valid[np.lexsort((valid, -xb[valid]))]
    if order.size <= k:
        return order, order, order
    xk, xk1 = xb[order[k - 1]], xb[order[k]]
    s_minus = valid[xb[valid] > xk1 + tol_x]
    s_plus = valid[xb[valid] >= xk - tol_x]
    return order, s_minus, s_plus


def topk_pick_margin(x, s, k, tol_x):
    """How robust the top-k sample of each row is when x (and with it s) may be
    off by up to tol_x / 2 per id, as a GPU's FP32 logits are.

    Every top-k set the perturbed x can give lies between S- and S+ (see
    _topk_bounds), and the sample over any set between them is the same
    exactly when the argmax of s over S+ lies in S-.  Then the returned value
    is the top-two gap of s over S+ (the noise error the sample withstands);
    otherwise 0.  With x(k) - x(k+1) > 2 tol_x, S- = S+ = the top-k set and
    this is topk_sample's own gap.  Rows with no valid id give inf."""
    x = np.asarray(x, np.float64)
    s = np.asarray(s, np.float64)
    out = np.full(x.shape[0], math.inf)
    for b in range(x.shape[0]):
        order, s_minus, s_plus = _topk_bounds(x[b], k, tol_x)
        if order.size == 0:
            continue
        j, _ = first_argmax(s[b, s_plus])
        w = s_plus[j]
        out[b] = top_two_gap(s[b, s_plus]) if w in set(s_minus.tolist()) else 0.0
    return out


def topp_pick_margin(x, s, k, top_p, tol_x, tol_mass):
    """How robust the top-p-after-top-k sample of each row is when x (and s)
    may be off by up to tol_x / 2 per id and the exclusive masses by tol_mass.

    top_p = 1 keeps the whole top-k set: the top-k question
    (topk_pick_margin).  Otherwise, for every possible member j of the top-k
    set (S+), the mass ranked before it and the set's total mass are bounded
    over all admissible perturbations: weights scale by at most 1 +- rho
    (rho = e^(tol_x/2) - 1); at least the certain members (S-) with x above
    x_j + tol_x rank before j, at most every possible member with x at least
    x_j - tol_x does; the total lies between the smallest and largest sums of
    k possible members.  j is certainly kept when it is a certain member and
    even its largest exclusive mass stays below top_p - tol_mass, possibly
    kept when its smallest one is below top_p + tol_mass.  The sample is the
    same for every admissible kept set exactly when the argmax of s over the
    possibly kept ids is certainly kept; the value is then the top-two gap of
    s over the possibly kept ids, otherwise 0."""
    x = np.asarray(x, np.float64)
    s = np.asarray(s, np.float64)
    out = np.full(x.shape[0], math.inf)
    if top_p >= 1:
        return topk_pick_margin(x, s, k, tol_x)
    rho = math.expm1(tol_x / 2)
    for b in range(x.shape[0]):
        order, s_minus, s_plus = _topk_bounds(x[b], k, tol_x)
        if order.size == 0:
            continue
        cand = s_plus[np.lexsort((s_plus, -x[b, s_plus]))]   # by x descending, then id
        xc = x[b, cand]
        wc = np.exp(xc - xc[0])
        sure = np.isin(cand, s_minus)
        zone = np.sort(wc[~sure])
        n_more = min(k, cand.size) - int(sure.sum())
        z_sure = wc[sure].sum()
        z_lo = (z_sure + (zone[:n_more].sum() if n_more > 0 else 0.0)) * (1 - rho)
        z_hi = (z_sure + (zone[zone.size - n_more:].sum() if n_more > 0 else 0.0)) * (1 + rho)
        csum_sure = np.concatenate([[0.0], np.cumsum(np.where(sure, wc, 0.0))])
        csum_all = np.concatenate([[0.0], np.cumsum(wc)])
        before_min = np.searchsorted(-xc, -(xc + tol_x), side="left")    # x_i > x_j + tol_x
        before_max = np.searchsorted(-xc, -(xc - tol_x), side="right")   # x_i >= x_j - tol_x
        p_min = csum_sure[before_min] * (1 - rho)
        p_max = (csum_all[before_max] - wc) * (1 + rho)
        certain = sure & (p_max / z_lo < top_p - tol_mass)
        possible = p_min / z_hi < top_p + tol_mass
        k_plus = np.sort(cand[possible])
        k_minus = set(cand[certain].tolist())
        j, _ = first_argmax(s[b, k_plus])
        out[b] = top_two_gap(s[b, k_plus]) if int(k_plus[j]) in k_minus else 0.0
    return out


def multinomial(x, temp=None, seed=0, step=0, flags=0, id0=0):
    """Unfused baseline: inverse-CDF draw from softmax(x) ([FS-kr] problem
    statement: logits are written, read back, turned into probabilities and
    a draw is made).  u = (r + 1/2) 2^-32 with r word 0 of the stream-3
    block (0, b, step, 3); i = smallest id with cumsum(p)_i > u.
    Greedy rows return argmax x.
    Returns (idx [B], distance of u to the nearest CDF boundary [B])."""
    x = np.asarray(x, np.float64)
    B, V = x.shape
    greedy = greedy_rows(temp, B, flags)
    out = np.full(B, -1, np.int64)
    margin = np.full(B, math.inf)
    for b in range(B):
        if greedy[b]:
            j, _ = first_argmax(x[b])
            out[b] = -1 if j < 0 else id0 + j
            continue
        lse = log_sum_exp(x[b])
        if lse == NEG_INF:
            continue
        p = np.exp(x[b] - lse)
        cdf = np.cumsum(p)
        u = float(uniform_from_word(px.noise_words(row_seed(seed, b), b, np.array([0]), step,
                                                   px.STREAM_MULTINOMIAL))[0])
        j = int(np.searchsorted(cdf, u, side="right"))
        if j >= V:                       # u beyond the rounded total: last valid id
            j = int(np.nonzero(np.isfinite(x[b]))[0][-1])
        out[b] = id0 + j
        lo = cdf[j - 1] if j > 0 else 0.0
        margin[b] = min(u - lo, cdf[j] - u)
    return out, margin


# ----------------------------------------------------------------------------
# one full call, as the library's entry points define it
# ----------------------------------------------------------------------------
def run_call(l, temp=None, n_valid=None, allow=None, seed=0, step=0, flags=0,
             tile_v=128, id0=0):
    """Everything the fused entry points return, from logits l [B, V].

    Returns a dict with x, s, flat (idx, max, gap), tile records
    (m, idx, L, gap) and the hierarchical sample (idx, gap)."""
    B = l.shape[0]
    greedy = greedy_rows(temp, B, flags)
    x = tempered(l, temp, n_valid, allow, flags, id0)
    s = scores(x, temp, seed, step, flags, id0)
    fidx, fmax, fgap = sample_flat(s, id0)
    m, tidx, L, tgap = tile_records(x, s, tile_v, greedy, id0)
    gidx, ggap, gt = sample_grouped(tidx, L, temp, seed, step, flags)
    return dict(x=x, s=s, greedy=greedy, flat_idx=fidx, flat_max=fmax, flat_gap=fgap,
                tile_m=m, tile_idx=tidx, tile_L=L, tile_gap=tgap,
                grp_idx=gidx, grp_gap=ggap, grp_tile=gt)
