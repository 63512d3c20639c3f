"""Goodness-of-fit helpers shared by the statistical tests."""
import numpy as np
from scipy import stats


def equal_mass_bins(p, min_expected, n):
    """Group categories (sorted by probability) into bins whose expected count
    n * sum(p) is at least `min_expected`.  Returns a bin id per category."""
    p = np.asarray(p, np.float64)
    order = np.argsort(-p, kind="stable")
    bins = np.empty(p.size, np.int64)
    cur, acc = 0, 0.0
    for j in order:
        bins[j] = cur
        acc += p[j] * n
        if acc >= min_expected:
            cur, acc = cur + 1, 0.0
    if acc > 0 and cur > 0:          # fold an under-filled last bin into the previous one
        bins[bins == cur] = cur - 1
    return bins


def chi_square_p(samples, p, min_expected=5.0):
    """p-value of Pearson's chi-square test of `samples` (category ids)
    against probabilities `p`; categories are pooled so every expected count
    is at least `min_expected`.  A sample outside the support of p fails."""
    samples = np.asarray(samples, np.int64)
    p = np.asarray(p, np.float64)
    n = samples.size
    if np.any(samples < 0) or np.any(samples >= p.size) or np.any(p[samples] <= 0):
        return 0.0
    support = p > 0
    idx = np.nonzero(support)[0]
    bins = equal_mass_bins(p[idx], min_expected, n)
    nb = int(bins.max()) + 1
    if nb < 2:
        return 1.0
    remap = np.full(p.size, -1, np.int64)
    remap[idx] = bins
    obs = np.bincount(remap[samples], minlength=nb).astype(np.float64)
    exp = np.bincount(bins, weights=p[idx] * n, minlength=nb)
    return float(stats.chisquare(obs, exp).pvalue)


def softmax(x):
    x = np.asarray(x, np.float64)
    m = np.max(x)
    e = np.exp(x - m)
    return e / e.sum()


def chi_square_rows_p(samples_rows, p_rows, min_expected=5.0):
    """Pooled Pearson chi-square over several independent rows: row r's
    draws `samples_rows[r]` against its own probabilities `p_rows[r]`, each
    row binned to expected counts >= min_expected.  Returns the p-value of the
    summed statistic (degrees of freedom summed over rows)."""
    stat, dof = 0.0, 0
    for samples, p in zip(samples_rows, p_rows):
        samples = np.asarray(samples, np.int64)
        p = np.asarray(p, np.float64)
        n = samples.size
        if np.any(samples < 0) or np.any(samples >= p.size) or np.any(p[samples] <= 0):
            return 0.0
        idx = np.nonzero(p > 0)[0]
        bins = equal_mass_bins(p[idx], min_expected, n)
        nb = int(bins.max()) + 1
        if nb < 2:
            continue
        remap = np.full(p.size, -1, np.int64)
        remap[idx] = bins
        obs = np.bincount(remap[samples], minlength=nb).astype(np.float64)
        exp = np.bincount(bins, weights=p[idx] * n, minlength=nb)
        stat += float(((obs - exp) ** 2 / exp).sum())
        dof += nb - 1
    if dof == 0:
        return 1.0
    return float(stats.chi2.sf(stat, dof))
