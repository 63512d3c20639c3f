"""Pins for the oracle's Philox-4x32-10 and its Gumbel transform (CPU only).

The oracle's generator is checked against (1) the published known-answer
vectors of the generator's authors, (2) rocRAND's independent open-source
implementation on thousands of random (counter, key) tuples, and (3) the
statistics a uniform 32-bit stream must show.  The Gumbel transform is
checked against the Gumbel law's closed forms.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import fs_oracle as O
from oracle import philox as px

HERE = os.path.dirname(os.path.abspath(__file__))
EULER_GAMMA = 0.5772156649015329


def _kat_rows():
    rows = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(t, 16) for t in line.split()])
    return rows


def test_philox_known_answers():
    rows = _kat_rows()
    assert len(rows) == 3
    for r in rows:
        out = px.philox4x32_10(*r[:6])
        assert [int(v) for v in out] == r[6:]


@pytest.fixture(scope="module")
def rocrand_probe(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    inc = "/opt/rocm/include"
    if cxx is None or not os.path.exists(os.path.join(inc, "rocrand", "rocrand_philox4x32_10.h")):
        pytest.skip("rocRAND headers or a host C++ compiler are not available")
    exe = str(tmp_path_factory.mktemp("rocrand") / "probe")
    subprocess.run([cxx, "-O1", "-D__HIP_PLATFORM_AMD__", "-I", inc,
                    os.path.join(HERE, "helpers", "philox_rocrand_probe.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def test_philox_matches_rocrand(rocrand_probe):
    rng = np.random.default_rng(7)
    n = 4096
    tup = rng.integers(0, 2 ** 32, size=(n, 6), dtype=np.uint64).astype(np.uint32)
    tup[:16] = 0                                  # a few degenerate counters and keys
    tup[16:32] = 0xFFFFFFFF
    inp = "\n".join(" ".join(str(int(v)) for v in row) for row in tup) + "\n"
    res = subprocess.run([rocrand_probe], input=inp, capture_output=True, text=True, check=True)
    ref = np.array([[int(t) for t in ln.split()] for ln in res.stdout.strip().splitlines()],
                   dtype=np.uint64)
    out = px.philox4x32_10(tup[:, 0], tup[:, 1], tup[:, 2], tup[:, 3], tup[:, 4], tup[:, 5])
    mine = np.stack([o.astype(np.uint64) for o in out], axis=1)
    assert ref.shape == mine.shape
    assert np.array_equal(ref, mine)


def test_noise_word_layout_selects_block_words():
    # ids 4j..4j+3 of one row take the four words of block (j, b, step, stream)
    seed, b, step = 0x1234_5678_9ABC_DEF0, 5, 77
    k0, k1 = px.key_words(seed)
    assert (int(k0), int(k1)) == (0x9ABCDEF0, 0x12345678)
    ids = np.arange(40, 48)
    words = px.noise_words(seed, b, ids, step, px.STREAM_GROUP)
    for j in (10, 11):
        blk = px.philox4x32_10(j, b, step, px.STREAM_GROUP, k0, k1)
        assert [int(w) for w in blk] == [int(w) for w in words[(j - 10) * 4:(j - 10) * 4 + 4]]


def test_philox_stream_uniformity():
    # 2^20 words from consecutive counters: chi-square over 4096 equal bins
    # and the balance of every bit position.
    ids = np.arange(1 << 20)
    w = px.noise_words(1234, 0, ids, 0, px.STREAM_TOKEN).astype(np.uint64)
    counts = np.bincount((w >> np.uint64(20)).astype(np.int64), minlength=4096)
    p = stats.chisquare(counts).pvalue
    assert p > 1e-4
    n = w.size
    for bit in range(32):
        ones = int(((w >> np.uint64(bit)) & np.uint64(1)).sum())
        assert abs(ones - n / 2) < 5 * math.sqrt(n / 4)


def test_streams_and_rows_are_distinct():
    ids = np.arange(1024)
    a = px.noise_words(1234, 0, ids, 0, 0)
    for other in (px.noise_words(1234, 1, ids, 0, 0), px.noise_words(1234, 0, ids, 1, 0),
                  px.noise_words(1234, 0, ids, 0, 1), px.noise_words(1235, 0, ids, 0, 0)):
        assert np.mean(a == other) < 0.01


def test_gumbel_law():
    # g from 2^20 consecutive words: moments and the Gumbel CDF exp(-exp(-g)).
    w = px.noise_words(99, 3, np.arange(1 << 20), 5, px.STREAM_TOKEN)
    g = O.gumbel_from_word(w)
    assert abs(g.mean() - EULER_GAMMA) < 5 * (math.pi / math.sqrt(6)) / math.sqrt(g.size)
    assert abs(g.var() - math.pi ** 2 / 6) < 0.02
    ks = stats.kstest(g, lambda t: np.exp(-np.exp(-t)))
    assert ks.pvalue > 1e-3


def test_gumbel_transform_endpoints_and_order():
    r = np.array([0, 1, 2 ** 20, 2 ** 31, 2 ** 32 - 2, 2 ** 32 - 1], dtype=np.uint64)
    g = O.gumbel_from_word(r)
    assert np.all(np.isfinite(g))
    assert np.all(np.diff(g) < 0)                 # larger word -> larger v -> smaller u -> smaller g
    # r = 0: v = 2^-33, -log u = v (1 + v/2 + ...), so g = 33 ln 2 to within 1e-9
    assert abs(g[0] - 33 * math.log(2)) < 1e-9
    # r = 2^32 - 1: u = 2^-33, so g = -log(33 ln 2)
    assert abs(g[-1] + math.log(33 * math.log(2))) < 1e-9
    # v = 1 - 1/e gives u = 1/e, -log u = 1, g = 0; the nearest word is within one step
    r0 = int(round((1 - math.exp(-1)) * 2 ** 32 - 0.5))
    assert abs(float(O.gumbel_from_word(np.array([r0], np.uint64))[0])) < 1e-8


def test_uniform_grid_is_open_interval():
    v = O.uniform_from_word(np.array([0, 2 ** 32 - 1], dtype=np.uint64))
    assert v[0] == 2.0 ** -33 and v[1] == 1 - 2.0 ** -33
