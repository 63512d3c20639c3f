"""Philox-4x32-10 counter-based generator, written out in numpy (test infrastructure).

This module belongs to the CPU oracle.  Only the test suite, the smoke check and
the CPU-baseline leg of the benchmark may import it; the product library never
does, and it shares no code with the HIP sources.

Definition followed: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), section 3 ("Philox").
Philox-4x32 keeps a 128-bit counter as four 32-bit words X0..X3 and a 64-bit
key as two words K0, K1.  One round multiplies X0 and X2 by the fixed
multipliers M0 and M1 (full 64-bit products) and emits

    X0' = hi(M1*X2) xor X1 xor K0     X1' = lo(M1*X2)
    X2' = hi(M0*X0) xor X3 xor K1     X3' = lo(M0*X0)

and between rounds the key is advanced by the Weyl increments W0, W1
(K0 += W0, K1 += W1, modulo 2^32).  The -10 variant applies ten rounds.  The
four output words are the 128-bit random block for that (counter, key).

The pages name only a counter-based generator keyed by seed and offsets
(FlashInfer cake_sampling documentation, "Correctness contract" and the sparse
top-p kernel description) and Gumbel noise drawn from uniforms
(aitrends.kr FlashSampling explainer, Stage 1 paragraph); the block layout
used by this project is in `noise_words` below.
"""
import numpy as np

# Multipliers and Weyl key increments of Philox-4x32 (SC'11, section 3).
M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = np.uint32(0x9E3779B9)
W1 = np.uint32(0xBB67AE85)
_LO = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)

# Noise streams: counter word 3 separates the independent uses of the generator.
STREAM_TOKEN = 0      # per-token Gumbel noise
STREAM_GROUP = 1      # per-group Gumbel noise of the hierarchical resample
STREAM_MERGE = 2      # Bernoulli uniforms of the online binary merge
STREAM_MULTINOMIAL = 3  # inverse-CDF uniform of the unfused baseline


def philox4x32_10(c0, c1, c2, c3, k0, k1, rounds=10):
    """Return the four output words of Philox-4x32-`rounds` (numpy uint32, broadcast).

    c0..c3 are the counter words, k0/k1 the key words; any mix of scalars and
    arrays broadcasts.  All arithmetic is exact integer arithmetic.
    """
    x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint32) for c in (c0, c1, c2, c3))
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    key0 = np.asarray(k0, dtype=np.uint64)
    key1 = np.asarray(k1, dtype=np.uint64)
    for rnd in range(rounds):
        if rnd > 0:  # key schedule: add the Weyl increments modulo 2^32
            key0 = (key0 + np.uint64(W0)) & _LO
            key1 = (key1 + np.uint64(W1)) & _LO
        p0 = x0.astype(np.uint64) * M0
        p1 = x2.astype(np.uint64) * M1
        hi0 = (p0 >> _S32).astype(np.uint32)
        lo0 = (p0 & _LO).astype(np.uint32)
        hi1 = (p1 >> _S32).astype(np.uint32)
        lo1 = (p1 & _LO).astype(np.uint32)
        x0, x1, x2, x3 = (hi1 ^ x1 ^ key0.astype(np.uint32), lo1,
                          hi0 ^ x3 ^ key1.astype(np.uint32), lo0)
    return x0, x1, x2, x3


def key_words(seed):
    """Split a 64-bit seed into the Philox key words (low word first)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return np.uint32(seed & 0xFFFFFFFF), np.uint32(seed >> 32)


def noise_words(seed, b, ids, step, stream):
    """Raw 32-bit noise word for row `b`, global ids `ids`, decode `step`, `stream`.

    Layout: the block with counter (id >> 2, b, step, stream) under key
    (seed low word, seed high word) supplies the words of the four ids that
    share id >> 2; id & 3 selects the word.  Keying by the global id (not by
    tile or thread) makes the noise independent of how the vocabulary is
    partitioned.  `b`, `ids` and `step` broadcast against each other.
    """
    ids = np.asarray(ids, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    step = np.asarray(step, dtype=np.int64)
    ids, b, step = np.broadcast_arrays(ids, b, step)
    k0, k1 = key_words(seed)
    w = philox4x32_10((ids >> 2).astype(np.uint32), b.astype(np.uint32),
                      step.astype(np.uint32), np.uint32(stream), k0, k1)
    sel = ids & 3
    return np.where(sel == 0, w[0], np.where(sel == 1, w[1], np.where(sel == 2, w[2], w[3])))
