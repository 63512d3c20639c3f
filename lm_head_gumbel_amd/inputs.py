"""Seeded synthetic inputs for fused LM-head sampling workloads.

This module only draws and rounds data; it holds none of the sampling method's
arithmetic.  The test suite and the benchmark use it to feed the same values
to the HIP library and to the CPU oracle.

Workloads stand in for the decode-time LM heads the FlashSampling pages
measure (Qwen3-class vocabularies of about 150k ids): hidden states
H ~ N(0, 1) and weights W ~ N(0, 0.02^2), drawn in float32 with numpy's
PCG64 generator and rounded to bfloat16 (round to nearest even).  The data
seeds are fixed per tensor: W uses 0, H uses 1, per-row temperatures use 2.
No dataset or trained weights are involved.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

SEED_W, SEED_H, SEED_T = 0, 1, 2
PHILOX_SEED = 1234


def f32_to_bf16_bits(a):
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_f32(shape, std, seed, chunk_rows=16384):
    """float32 N(0, std^2) array drawn row-chunk by row-chunk from one PCG64 stream."""
    rng = np.random.default_rng(seed)
    out = np.empty(shape, np.float32)
    rows = shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = rng.standard_normal((r1 - r0,) + tuple(shape[1:]), dtype=np.float32)
        if std != 1.0:
            out[r0:r1] *= np.float32(std)
    return out


def weights_bf16(V, d, std=0.02, seed=SEED_W):
    """W [V, d] as bfloat16 bit patterns, row-major (one vocab id per row)."""
    W = np.empty((V, d), np.uint16)
    rng = np.random.default_rng(seed)
    chunk = max(1, (1 << 24) // max(d, 1))
    for r0 in range(0, V, chunk):
        r1 = min(V, r0 + chunk)
        blk = rng.standard_normal((r1 - r0, d), dtype=np.float32)
        if std != 1.0:
            blk *= np.float32(std)
        W[r0:r1] = f32_to_bf16_bits(blk)
    return W


def hidden_bf16(B, d, seed=SEED_H):
    """H [B, d] ~ N(0, 1) as bfloat16 bit patterns."""
    return f32_to_bf16_bits(normal_f32((B, d), 1.0, seed))


def temperatures(B, lo, hi, seed=SEED_T):
    """Per-row temperatures uniform on [lo, hi] (float32)."""
    return np.random.default_rng(seed).uniform(lo, hi, size=B).astype(np.float32)


@dataclass
class Workload:
    """One synthetic LM-head workload (shapes and sampling settings)."""
    name: str
    B: int
    d: int
    V: int
    tile_v: int = 128
    temp: Tuple[float, float] = (1.0, 1.0)   # fixed value, or a uniform range
    n_valid: Optional[int] = None            # ids >= n_valid are masked
    w_std: float = 0.02
    k: int = 0                               # top-k size (0: not a top-k workload)
    chunks: int = 0                          # online-merge chunks (0: none)
    steps: int = 1

    def temps(self):
        lo, hi = self.temp
        if lo == hi:
            return np.full(self.B, lo, np.float32)
        return temperatures(self.B, lo, hi)

    def hidden(self):
        return hidden_bf16(self.B, self.d)

    def weights(self):
        return weights_bf16(self.V, self.d, self.w_std)


def tiny_reference():
    """Tiny workload: B=4, d=256, V=4096, float32 H ~ N(0,1) and W ~ N(0, 1/d),
    temperature 1, tiles of 512 ids (8 tiles).  Returns (workload, H f32, W f32);
    the library receives bfloat16-rounded copies of H and W."""
    wl = Workload("tiny", B=4, d=256, V=4096, tile_v=512, w_std=(1.0 / 256) ** 0.5)
    H = normal_f32((4, 256), 1.0, SEED_H)
    W = normal_f32((4096, 256), wl.w_std, SEED_W)
    return wl, H, W


WORKLOADS = {
    # small-model LM head: d=2048, V=151936, T=0.7, 1000 decode steps
    "small_b1": Workload("small_b1", 1, 2048, 151936, 256, (0.7, 0.7), steps=1000),
    "small_b8": Workload("small_b8", 8, 2048, 151936, 256, (0.7, 0.7), steps=1000),
    "small_b32": Workload("small_b32", 32, 2048, 151936, 256, (0.7, 0.7), steps=1000),
    # mid-size LM head, last 285 ids masked (padding), grouped variant
    **{f"mid_b{b}": Workload(f"mid_b{b}", b, 4096, 151936, 128, (1.0, 1.0), n_valid=151936 - 285)
       for b in (1, 4, 16, 64)},
    # compute-leaning: per-row temperatures uniform on [0.3, 1.5], 200 steps
    **{f"large_b{b}": Workload(f"large_b{b}", b, 4096, 128256, 256, (0.3, 1.5), steps=200)
       for b in (128, 256)},
    # top-k (k=40) and an online merge over 8 chunks of 19008 ids
    "topk_b32": Workload("topk_b32", 32, 5120, 152064, 256, (1.0, 1.0), k=40, chunks=8),
}

# The headline sweep: d=4096, V=151936, B in 1..256.
SWEEP_BATCHES = (1, 2, 4, 8, 16, 32, 64, 128, 256)


def sweep_workload(B):
    return Workload(f"sweep_b{B}", B, 4096, 151936, 128, (1.0, 1.0))
