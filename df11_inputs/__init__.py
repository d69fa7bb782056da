"""Seeded synthetic BF16 inputs shared by the oracle tests, the GPU tests and
the benchmark.

This module holds no part of the coding method: it only draws numbers and
rounds them to BF16.  Every generator returns raw BF16 bit patterns as a flat
``numpy.uint16`` array (matrices concatenated row-major in the order given).

Workloads (stand-ins for real checkpoint weights, which are not available):
  C1  one 256x256 matrix, N(0, 0.02^2)                                seed 1
  C2  one 4096x4096 matrix, N(0, 0.02^2)                              seed 2
  C3  Llama-3.1-8B-shaped block q,k,v,o,gate,up,down with hidden 4096,
      kv 1024, ffn 14336; row r of each matrix ~ N(0, (0.02 u_r)^2),
      u_r ~ U(0.5, 2)                                                 seed 3
  C4  Llama-3.1-70B-shaped block (8192, 1024, 28672), sigma 0.015     seed 4
  C5  Llama-3.1-405B-shaped block (16384, 1024, 53248),
      0.01 * Student-t(df=3), i.i.d.                                  seed 5
  E8  one Llama-3.1-8B token-embedding / LM-head-shaped matrix,
      128256 x 4096, row r ~ N(0, (0.015 u_r)^2), u_r ~ U(0.5, 2),
      its own codebook                                                seed 6

Recipe (fixed, independent of the thread count): every matrix is cut into
row blocks of ``ROW_BLOCK`` rows; block b of matrix m draws from
``Generator(PCG64(SeedSequence([seed, m, b])))``: first the row scales
(uniform(0.5, 2.0) per row, when the config has them), then the values
row-major.  Normal values are drawn as float32 and multiplied by the float32
scale ``sigma * u_r``; Student-t values are drawn as float64, multiplied by the
scale and cast to float32.  float32 -> BF16 uses round-to-nearest-even
(torch's conversion).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

ROW_BLOCK = 256


@dataclass(frozen=True)
class Matrix:
    name: str
    rows: int
    cols: int


@dataclass(frozen=True)
class Workload:
    key: str
    description: str
    mats: tuple
    dist: str            # "normal" or "t3"
    scale: float
    row_scale: bool
    seed: int
    shared_codebook: bool = True

    @property
    def numel(self) -> int:
        return sum(m.rows * m.cols for m in self.mats)

    @property
    def mat_numel(self) -> list:
        return [m.rows * m.cols for m in self.mats]


def _llama_block(hidden: int, kv: int, ffn: int) -> tuple:
    return (
        Matrix("q_proj", hidden, hidden),
        Matrix("k_proj", kv, hidden),
        Matrix("v_proj", kv, hidden),
        Matrix("o_proj", hidden, hidden),
        Matrix("gate_proj", ffn, hidden),
        Matrix("up_proj", ffn, hidden),
        Matrix("down_proj", hidden, ffn),
    )


WORKLOADS = {
    "C1": Workload("C1", "single 256x256 BF16 matrix, N(0, 0.02)",
                   (Matrix("w", 256, 256),), "normal", 0.02, False, 1, False),
    "C2": Workload("C2", "single 4096x4096 BF16 matrix, N(0, 0.02)",
                   (Matrix("w", 4096, 4096),), "normal", 0.02, False, 2, False),
    "C3": Workload("C3", "Llama-3.1-8B-shaped transformer block, N(0, 0.02) x U(0.5,2) row scale",
                   _llama_block(4096, 1024, 14336), "normal", 0.02, True, 3),
    "C4": Workload("C4", "Llama-3.1-70B-shaped transformer block, N(0, 0.015) x U(0.5,2) row scale",
                   _llama_block(8192, 1024, 28672), "normal", 0.015, True, 4),
    "C5": Workload("C5", "Llama-3.1-405B-shaped transformer block, 0.01 x Student-t(3)",
                   _llama_block(16384, 1024, 53248), "t3", 0.01, False, 5),
    "E8": Workload("E8", "Llama-3.1-8B token-embedding / LM-head-shaped matrix 128256x4096, "
                   "N(0, 0.015) x U(0.5,2) row scale, own codebook",
                   (Matrix("embed_tokens", 128256, 4096),), "normal", 0.015, True, 6, False),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns with round-to-nearest-even (torch)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _block_values(wl: Workload, m_idx: int, mat: Matrix, b: int) -> np.ndarray:
    r0 = b * ROW_BLOCK
    rows = min(ROW_BLOCK, mat.rows - r0)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, m_idx, b])))
    if wl.row_scale:
        u = rng.uniform(0.5, 2.0, size=rows)
        s = (wl.scale * u).astype(np.float32)[:, None]
    else:
        s = np.float32(wl.scale)
    if wl.dist == "normal":
        v = rng.standard_normal((rows, mat.cols), dtype=np.float32)
        v *= s
        return v
    if wl.dist == "t3":
        v = rng.standard_t(3.0, size=(rows, mat.cols))
        v *= np.float64(wl.scale) if not wl.row_scale else s.astype(np.float64)
        return v.astype(np.float32)
    raise ValueError(wl.dist)


def generate(key: str, threads: int | None = None) -> np.ndarray:
    """Flat uint16 BF16 bits of workload `key` (C1..C5, E8)."""
    wl = WORKLOADS[key]
    out = np.empty(wl.numel, dtype=np.uint16)
    jobs = []
    off = 0
    for m_idx, mat in enumerate(wl.mats):
        for b in range((mat.rows + ROW_BLOCK - 1) // ROW_BLOCK):
            r0 = b * ROW_BLOCK
            rows = min(ROW_BLOCK, mat.rows - r0)
            jobs.append((m_idx, mat, b, off + r0 * mat.cols, rows * mat.cols))
        off += mat.rows * mat.cols

    def run(job):
        m_idx, mat, b, start, count = job
        out[start:start + count] = f32_to_bf16_bits(_block_values(wl, m_idx, mat, b)).reshape(-1)

    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if threads <= 1 or len(jobs) == 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(run, jobs))
    return out


def split(key: str, flat: np.ndarray) -> list:
    """Per-matrix views of a generated block."""
    wl = WORKLOADS[key]
    views, off = [], 0
    for m in wl.mats:
        n = m.rows * m.cols
        views.append(flat[off:off + n])
        off += n
    return views


# ---------------------------------------------------------------- edge inputs

def all_bf16_patterns(seed: int | None = None) -> np.ndarray:
    """All 65,536 BF16 bit patterns, in order or in a seeded permutation."""
    a = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if seed is not None:
        a = a[np.random.Generator(np.random.PCG64(seed)).permutation(65536)]
    return a


def from_exponents(exps: np.ndarray, seed: int) -> np.ndarray:
    """BF16 patterns with the given exponent fields and random sign/mantissa."""
    exps = np.asarray(exps, dtype=np.uint16)
    rng = np.random.Generator(np.random.PCG64(seed))
    sign = rng.integers(0, 2, size=exps.size, dtype=np.uint16)
    mant = rng.integers(0, 128, size=exps.size, dtype=np.uint16)
    return ((sign << 15) | ((exps & 0xFF) << 7) | mant).astype(np.uint16)


def high_exponents(n: int, seed: int) -> np.ndarray:
    """Only exponent fields 240..255 (huge values, Inf and NaN patterns)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return from_exponents(rng.integers(240, 256, size=n), seed + 1)


def single_exponent(n: int, exponent: int, seed: int) -> np.ndarray:
    return from_exponents(np.full(n, exponent), seed)


def fibonacci_exponents(k: int = 34, first_exponent: int = 100, seed: int = 34) -> np.ndarray:
    """k distinct exponents with Fibonacci counts 1,1,2,3,5,... shuffled.

    With k = 34 the unrestricted Huffman code is 33 bits deep."""
    fib = [1, 1]
    while len(fib) < k:
        fib.append(fib[-1] + fib[-2])
    fib = fib[:k]
    exps = np.repeat(np.arange(first_exponent, first_exponent + k, dtype=np.uint16),
                     np.asarray(fib, dtype=np.int64))
    rng = np.random.Generator(np.random.PCG64(seed))
    rng.shuffle(exps)
    return from_exponents(exps, seed + 1)


def skewed(n: int, n_symbols: int, alpha: float, seed: int) -> np.ndarray:
    """Exponents drawn from a Zipf-like law over n_symbols random exponents."""
    rng = np.random.Generator(np.random.PCG64(seed))
    syms = rng.choice(256, size=n_symbols, replace=False)
    p = 1.0 / np.arange(1, n_symbols + 1, dtype=np.float64) ** alpha
    p /= p.sum()
    return from_exponents(syms[rng.choice(n_symbols, size=n, p=p)], seed + 1)


def random_normal(n: int, sigma: float, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return f32_to_bf16_bits(rng.standard_normal(n, dtype=np.float32) * np.float32(sigma))


def many_subtables(r: int = 1000, seed: int = 127) -> np.ndarray:
    """Exponent counts A: 300r, B: 2r and r for each of the other 254 values.

    The Huffman code then has one 1-bit code, one 8-bit code and 254 9-bit
    codes, which need 127 second-level decode tables."""
    a, b = 127, 126
    others = np.array([e for e in range(256) if e not in (a, b)], dtype=np.uint16)
    exps = np.concatenate([np.full(300 * r, a, np.uint16), np.full(2 * r, b, np.uint16),
                           np.repeat(others, r)])
    rng = np.random.Generator(np.random.PCG64(seed))
    rng.shuffle(exps)
    return from_exponents(exps, seed + 1)


# ---------------------------------------------------------------- random blocks

RANDOM_FAMILIES = ("normal", "student_t", "any_pattern", "sparse", "skewed", "row_scaled")


def random_block(seed: int, max_n: int = 1 << 20, min_n: int = 1) -> tuple:
    """A seeded random block for property tests: (flat BF16 bits, matrix split,
    description).  The seed picks a value family (normal with a log-uniform
    sigma, scaled Student-t, any 16-bit pattern, mostly zeros, a Zipf law over
    random exponents, or rows with their own scales), a log-uniform size in
    [min_n, max_n] and a split into 1 to 7 matrices at random points."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([7919, seed])))
    family = RANDOM_FAMILIES[seed % len(RANDOM_FAMILIES)]
    n = int(np.exp(rng.uniform(np.log(min_n), np.log(max_n))))
    sub = int(rng.integers(0, 2**31))
    if family == "normal":
        sigma = float(np.exp(rng.uniform(np.log(1e-4), np.log(10.0))))
        x = random_normal(n, sigma, sub)
        what = f"normal sigma={sigma:.3g}"
    elif family == "student_t":
        df = float(rng.choice([1.0, 2.0, 3.0, 5.0]))
        scale = float(np.exp(rng.uniform(np.log(1e-3), np.log(1.0))))
        g = np.random.Generator(np.random.PCG64(sub))
        x = f32_to_bf16_bits((g.standard_t(df, size=n) * scale).astype(np.float32))
        what = f"student_t df={df:g} scale={scale:.3g}"
    elif family == "any_pattern":
        g = np.random.Generator(np.random.PCG64(sub))
        x = g.integers(0, 65536, size=n, dtype=np.uint32).astype(np.uint16)
        what = "any 16-bit pattern"
    elif family == "sparse":
        frac = float(rng.uniform(0.5, 0.999))
        g = np.random.Generator(np.random.PCG64(sub))
        v = g.standard_normal(n, dtype=np.float32) * np.float32(0.02)
        v[g.random(n) < frac] = 0.0
        x = f32_to_bf16_bits(v)
        what = f"sparse zeros={frac:.3f}"
    elif family == "skewed":
        k = int(rng.integers(1, 257))
        alpha = float(rng.uniform(0.0, 3.0))
        x = skewed(n, k, alpha, sub)
        what = f"skewed symbols={k} alpha={alpha:.2f}"
    else:
        cols = int(rng.integers(1, 2049))
        rows = max(1, n // cols)
        g = np.random.Generator(np.random.PCG64(sub))
        u = g.uniform(0.5, 2.0, size=rows).astype(np.float32)
        x = f32_to_bf16_bits((g.standard_normal((rows, cols), dtype=np.float32) *
                              (np.float32(0.02) * u)[:, None]).reshape(-1))
        n = x.size
        what = f"row_scaled {rows}x{cols}"
    k = int(rng.integers(1, 8))
    cuts = np.sort(rng.integers(0, n + 1, size=k - 1)) if n else np.zeros(k - 1, dtype=np.int64)
    mats = np.split(x, cuts)
    return x, mats, f"{family} n={n} mats={k} ({what})"
