"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module only draws random numbers and rounds them to bfloat16; it holds none
of the compression method's arithmetic.  Both the HIP path and the CPU oracle
receive the same host bytes produced here.

Workloads stand in for the tensors a tensor-parallel rank exchanges while
training Qwen-7B (hidden size 4096, MLP intermediate size 11008), the setting of
"FP4Quant: Efficient 4-Bit Communication Compression for Model-Parallel LLM
Training" (abstract; zot.news digest, "Read it as").  No dataset or checkpoint is
involved: every tensor is drawn from numpy's PCG64 generator.

Recipe: draws are float64, cast to float32 (round to nearest even), then rounded
to bfloat16 (round to nearest even) by bit arithmetic.  Large tensors are drawn
in chunks of ``CHUNK_ROWS`` rows, in row order; within a chunk the main draw comes
first and any per-row draw after it.  That chunking is part of the definition.
"""
from __future__ import annotations

import numpy as np

CHUNK_ROWS = 4096

#: name -> (rows, row_len, seed, kind, kind-specific parameter)
CONFIGS = {
    "tiny": (4, 256, 0, "normal", None),
    "act2048": (2048, 4096, 1, "row_scaled_normal", 0.5),
    "outlier8192": (8192, 4096, 2, "student_t_outlier_cols", (3.0, 4, 100.0)),
    "large32768": (32768, 4096, 3, "normal", None),
}
#: receiver-side reduce workload: k peers of rows x row_len, N(0, sigma)
REDUCE_CONFIG = {"name": "reduce_k8_4096x11008", "k": 8, "rows": 4096, "row_len": 11008,
                 "sigma": 1e-3, "seeds": tuple(range(4, 12))}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.

    Inputs must be finite (all generators here produce finite values)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _chunks(rows: int):
    r0 = 0
    while r0 < rows:
        r1 = min(rows, r0 + CHUNK_ROWS)
        yield r0, r1
        r0 = r1


def make_config(name: str, rows: int | None = None) -> np.ndarray:
    """bf16 bit patterns (uint16, shape [rows, row_len]) of a named workload.

    ``rows`` may truncate the row count (the first rows of the same stream)."""
    full_rows, row_len, seed, kind, par = CONFIGS[name]
    n_rows = full_rows if rows is None else min(rows, full_rows)
    rng = np.random.default_rng(seed)
    out = np.empty((n_rows, row_len), dtype=np.uint16)
    if kind == "normal":
        for r0, r1 in _chunks(full_rows):
            if r0 >= n_rows:
                break
            z = rng.standard_normal((r1 - r0, row_len))
            take = min(r1, n_rows) - r0
            out[r0:r0 + take] = f32_to_bf16_bits(z[:take].astype(np.float32))
    elif kind == "row_scaled_normal":
        for r0, r1 in _chunks(full_rows):
            if r0 >= n_rows:
                break
            z = rng.standard_normal((r1 - r0, row_len))
            c = np.exp(rng.normal(0.0, par, size=(r1 - r0, 1)))
            take = min(r1, n_rows) - r0
            out[r0:r0 + take] = f32_to_bf16_bits((c * z)[:take].astype(np.float32))
    elif kind == "student_t_outlier_cols":
        nu, ncols, factor = par
        vals = np.empty((n_rows, row_len), dtype=np.float64)
        for r0, r1 in _chunks(full_rows):
            t = rng.standard_t(nu, size=(r1 - r0, row_len))
            if r0 < n_rows:
                take = min(r1, n_rows) - r0
                vals[r0:r0 + take] = t[:take]
        cols = rng.choice(row_len, ncols, replace=False)
        vals[:, cols] *= factor
        out[:] = f32_to_bf16_bits(vals.astype(np.float32))
    else:  # pragma: no cover
        raise ValueError(kind)
    return out


def outlier_columns(name: str = "outlier8192") -> np.ndarray:
    """The fixed outlier channels of the Student-t workload (drawn after all t samples)."""
    full_rows, row_len, seed, kind, (nu, ncols, _f) = CONFIGS[name]
    rng = np.random.default_rng(seed)
    for r0, r1 in _chunks(full_rows):
        rng.standard_t(nu, size=(r1 - r0, row_len))
    return np.sort(rng.choice(row_len, ncols, replace=False))


def make_reduce_peer(p: int, rows: int | None = None, row_len: int | None = None) -> np.ndarray:
    """Peer ``p`` of the receiver-side reduce workload: N(0, 1e-3) in bf16 bits."""
    cfg = REDUCE_CONFIG
    n_rows = cfg["rows"] if rows is None else rows
    L = cfg["row_len"] if row_len is None else row_len
    rng = np.random.default_rng(cfg["seeds"][p])
    out = np.empty((n_rows, L), dtype=np.uint16)
    for r0, r1 in _chunks(n_rows):
        z = rng.normal(0.0, cfg["sigma"], size=(r1 - r0, L))
        out[r0:r1] = f32_to_bf16_bits(z.astype(np.float32))
    return out


def make_normal(rows: int, row_len: int, seed: int, scale: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits((scale * rng.standard_normal((rows, row_len))).astype(np.float32))


def make_edge_case(kind: str, rows: int, row_len: int, seed: int = 0) -> np.ndarray:
    """Degenerate and extreme inputs (bf16 bits) for parity edge cases.

    kinds: zeros, ones, spike (16 at the first element of every 256-block),
    tiny (bfloat16 subnormals and values near underflow), huge (|x| up to about
    2**103), sparse (90 % zeros), ties (small integers, which make exact
    rounding ties common), mixed_blocks (a different kind per 256-block)."""
    rng = np.random.default_rng(seed)
    n = rows * row_len
    if kind == "zeros":
        v = np.zeros(n, np.float32)
    elif kind == "ones":
        v = np.ones(n, np.float32)
    elif kind == "spike":
        v = np.zeros(n, np.float32)
        v[::256] = 16.0
    elif kind == "tiny":
        e = rng.integers(-133, -100, size=n)
        v = (rng.standard_normal(n) * np.exp2(e)).astype(np.float32)
    elif kind == "huge":
        e = rng.integers(60, 101, size=n)
        v = (rng.standard_normal(n) * np.exp2(e)).astype(np.float32)
    elif kind == "sparse":
        v = rng.standard_normal(n).astype(np.float32)
        v[rng.random(n) < 0.9] = 0.0
    elif kind == "ties":
        v = rng.integers(-8, 9, size=n).astype(np.float32)
    elif kind == "mixed_blocks":
        kinds = ["zeros", "ones", "spike", "tiny", "huge", "sparse", "ties", "normal"]
        v = np.empty(n, np.float32)
        nb = n // 256
        for b in range(nb):
            k = kinds[b % len(kinds)]
            if k == "normal":
                blk = rng.standard_normal(256).astype(np.float32)
            else:
                blk = bf16_bits_to_f32(make_edge_case(k, 1, 256, seed + b)).reshape(-1)
            v[256 * b:256 * (b + 1)] = blk
    else:
        raise ValueError(kind)
    return f32_to_bf16_bits(v).reshape(rows, row_len)


def make_random_mixture(rows: int, row_len: int, seed: int) -> np.ndarray:
    """Random stress input (bf16 bits): every row has its own scale 2^u, u uniform
    in [-30, 30], and every 256-block its own kind -- normal, Student-t (nu=2),
    uniform, sparse normal (75 % zeros), constant, one spike among small
    values, bf16-subnormal tiny values, or small integers (rounding ties)."""
    rng = np.random.default_rng(seed)
    nb = row_len // 256
    v = np.empty((rows, nb, 256), np.float64)
    kinds = rng.integers(0, 8, size=(rows, nb))
    for r in range(rows):
        scale = 2.0 ** rng.uniform(-30, 30)
        for b in range(nb):
            k = kinds[r, b]
            if k == 0:
                blk = rng.standard_normal(256)
            elif k == 1:
                blk = rng.standard_t(2, 256)
            elif k == 2:
                blk = rng.uniform(-1, 1, 256)
            elif k == 3:
                blk = rng.standard_normal(256) * (rng.random(256) < 0.25)
            elif k == 4:
                blk = np.full(256, rng.standard_normal())
            elif k == 5:
                blk = rng.standard_normal(256) * 1e-3
                blk[rng.integers(256)] = 100.0
            elif k == 6:
                blk = rng.standard_normal(256) * 2.0 ** -128 / scale
            else:
                blk = rng.integers(-6, 7, 256).astype(np.float64) / scale
            v[r, b] = blk * scale
    return f32_to_bf16_bits(v.reshape(rows, row_len).astype(np.float32))
