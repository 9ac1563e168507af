"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's callers.

This module draws numbers and rounds them to the storage dtype; it contains none of
the attention arithmetic.  Both the HIP path and the CPU oracle receive the very same
bytes: fp32 N(0,1) samples rounded to bf16 (round to nearest, ties to even) on the
host for bf16 workloads, plain fp32 samples for fp32 workloads.

Streams: numpy PCG64 seeded by SeedSequence(seed).spawn(...) in the fixed tensor order
below.  Large tensors are generated in fixed blocks of BLOCK elements, each from its own
spawned child, so the values do not depend on the number of threads used.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Sequence

import numpy as np

from .configs import Workload

# new names go at the end: a stream's seed depends on its index only
STREAMS = ["q", "k_p", "v_p", "k_r", "v_r", "d_o", "q_idx", "k_idx", "r_len", "rows", "k_layer", "v_layer",
           "alpha"]
BLOCK = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _stream_seed(seed: int, name: str) -> np.random.SeedSequence:
    return np.random.SeedSequence(seed).spawn(len(STREAMS))[STREAMS.index(name)]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(seed: int, name: str, shape: Sequence[int], dtype: str) -> np.ndarray:
    """N(0,1) tensor of `shape`: fp32 values (dtype "f32") or bf16 bit patterns (dtype "bf16")."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    nblk = max(1, -(-n // BLOCK))
    kids = _stream_seed(seed, name).spawn(nblk)

    def fill(i: int) -> None:
        lo, hi = i * BLOCK, min(n, (i + 1) * BLOCK)
        x = np.random.Generator(np.random.PCG64(kids[i])).standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = x if dtype == "f32" else f32_to_bf16_bits(x)

    if nblk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values (fp32, or bf16 bit patterns) to fp64 for the oracle."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64)
    return bf16_bits_to_f32(x).astype(np.float64)


def response_lengths(w: Workload) -> np.ndarray:
    """Lengths R_g of the G serially replayed members (integers, inclusive range)."""
    if w.r_min is None:
        return np.full(w.G, w.R, dtype=np.int64)
    g = np.random.Generator(np.random.PCG64(_stream_seed(w.seed, "r_len")))
    return g.integers(w.r_min, w.R, size=w.G, endpoint=True).astype(np.int64)


def resident(w: Workload) -> Dict[str, np.ndarray]:
    """Resident prompt state: K_p, V_p `[P][Hkv][d]` (dense) or the latent rows `[P][d_qk]`
    plus fp32 index keys `[P][idx_dim]` (latent variant)."""
    if w.latent:
        out = {"latent_p": normal(w.seed, "k_p", (w.P, w.d_qk), w.dtype)}
        if w.topk:
            out["k_idx"] = normal(w.seed, "k_idx", (w.P, w.idx_dim), "f32")
        return out
    return {"k_p": normal(w.seed, "k_p", (w.P, w.Hkv, w.d_qk), w.dtype),
            "v_p": normal(w.seed, "v_p", (w.P, w.Hkv, w.d_v), w.dtype)}


def member(w: Workload, g: int = 0, R: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs of replayed member g: Q, the response's own K/V, upstream dO (and q_idx).

    Member g > 0 draws from seed (w.seed + 7919 * g) so every member has its own tensors.
    """
    R = w.R if R is None else R
    seed = w.seed + 7919 * g
    out = {"q": normal(seed, "q", (R, w.Hq, w.d_qk), w.dtype),
           "d_o": normal(seed, "d_o", (R, w.Hq, w.d_v), w.dtype)}
    if w.latent:
        out["latent_r"] = normal(seed, "k_r", (R, w.d_qk), w.dtype)
        if w.topk:
            out["q_idx"] = normal(seed, "q_idx", (R, w.idx_dim), "f32")
    else:
        out["k_r"] = normal(seed, "k_r", (R, w.Hkv, w.d_qk), w.dtype)
        out["v_r"] = normal(seed, "v_r", (R, w.Hkv, w.d_v), w.dtype)
    return out


def lastkv_sequence(seed: int, N: int, Hq: int, Hkv: int, d: int, dtype: str) -> Dict[str, np.ndarray]:
    """Inputs of one layer of a LastKV chunk recurrence over N positions: Q and dO
    [N][Hq][d], the layer's own K/V and the last layer's K/V [N][Hkv][d] (N(0,1), stored in
    `dtype`), and the layer's gates alpha [Hkv] (fp32, uniform in [0.05, 0.95])."""
    g = np.random.Generator(np.random.PCG64(_stream_seed(seed, "alpha")))
    return {"q": normal(seed, "q", (N, Hq, d), dtype), "d_o": normal(seed, "d_o", (N, Hq, d), dtype),
            "k_layer": normal(seed, "k_layer", (N, Hkv, d), dtype),
            "v_layer": normal(seed, "v_layer", (N, Hkv, d), dtype),
            "k_last": normal(seed, "k_p", (N, Hkv, d), dtype), "v_last": normal(seed, "v_p", (N, Hkv, d), dtype),
            "alpha": g.uniform(0.05, 0.95, Hkv).astype(np.float32)}


def lastkv_chunk(w: Workload) -> Dict[str, np.ndarray]:
    """The current chunk of a LastKV workload (w.R positions, after w.P positions of
    history): the last layer's K/V of the whole history [P][Hkv][d], this layer's K/V of the
    previous chunk (the history's last R positions), and Q, K/V, dO of the current chunk;
    gates alpha [Hkv]."""
    C = w.R
    g = np.random.Generator(np.random.PCG64(_stream_seed(w.seed, "alpha")))
    return {"k_last": normal(w.seed, "k_p", (w.P, w.Hkv, w.d_qk), w.dtype),
            "v_last": normal(w.seed, "v_p", (w.P, w.Hkv, w.d_v), w.dtype),
            "k_prev_layer": normal(w.seed, "k_layer", (C, w.Hkv, w.d_qk), w.dtype),
            "v_prev_layer": normal(w.seed, "v_layer", (C, w.Hkv, w.d_v), w.dtype),
            "q": normal(w.seed, "q", (C, w.Hq, w.d_qk), w.dtype),
            "k_cur": normal(w.seed, "k_r", (C, w.Hkv, w.d_qk), w.dtype),
            "v_cur": normal(w.seed, "v_r", (C, w.Hkv, w.d_v), w.dtype),
            "d_o": normal(w.seed, "d_o", (C, w.Hq, w.d_v), w.dtype),
            "alpha": g.uniform(0.05, 0.95, w.Hkv).astype(np.float32)}


def _must_rows(R: int, block: int) -> list:
    """Row 0, row R-1 and both sides of every block boundary (the first row of a partial
    last block among them)."""
    must = {0, R - 1}
    for b in range(block, R, block):
        must.update({b - 1, b})
    return sorted(r for r in must if 0 <= r < R)


def sample_rows(seed: int, R: int, n: int, block: int) -> np.ndarray:
    """Sorted query rows to check at full size: row 0, row R-1, both sides of every block
    boundary, the first row of a partial last block, then seeded rows without replacement."""
    must = _must_rows(R, block)
    if len(must) >= n or len(must) >= R:
        return np.array(must[:max(n, 0)] if len(must) > n else must, dtype=np.int64)
    g = np.random.Generator(np.random.PCG64(_stream_seed(seed, "rows")))
    rest = np.setdiff1d(np.arange(R), np.array(must))
    extra = g.choice(rest, size=min(n - len(must), rest.size), replace=False)
    return np.sort(np.concatenate([np.array(must), extra])).astype(np.int64)


def sample_query_rows(seed: int, R: int, Hq: int, n: int, block: int):
    """n query rows of single heads to check at full size, as (positions, heads) sorted by
    position then head: every position of _must_rows with a seeded head, then seeded
    (position, head) pairs without replacement from the rest."""
    g = np.random.Generator(np.random.PCG64(_stream_seed(seed, "rows")))
    must = np.array(_must_rows(R, block), dtype=np.int64)
    flat = must * Hq + g.integers(0, Hq, must.size)
    k = min(n, R * Hq) - flat.size
    if k > 0:
        rest = np.setdiff1d(np.arange(R * Hq, dtype=np.int64), flat)
        flat = np.concatenate([flat, g.choice(rest, size=k, replace=False)])
    flat = np.sort(flat)
    return flat // Hq, flat % Hq
