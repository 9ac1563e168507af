"""Latent-page sparse variant, fp64 (index scores fp32), step by step.  TEST INFRASTRUCTURE ONLY.

Source: ai.thesatyajit.com/articles/longstraw-2m-rl, section "Two incompatible
architectures, same transaction" (GLM instantiation): resident MLA latent pages and DSA
index-key pages, with the sparse selection rebuilt before attention.  The selection is a
heuristic, so this module follows its steps in order rather than a closed form:

  1. index scores   sigma_ij = q_idx_i . k_idx_j over prompt positions j
  2. selection      the top-k positions of row i by sigma, ties toward the lower j
  3. attention      over the selected latent rows plus the response rows 0..i; every
                    head reads the same latent row: key = all d_qk dims, value = its
                    first d_v dims
  4. backward       response-only: dq, and the response latent rows' gradients split into
                    the key part dk_r [R][d_qk] and the value part dv_r [R][d_v]; nothing
                    flows through the scores or the selection.

Shapes: q [R][H][d_qk], latent_p [P][d_qk], latent_r [R][d_qk], d_o [R][H][d_v],
q_idx [R][di], k_idx [P][di], idx [R][k] (ascending prompt positions).
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np


def index_scores(q_idx: np.ndarray, k_idx: np.ndarray) -> np.ndarray:
    """sigma [R][P] = q_idx . k_idx in fp32 arithmetic.  The scores only decide the
    selection (an integer result), and the pages give them no precision, so they are
    taken in the precision the GPU path takes them in; the summation order still differs,
    so near-ties may rank differently on the two sides."""
    return np.asarray(q_idx, dtype=np.float32) @ np.asarray(k_idx, dtype=np.float32).T


def topk_row(sigma_row: np.ndarray, k: int) -> np.ndarray:
    """Top-k positions of one row by score, ties broken toward the lower position;
    returned in ascending position order.  k >= P selects every position."""
    P = sigma_row.size
    if k >= P:
        return np.arange(P, dtype=np.int64)
    t = np.partition(sigma_row, P - k)[P - k]          # the k-th largest score
    above = np.flatnonzero(sigma_row > t)
    ties = np.flatnonzero(sigma_row == t)[:k - above.size]
    return np.sort(np.concatenate([above, ties])).astype(np.int64)


def topk_select(sigma: np.ndarray, k: int) -> np.ndarray:
    return np.stack([topk_row(sigma[i], k) for i in range(sigma.shape[0])])


def _row_keys(latent_p, latent_r, idx_row, i):
    return np.concatenate([latent_p[idx_row], latent_r[:i + 1]], axis=0)


def sparse_attend(q, latent_p, latent_r, idx, tau: float, d_v: int,
                  rows: Optional[Sequence[int]] = None):
    """O [n][H][d_v], lse [n][H] of the given rows (default all)."""
    R, H, _ = q.shape
    rows = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((rows.size, H, d_v))
    lse = np.zeros((rows.size, H))
    for n, i in enumerate(rows):
        keys = _row_keys(latent_p, latent_r, idx[i], int(i))
        s = tau * (q[i] @ keys.T)                        # [H][n_keys]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        den = e.sum(axis=1, keepdims=True)
        o[n] = (e / den) @ keys[:, :d_v]
        lse[n] = m[:, 0] + np.log(den[:, 0])
    return o, lse


def sparse_attend_bwd(q, latent_p, latent_r, idx, d_o, tau: float, d_v: int,
                      rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Response-only backward of L = sum d_o . O: dq for the given rows, and those rows'
    contributions to dk_r [R][d_qk] and dv_r [R][d_v] (the response latent rows)."""
    R, H, d_qk = q.shape
    rows = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    dq = np.zeros((rows.size, H, d_qk))
    dk_r = np.zeros((R, d_qk))
    dv_r = np.zeros((R, d_v))
    k = idx.shape[1]
    for n, i in enumerate(rows):
        i = int(i)
        keys = _row_keys(latent_p, latent_r, idx[i], i)
        vals = keys[:, :d_v]
        s = tau * (q[i] @ keys.T)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        p = e / e.sum(axis=1, keepdims=True)           # [H][n_keys]
        o = p @ vals
        D = np.sum(d_o[i] * o, axis=1)
        dp = d_o[i] @ vals.T
        ds = p * (dp - D[:, None])
        dq[n] = tau * (ds @ keys)
        dk_r[:i + 1] += tau * (ds[:, k:].T @ q[i])
        dv_r[:i + 1] += p[:, k:].T @ d_o[i]
    return {"dq": dq, "dk_r": dk_r, "dv_r": dv_r}
