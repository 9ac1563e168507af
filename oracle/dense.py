"""Dense response-replay attention, fp64, by definition.  TEST INFRASTRUCTURE ONLY.

Notation (one replayed response; a replay microbatch of K responses is K independent
calls):
  q    [R][Hq][d_qk]   queries of the replayed response rows
  k_p  [P][Hkv][d_qk]  resident prompt keys   (stop-gradient state)
  v_p  [P][Hkv][d_v]   resident prompt values (stop-gradient state)
  k_r  [R][Hkv][d_qk]  the response's own keys
  v_r  [R][Hkv][d_v]   the response's own values
  d_o  [R][Hq][d_v]    upstream gradient of the output
  tau                  softmax scale
Query head h reads KV head h // (Hq // Hkv) (contiguous GQA groups).  Row i sees every
prompt position and the response positions 0..i (diagonal included).

Sources
  * Resident state z_p = stopgrad(z_p(theta)) and response replay:
    ai.thesatyajit.com/articles/longstraw-2m-rl, section "The move: change the graph
    boundary".  The gradient kept is the direct response term; the term through the
    prompt state is dropped (same section), which here means no gradient for k_p, v_p.
  * Rank-local softmax statistics composed into the exact global output, and response
    blocks replayed in reverse: same page, section "Two incompatible architectures,
    same transaction".
  * Serial replay with accumulation up to one update: same page, section "Serial replay
    makes G a schedule, not a memory multiplier"; and
    networkfinds.com/long-context-rl-is-a-state-lifetime-problem, section "Account for
    memory by lifetime" (update-boundary state).

Because the chunked and block-wise method reaches exactly the plain attention result,
`attend`, `attend_bwd` and `attend_rows` (the same for single query rows of one head)
compute the plain definition: no chunks, no blocks, no online rescaling.  `chunk_partials` and `merge` follow the method's composition step for the
functions that expose it.  Rows are processed in batches only to bound memory; each row
is computed independently, as the definition has it.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

_BATCH_BYTES = 1 << 30


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head h (contiguous groups of Hq // Hkv query heads)."""
    return h // (Hq // Hkv)


def _row_batches(rows: np.ndarray, n_keys: int, batch_bytes: int = _BATCH_BYTES):
    step = max(1, batch_bytes // (8 * max(1, n_keys)))
    for a in range(0, rows.size, step):
        yield rows[a:a + step]


def _visible(k_p, v_p, k_r, v_r, g, last_row):
    """Keys and values one KV head offers to rows <= last_row: all prompt positions,
    then response positions 0..last_row, in fp64 (narrower inputs are widened exactly)."""
    keys = np.concatenate([k_p[:, g, :], k_r[:last_row + 1, g, :]], axis=0, dtype=np.float64)
    vals = np.concatenate([v_p[:, g, :], v_r[:last_row + 1, g, :]], axis=0, dtype=np.float64)
    return keys, vals


def _softmax_rows(s: np.ndarray):
    """Row-wise softmax of s (masked entries -inf); returns (p, lse) with natural-log lse."""
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=1, keepdims=True)
    return e / den, m[:, 0] + np.log(den[:, 0])


def _scores(qh, keys, rows, P, tau):
    """tau * q . k over the visible keys of each row; response key j > row is -inf."""
    s = qh @ keys.T
    s *= tau
    j = np.arange(keys.shape[0] - P)
    s[:, P:][j[None, :] > rows[:, None]] = -np.inf
    return s


def attend(q, k_p, v_p, k_r, v_r, tau: float, rows: Optional[Sequence[int]] = None,
           return_probs: bool = False):
    """Exact attention output O [n][Hq][d_v] and natural-log lse [n][Hq] of the given
    response rows (default: all).  With return_probs (tiny inputs only) also returns the
    probabilities p [n][Hq][P + R] over [prompt; response] positions."""
    R, Hq, _ = q.shape
    P, Hkv, d_v = v_p.shape
    rows = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((rows.size, Hq, d_v))
    lse = np.zeros((rows.size, Hq))
    probs = np.zeros((rows.size, Hq, P + R)) if return_probs else None
    pos = {int(r): n for n, r in enumerate(rows)}
    for rb in _row_batches(rows, P + R):
        at = np.array([pos[int(r)] for r in rb])
        for g in range(Hkv):
            keys, vals = _visible(k_p, v_p, k_r, v_r, g, int(rb.max()))
            for h in (h for h in range(Hq) if kv_head(h, Hq, Hkv) == g):
                p, l = _softmax_rows(_scores(q[rb, h, :], keys, rb, P, tau))
                o[at, h, :] = p @ vals
                lse[at, h] = l
                if return_probs:
                    probs[at, h, :p.shape[1]] = p
    return (o, lse, probs) if return_probs else (o, lse)


def attend_bwd(q, k_p, v_p, k_r, v_r, d_o, tau: float, rows: Optional[Sequence[int]] = None,
               full_sequence: bool = False) -> Dict[str, np.ndarray]:
    """Response-only backward of L = sum_{i,h} d_o[i,h] . O[i,h].

    Returns dq for the given rows (default all) and the contributions of those rows to
    dk_r [R][Hkv][d_qk] and dv_r [R][Hkv][d_v]; with every row included these are the
    full response-key gradients.  Per row i and head h:
      p_ij = exp(tau q.k_j - lse_i),  D_i = d_o_i . O_i,  dp_ij = d_o_i . v_j,
      ds_ij = p_ij (dp_ij - D_i),
      dq_i = tau sum_j ds_ij k_j,  dk_r[j] += tau ds_ij q_i,  dv_r[j] += p_ij d_o_i.
    Prompt keys receive no gradient (stop-gradient resident state).  full_sequence=True
    additionally returns dk_p, dv_p: the prompt-side term the response-only contract
    drops, for differential comparisons only."""
    R, Hq, d_qk = q.shape
    P, Hkv, d_v = v_p.shape
    rows = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    dq = np.zeros((rows.size, Hq, d_qk))
    dk_r = np.zeros((R, Hkv, d_qk))
    dv_r = np.zeros((R, Hkv, d_v))
    if full_sequence:
        dk_p = np.zeros((P, Hkv, d_qk))
        dv_p = np.zeros((P, Hkv, d_v))
    pos = {int(r): n for n, r in enumerate(rows)}
    for rb in _row_batches(rows, P + R):
        last = int(rb.max())
        at = np.array([pos[int(r)] for r in rb])
        for g in range(Hkv):
            keys, vals = _visible(k_p, v_p, k_r, v_r, g, last)
            for h in (h for h in range(Hq) if kv_head(h, Hq, Hkv) == g):
                qh, doh = q[rb, h, :], d_o[rb, h, :]
                p, _ = _softmax_rows(_scores(qh, keys, rb, P, tau))
                o = p @ vals
                D = np.sum(doh * o, axis=1)
                dp = doh @ vals.T
                ds = p * (dp - D[:, None])
                dq[at, h, :] = tau * (ds @ keys)
                dk_r[:last + 1, g, :] += tau * (ds[:, P:].T @ qh)
                dv_r[:last + 1, g, :] += p[:, P:].T @ doh
                if full_sequence:
                    dk_p[:, g, :] += tau * (ds[:, :P].T @ qh)
                    dv_p[:, g, :] += p[:, :P].T @ doh
    out = {"dq": dq, "dk_r": dk_r, "dv_r": dv_r}
    if full_sequence:
        out.update(dk_p=dk_p, dv_p=dv_p)
    return out


def attend_rows(q, k_p, v_p, k_r, v_r, d_o, tau: float, rows: Sequence[int],
                heads: Sequence[int], batch_bytes: int = _BATCH_BYTES) -> Dict[str, np.ndarray]:
    """Forward and response-only backward of individual query rows: entry n is row rows[n]
    of query head heads[n] (one row of that head's query matrix), with everything the
    definition gives for it in one pass over its visible keys:
      o [n][d_v], lse [n] (natural log), D [n] = d_o . o, dq [n][d_qk],
    and the contributions of these query rows to dk_r [R][Hkv][d_qk], dv_r [R][Hkv][d_v]
    (per row and head, the formulas of attend_bwd).  Where the selection holds every head
    of rows j0..R-1, dk_r[j0:] and dv_r[j0:] are the full response-key gradients, as only
    those rows see response keys >= j0.  batch_bytes bounds the fp64 scores held at once
    (a larger batch reads the gathered keys fewer times)."""
    R, Hq, d_qk = q.shape
    P, Hkv, d_v = v_p.shape
    rows = np.asarray(rows, dtype=np.int64)
    heads = np.asarray(heads, dtype=np.int64)
    o = np.zeros((rows.size, d_v))
    lse = np.zeros(rows.size)
    Dv = np.zeros(rows.size)
    dq = np.zeros((rows.size, d_qk))
    dk_r = np.zeros((R, Hkv, d_qk))
    dv_r = np.zeros((R, Hkv, d_v))
    for g in range(Hkv):
        sel = np.flatnonzero(heads // (Hq // Hkv) == g)
        if sel.size == 0:
            continue
        last = int(rows[sel].max())
        keys, vals = _visible(k_p, v_p, k_r, v_r, g, last)
        for b in _row_batches(sel, keys.shape[0], batch_bytes):
            r, h = rows[b], heads[b]
            qb, dob = q[r, h, :], d_o[r, h, :]
            # the softmax and dS = p (dp - D) are formed in place: these arrays hold one
            # value per visible key and row, gigabytes at long prompts
            p = _scores(qb, keys, r, P, tau)
            m = p.max(axis=1, keepdims=True)
            p -= m
            np.exp(p, out=p)
            den = p.sum(axis=1, keepdims=True)
            p /= den
            lse[b] = m[:, 0] + np.log(den[:, 0])
            o[b] = p @ vals
            D = np.sum(dob * o[b], axis=1)
            Dv[b] = D
            ds = dob @ vals.T
            ds -= D[:, None]
            ds *= p
            dq[b] = tau * (ds @ keys)
            dk_r[:last + 1, g, :] += tau * (ds[:, P:].T @ qb)
            dv_r[:last + 1, g, :] += p[:, P:].T @ dob
    return {"o": o, "lse": lse, "D": Dv, "dq": dq, "dk_r": dk_r, "dv_r": dv_r}


def prompt_grads_given_stats(q, k_p, v_p, d_o, o, lse, tau: float, keys: Sequence[int]):
    """dk_p, dv_p [n][Hkv][d] of the given prompt positions (the term the response-only
    contract drops; full-sequence differential mode), from the rows' global output O and
    natural-log lse instead of recomputing them over the whole prompt.  q, d_o, o, lse are
    those of every row that sees the prompt (any number of responses stacked along the
    row axis: every row sees every prompt position).  Per row i, head h, key j:
      p_ij = exp(tau q.k_j - lse_i),  D_i = d_o_i . O_i,  ds_ij = p_ij (d_o_i . v_j - D_i),
      dk_p[j] = tau sum_{i,h} ds_ij q_ih,  dv_p[j] = sum_{i,h} p_ij d_o_ih
    over the query heads h of key j's KV head.  With exact O and lse this is the dk_p,
    dv_p of attend_bwd(full_sequence=True); with a device's O and lse it is exact
    conditional on them."""
    R, Hq, d_qk = q.shape
    P, Hkv, d_v = v_p.shape
    keys = np.asarray(keys, dtype=np.int64)
    dk = np.zeros((keys.size, Hkv, d_qk))
    dv = np.zeros((keys.size, Hkv, d_v))
    for h in range(Hq):
        g = kv_head(h, Hq, Hkv)
        qh, doh = q[:, h, :], d_o[:, h, :]
        D = np.sum(doh * o[:, h, :], axis=1)
        p = np.exp(tau * (qh @ k_p[keys, g, :].T) - lse[:, h][:, None])   # [R][n]
        ds = p * (doh @ v_p[keys, g, :].T - D[:, None])
        dk[:, g, :] += tau * (ds.T @ qh)
        dv[:, g, :] += p.T @ doh
    return dk, dv


def chunk_bounds(P: int, chunk: int) -> List[tuple]:
    """Contiguous prompt chunks [c*chunk, min((c+1)*chunk, P)); the last may be partial."""
    return [(a, min(a + chunk, P)) for a in range(0, P, chunk)]


def _partial(s: np.ndarray, vals: np.ndarray):
    """Softmax statistics of one key subset: (O_c normalised, lse_c); an empty subset
    (all entries -inf) gives O_c = 0 and lse_c = -inf."""
    m = s.max(axis=1)
    o = np.zeros((s.shape[0], vals.shape[1]))
    lse = np.full(s.shape[0], -np.inf)
    live = np.isfinite(m)
    if np.any(live):
        e = np.exp(s[live] - m[live, None])
        den = e.sum(axis=1)
        o[live] = (e @ vals) / den[:, None]
        lse[live] = m[live] + np.log(den)
    return o, lse


def chunk_partials(q, k_p, v_p, k_r, v_r, tau: float, bounds: Sequence[tuple],
                   rows: Optional[Sequence[int]] = None):
    """Per-part softmax statistics: one part per prompt chunk in `bounds`, then one part
    for the response's own causal keys.  Returns (parts_o [n+1][rows][Hq][d_v],
    parts_lse [n+1][rows][Hq]).  This is the rank-local / chunk-local half of the
    composition; `merge` is the other half."""
    R, Hq, _ = q.shape
    P, Hkv, d_v = v_p.shape
    rows = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    n = len(bounds)
    po = np.zeros((n + 1, rows.size, Hq, d_v))
    pl = np.zeros((n + 1, rows.size, Hq))
    for h in range(Hq):
        g = kv_head(h, Hq, Hkv)
        qh = q[rows, h, :]
        for c, (a, b) in enumerate(bounds):
            s = tau * (qh @ k_p[a:b, g, :].T)
            po[c, :, h, :], pl[c, :, h] = _partial(s, v_p[a:b, g, :])
        s = tau * (qh @ k_r[:, g, :].T)
        s[np.arange(R)[None, :] > rows[:, None]] = -np.inf
        po[n, :, h, :], pl[n, :, h] = _partial(s, v_r[:, g, :])
    return po, pl


def merge(parts_o: np.ndarray, parts_lse: np.ndarray):
    """Exact composition of softmax-statistics partials (axis 0 indexes the parts):
    lse = log sum_c exp(lse_c),  O = sum_c exp(lse_c - lse) O_c.
    A part with lse_c = -inf has weight 0; rows where every part is empty give O = 0 and
    lse = -inf."""
    m = parts_lse.max(axis=0)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(parts_lse - safe_m[None])
    den = w.sum(axis=0)
    live = den > 0
    lse = np.where(live, safe_m + np.log(np.where(live, den, 1.0)), -np.inf)
    wn = w / np.where(live, den, 1.0)[None]
    o = np.einsum("c...,c...d->...d", wn, parts_o)
    return o, lse


def accumulate(grads: Sequence[np.ndarray], rows_max: int) -> np.ndarray:
    """Update-boundary accumulation of serially replayed members: the sum over members of
    each member's gradient, zero-padded along axis 0 to rows_max positions."""
    acc = np.zeros((rows_max,) + tuple(grads[0].shape[1:]))
    for gr in grads:
        acc[:gr.shape[0]] += gr
    return acc
