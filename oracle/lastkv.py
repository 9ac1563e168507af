"""LastKV chunk recurrence with previous-chunk blending, fp64.  TEST INFRASTRUCTURE ONLY.

Source: zefan-cai.github.io/en/blog/lastkv-rl ("In RL, Does the Trainer Evaluate the
Policy That Generated the Rollout?"), section "LastKV: making recurrence boundaries part
of the policy".  For one layer l and a sequence cut into chunks of C positions:

  * chunk c attends to the last-layer K/V (K^L, V^L) of the completed chunks before it and
    to its own per-layer K/V (K^l, V^l) with a causal mask;
  * with previous-chunk blending, the most recent completed chunk c-1 enters as
        K~ = (1 - alpha_g) K^l_{c-1} + alpha_g K^L_{c-1}   (and V~ likewise),
    one gate alpha_g per KV head of this layer; chunks before c-1 enter as K^L alone.

So position t of chunk c = t // C reads, in order: K^L of positions [0, (c-1) C), K~ of
positions [(c-1) C, c C), K^l of positions [c C, t].  For c = 0 only the last part exists,
for c = 1 the first part is empty.  The end of a sequence need not be a chunk boundary:
the last chunk may hold fewer than C positions.

`sequence_attend` is that definition written out position by position.  `chunk_attend_bwd`
is the backward of one chunk with the history fixed as inputs; it takes the attention
gradients from dense.attend_bwd (keys [history; blended chunk] as the stop-gradient
prompt of the full-sequence mode, the chunk's own K/V as the causal part) and applies the
chain rule of the blend.  Shapes: per position [N][H][d] arrays; alpha [Hkv].
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from . import dense


def blend(x_layer: np.ndarray, x_last: np.ndarray, alpha: np.ndarray) -> np.ndarray:
    """(1 - alpha_g) x_layer + alpha_g x_last over [rows][Hkv][d]."""
    a = np.asarray(alpha, dtype=np.float64)[None, :, None]
    return (1.0 - a) * x_layer + a * x_last


def chunk_keys(k_layer, v_layer, k_last, v_last, alpha, C: int, c: int):
    """History keys/values of chunk c (the part every row of the chunk sees):
    [K^L of chunks < c-1; K~ of chunk c-1]."""
    lo = max(c - 1, 0) * C
    hk, hv = k_last[:lo], v_last[:lo]
    if c >= 1:
        bk = blend(k_layer[lo:c * C], k_last[lo:c * C], alpha)
        bv = blend(v_layer[lo:c * C], v_last[lo:c * C], alpha)
        hk = np.concatenate([hk, bk], 0)
        hv = np.concatenate([hv, bv], 0)
    return hk, hv


def sequence_attend(q, k_layer, v_layer, k_last, v_last, alpha, C: int, tau: float):
    """O [N][Hq][d_v] and natural-log lse [N][Hq] of every position of the sequence."""
    N, Hq, _ = q.shape
    Hkv = k_layer.shape[1]
    grp = Hq // Hkv
    o = np.zeros((N, Hq, v_layer.shape[2]))
    lse = np.zeros((N, Hq))
    for t in range(N):
        c = t // C
        hk, hv = chunk_keys(k_layer, v_layer, k_last, v_last, alpha, C, c)
        keys = np.concatenate([hk, k_layer[c * C:t + 1]], 0)
        vals = np.concatenate([hv, v_layer[c * C:t + 1]], 0)
        for h in range(Hq):
            g = h // grp
            s = tau * (keys[:, g, :] @ q[t, h, :])
            m = s.max()
            e = np.exp(s - m)
            o[t, h] = (e @ vals[:, g, :]) / e.sum()
            lse[t, h] = m + np.log(e.sum())
    return o, lse


def chunk_attend_bwd(q_c, d_o_c, k_layer, v_layer, k_last, v_last, alpha, C: int, c: int,
                     tau: float) -> Dict[str, np.ndarray]:
    """Backward of chunk c of L = sum d_o . O over the chunk's rows q_c [n][Hq][d]
    (positions c C .. c C + n - 1).  Returns dq [n], dk_c / dv_c [n] (the chunk's own
    per-layer K/V), dk_prev_layer / dv_prev_layer and dk_prev_last / dv_prev_last [C]
    (chunk c-1's two sources of the blend; zero-size for c = 0), d_alpha [Hkv], and
    dk_hist / dv_hist [(c-1) C] (the older last-layer history)."""
    n = q_c.shape[0]
    lo, hi = max(c - 1, 0) * C, c * C
    hk, hv = chunk_keys(k_layer, v_layer, k_last, v_last, alpha, C, c)
    g = dense.attend_bwd(q_c, hk, hv, k_layer[hi:hi + n], v_layer[hi:hi + n], d_o_c, tau,
                         full_sequence=True)
    out = {"dq": g["dq"], "dk_c": g["dk_r"], "dv_c": g["dv_r"],
           "dk_hist": g["dk_p"][:lo], "dv_hist": g["dv_p"][:lo]}
    dkb, dvb = g["dk_p"][lo:], g["dv_p"][lo:]        # gradients of K~, V~
    a = np.asarray(alpha, dtype=np.float64)[None, :, None]
    out["dk_prev_layer"] = (1.0 - a) * dkb
    out["dv_prev_layer"] = (1.0 - a) * dvb
    out["dk_prev_last"] = a * dkb
    out["dv_prev_last"] = a * dvb
    if c >= 1:
        dk_src = k_last[lo:hi] - k_layer[lo:hi]
        dv_src = v_last[lo:hi] - v_layer[lo:hi]
        out["d_alpha"] = np.sum(dk_src * dkb, axis=(0, 2)) + np.sum(dv_src * dvb, axis=(0, 2))
    else:
        out["d_alpha"] = np.zeros(k_layer.shape[1])
    return out
