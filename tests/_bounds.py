"""Element-wise error bounds of the bf16 backward, from its rounding model.

Used where scores are large enough that the benchmark spec's tolerances (relative to the
gradient's own size) cannot hold: when every row's scores carry a large common ramp,
dQ = tau sum_j dS_ij k_j relies on sum_j dS_ij = 0 to cancel the ramp, and rounding
each dS_ij to bf16 leaves the cancellation incomplete.  The bound states how far the
GPU may then be from the exact (fp64 oracle) gradient, element by element.

Rounding model of the bf16 path (one row i, head h, visible key j), with u16 = 2^-9 the
unit roundoff of bf16 and g = 128 * 2^-24 / (1 - 128 * 2^-24) the fp32 dot-product bound
for 128-term products:
  * forward: P rounded to bf16 before P V, the normaliser summing the same rounded
    values, so O is a weighted mean of the v_j with weights off by at most u16 each:
      |err O_e| <= u16 / (1 - u16) * sum_j p_j |v_je - O_e|, and lse is off by at most u16;
  * D = dO . O inherits |err D| <= sum_e |dO_e| |err O_e| + g sum_e |dO_e O_e|;
  * backward: s_j is recomputed in fp32 (off by tau * g * sum_e |q_e k_je|), p_j =
    exp(s_j - lse) inherits that and the lse error, and dS_j = p_j (dP_j - D) is rounded
    to bf16 before the dQ and dK products (u16), so
      |err dS_j| <= eta_j |dS_j| + p_j |err D|,  eta_j = 2 u16 + 2 tau g sum_e |q_e k_je|
    (the factor 2 covers the products of small terms and the fp32 dP);
  * dQ = tau sum_j dS_j k_j, dK_r[j] = tau sum_{i,h} dS q, dV_r[j] = sum_{i,h} p dO, each
    accumulated in fp32 (a further u16 |result| covers the accumulation and the final
    rounding with a wide margin);
  * terms below fp32's range (p < 2^-126, as for response keys behind a steep prompt
    ramp) are lost: an absolute 1e-30 covers a few thousand of them.
So
  B_dQ[i,h,:]  = tau (sum_j eta_j |dS_j| |k_j| + |err D| sum_j p_j |k_j|) + u16 |dQ|
  B_dK_r[j,g,:] = tau sum_{i>=j, h in g} (eta |dS| + p |err D|) |q_ih| + u16 |dK_r|
  B_dV_r[j,g,:] = sum_{i>=j, h in g} eta p |dO_ih| + u16 |dV_r|
each plus 1e-30, computed in fp64 from the exact values.  Test helper only (no kernel arithmetic).
"""
import numpy as np

U16 = 2.0 ** -9
G128 = 128 * 2.0 ** -24 / (1 - 128 * 2.0 ** -24)
UNDERFLOW = 1e-30


def bwd_bounds(q, k_p, v_p, k_r, v_r, d_o, tau, dq, dk_r, dv_r):
    """Bounds [R][Hq][d], [R][Hkv][d], [R][Hkv][d] for one response (fp64 inputs and the
    oracle's exact gradients dq, dk_r, dv_r)."""
    R, Hq, d = q.shape
    P, Hkv, _ = k_p.shape
    grp = Hq // Hkv
    b_dq = np.zeros_like(dq)
    b_dk = np.zeros_like(dk_r)
    b_dv = np.zeros_like(dv_r)
    rows = np.arange(R)
    for g in range(Hkv):
        keys = np.concatenate([k_p[:, g], k_r[:, g]])
        vals = np.concatenate([v_p[:, g], v_r[:, g]])
        vis = np.ones((R, P + R), dtype=bool)
        vis[:, P:] = rows[None, :] <= rows[:, None]
        ak, av = np.abs(keys), np.abs(vals)
        for h in range(g * grp, (g + 1) * grp):
            s = tau * (q[:, h] @ keys.T)
            s[~vis] = -np.inf
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            p = e / e.sum(axis=1, keepdims=True)
            o = p @ vals
            dp = d_o[:, h] @ vals.T
            D = np.sum(d_o[:, h] * o, axis=1)
            ds = p * (dp - D[:, None])
            eta = 2 * U16 + 2 * tau * G128 * (np.abs(q[:, h]) @ ak.T)
            # |err O| of the forward, row by row: u16 / (1 - u16) sum_j p_j |v_j - O|
            spread = np.stack([p[i] @ np.abs(vals - o[i]) for i in range(R)])
            dD = U16 / (1 - U16) * np.sum(np.abs(d_o[:, h]) * spread, axis=1) + G128 * np.sum(
                np.abs(d_o[:, h]) * np.abs(o), axis=1)
            w = eta * np.abs(ds) + p * dD[:, None]
            b_dq[:, h] = tau * (w @ ak)
            b_dk[:, g] += tau * (w[:, P:].T @ np.abs(q[:, h]))
            b_dv[:, g] += (eta * p)[:, P:].T @ np.abs(d_o[:, h])
    b_dq += U16 * np.abs(dq) + UNDERFLOW
    b_dk += U16 * np.abs(dk_r) + UNDERFLOW
    b_dv += U16 * np.abs(dv_r) + UNDERFLOW
    return b_dq, b_dk, b_dv


def worst_ratio(got, ref, bound):
    """max |got - ref| / bound (the test requires <= 1)."""
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref) / bound))
