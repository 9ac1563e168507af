"""Pins of the LastKV oracle against things other than itself (CPU only).

* library routine: torch CPU fp64 scaled_dot_product_attention over one key set holding
  every position three times (last-layer, blended, per-layer K/V) with a mask that picks,
  per row, the copy LastKV reads; its autograd gives the backward, the gate included;
* special cases: when every layer's K/V equals the last layer's (a one-layer model) the
  recurrence is ordinary causal attention, for any gate and chunk size; gate 1 is the
  rule without blending, gate 0 reads the whole previous chunk per-layer;
* central finite differences of the gate;
* sequence lengths C - 1, C, C + 1 and a ragged last chunk (the end of a sequence is not a
  chunk boundary).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import lastkv


def _inputs(seed, N, Hq, Hkv, d):
    g = np.random.default_rng(seed)
    f = lambda *s: g.standard_normal(s)
    return dict(q=f(N, Hq, d), k_layer=f(N, Hkv, d), v_layer=f(N, Hkv, d), k_last=f(N, Hkv, d),
                v_last=f(N, Hkv, d), d_o=f(N, Hq, d), alpha=g.uniform(0.05, 0.95, Hkv))


def _mask(N, C):
    """[N][3N]: row t reads K^L of positions < (c-1)C, the blended copy of chunk c-1 and the
    per-layer copy of positions c C .. t (c = t // C)."""
    m = np.zeros((N, 3 * N), dtype=bool)
    for t in range(N):
        c = t // C
        lo = max(c - 1, 0) * C
        m[t, :lo] = True
        if c >= 1:
            m[t, N + lo:N + c * C] = True
        m[t, 2 * N + c * C:2 * N + t + 1] = True
    return torch.tensor(m)


def _torch_lastkv(x, C, tau, rows=None):
    """Reference through torch's attention routine; returns O and the leaf tensors."""
    t = {k: torch.tensor(v, requires_grad=True) for k, v in x.items() if k != "d_o"}
    N, Hq, d = x["q"].shape
    Hkv = x["k_layer"].shape[1]
    a = t["alpha"][None, :, None]
    kb = (1 - a) * t["k_layer"] + a * t["k_last"]
    vb = (1 - a) * t["v_layer"] + a * t["v_last"]
    k = torch.cat([t["k_last"], kb, t["k_layer"]], 0).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    v = torch.cat([t["v_last"], vb, t["v_layer"]], 0).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    q = t["q"].permute(1, 0, 2)
    o = F.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=_mask(N, C), scale=tau)
    return o[0].permute(1, 0, 2), t


@pytest.mark.parametrize("N,C", [(7, 8), (8, 8), (9, 8), (29, 8), (24, 8), (20, 5)])
def test_sequence_matches_library_masked_attention(N, C):
    x = _inputs(N * 100 + C, N, 4, 2, 6)
    tau = 0.4
    o_ref, _ = _torch_lastkv(x, C, tau)
    o, _ = lastkv.sequence_attend(x["q"], x["k_layer"], x["v_layer"], x["k_last"], x["v_last"], x["alpha"],
                                  C, tau)
    np.testing.assert_allclose(o, o_ref.detach().numpy(), atol=1e-12, rtol=0)


@pytest.mark.parametrize("C", [1, 3, 8, 100])
def test_one_layer_model_is_ordinary_causal_attention(C):
    x = _inputs(5 + C, 23, 4, 1, 5)
    x["k_layer"], x["v_layer"] = x["k_last"], x["v_last"]
    tau = 0.5
    q = torch.tensor(x["q"]).permute(1, 0, 2)[None]
    k = torch.tensor(x["k_last"]).permute(1, 0, 2).repeat_interleave(4, 0)[None]
    v = torch.tensor(x["v_last"]).permute(1, 0, 2).repeat_interleave(4, 0)[None]
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=tau)[0].permute(1, 0, 2).numpy()
    o, _ = lastkv.sequence_attend(x["q"], x["k_layer"], x["v_layer"], x["k_last"], x["v_last"], x["alpha"],
                                  C, tau)
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("gate", [0.0, 1.0])
def test_gate_zero_and_one(gate):
    """Gate 1: chunk c reads K^L of all completed chunks (the rule without blending).
    Gate 0: the previous chunk is read with its per-layer K/V."""
    N, C, tau = 21, 6, 0.45
    x = _inputs(77, N, 2, 2, 4)
    x["alpha"] = np.full(2, gate)
    o, _ = lastkv.sequence_attend(x["q"], x["k_layer"], x["v_layer"], x["k_last"], x["v_last"], x["alpha"],
                                  C, tau)
    for t in range(N):
        c = t // C
        cut = c * C if gate == 1.0 else max(c - 1, 0) * C
        keys = np.concatenate([x["k_last"][:cut], x["k_layer"][cut:t + 1]], 0)
        vals = np.concatenate([x["v_last"][:cut], x["v_layer"][cut:t + 1]], 0)
        for h in range(2):
            s = tau * keys[:, h, :] @ x["q"][t, h]
            p = np.exp(s - s.max())
            np.testing.assert_allclose(o[t, h], p @ vals[:, h, :] / p.sum(), atol=1e-12, rtol=0)


@pytest.mark.parametrize("N,C,c", [(20, 8, 2), (17, 8, 2), (16, 8, 1), (8, 8, 0), (30, 7, 3)])
def test_chunk_backward_matches_library_autograd(N, C, c):
    x = _inputs(N + 10 * c, N, 4, 2, 5)
    tau = 0.35
    o_ref, t = _torch_lastkv(x, C, tau)
    lo, hi, n = max(c - 1, 0) * C, c * C, min(N, (c + 1) * C) - c * C
    (o_ref[hi:hi + n] * torch.tensor(x["d_o"][hi:hi + n])).sum().backward()
    g = lastkv.chunk_attend_bwd(x["q"][hi:hi + n], x["d_o"][hi:hi + n], x["k_layer"], x["v_layer"],
                                x["k_last"], x["v_last"], x["alpha"], C, c, tau)
    gr = {k: v.grad.numpy() for k, v in t.items()}
    close = lambda a, b: np.testing.assert_allclose(a, b, atol=1e-11, rtol=0)
    close(g["dq"], gr["q"][hi:hi + n])
    close(g["dk_c"], gr["k_layer"][hi:hi + n])
    close(g["dv_c"], gr["v_layer"][hi:hi + n])
    close(g["dk_prev_layer"], gr["k_layer"][lo:hi])
    close(g["dv_prev_layer"], gr["v_layer"][lo:hi])
    close(g["dk_prev_last"], gr["k_last"][lo:hi])
    close(g["dv_prev_last"], gr["v_last"][lo:hi])
    close(g["dk_hist"], gr["k_last"][:lo])
    close(g["dv_hist"], gr["v_last"][:lo])
    close(g["d_alpha"], gr["alpha"])


def test_gate_gradient_matches_finite_differences():
    N, C, c, tau = 19, 6, 2, 0.5
    x = _inputs(91, N, 2, 2, 4)
    hi, n = c * C, C
    loss = lambda al: float(np.sum(lastkv.sequence_attend(x["q"], x["k_layer"], x["v_layer"], x["k_last"],
                                                          x["v_last"], al, C, tau)[0][hi:hi + n]
                                   * x["d_o"][hi:hi + n]))
    g = lastkv.chunk_attend_bwd(x["q"][hi:hi + n], x["d_o"][hi:hi + n], x["k_layer"], x["v_layer"],
                                x["k_last"], x["v_last"], x["alpha"], C, c, tau)
    h = 1e-6
    for j in range(2):
        e = np.zeros(2)
        e[j] = h
        fd = (loss(x["alpha"] + e) - loss(x["alpha"] - e)) / (2 * h)
        assert abs(fd - g["d_alpha"][j]) <= 1e-6 * max(1.0, abs(fd))
