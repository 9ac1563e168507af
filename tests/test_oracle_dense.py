"""Pins of the dense oracle against things other than itself (CPU only).

* library special case: response rows of ordinary causal attention over the
  concatenated [prompt; response] sequence (torch CPU fp64 scaled_dot_product_attention,
  GQA by repeat_interleave), and torch fp64 autograd with the prompt K/V not requiring
  grad (the stop-gradient);
* lse through a probe key the library routine cannot distinguish from data;
* central finite differences on tiny inputs;
* closed forms (zero queries, constant values, equal keys);
* hand-derived fixture under tests/golden/.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import dense
from tests._helpers import load_golden, rand_problem


def _sdpa(x, tau, full_grad=False, extra_probe=False):
    """Response rows of causal attention over [prompt; response] via torch's routine."""
    q = torch.tensor(x["q"]).permute(1, 0, 2)[None]             # [1][Hq][R][d]
    kp, vp = torch.tensor(x["k_p"]), torch.tensor(x["v_p"])
    kr, vr = torch.tensor(x["k_r"]), torch.tensor(x["v_r"])
    if full_grad:
        kp.requires_grad_(True)
        vp.requires_grad_(True)
    q.requires_grad_(True)
    kr.requires_grad_(True)
    vr.requires_grad_(True)
    P, R, Hq, Hkv = kp.shape[0], kr.shape[0], q.shape[1], kp.shape[1]
    k = torch.cat([kp, kr], 0).permute(1, 0, 2)                  # [Hkv][P+R][d]
    v = torch.cat([vp, vr], 0).permute(1, 0, 2)
    mask = torch.ones(R, P + R, dtype=torch.bool)
    mask[:, P:] = torch.tril(torch.ones(R, R, dtype=torch.bool))
    if extra_probe:   # a zero key (score 0 for every row) carrying a one-hot extra value dim
        k = torch.cat([k, torch.zeros(Hkv, 1, k.shape[-1], dtype=k.dtype)], 1)
        v = torch.cat([v, torch.zeros(Hkv, v.shape[1], 1, dtype=v.dtype)], 2)
        probe_v = torch.zeros(Hkv, 1, v.shape[-1], dtype=v.dtype)
        probe_v[..., -1] = 1.0
        v = torch.cat([v, probe_v], 1)
        mask = torch.cat([mask, torch.ones(R, 1, dtype=torch.bool)], 1)
    grp = Hq // Hkv
    k = k.repeat_interleave(grp, 0)[None]
    v = v.repeat_interleave(grp, 0)[None]
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=tau)
    return o[0].permute(1, 0, 2), (q, kp, vp, kr, vr)


@pytest.mark.parametrize("P,R,Hq,Hkv,d", [(37, 11, 4, 2, 8), (64, 16, 6, 1, 16), (5, 9, 2, 2, 4)])
def test_output_matches_library_causal_attention(P, R, Hq, Hkv, d):
    x = rand_problem(1, P, R, Hq, Hkv, d)
    tau = 0.37
    o_ref, _ = _sdpa(x, tau)
    o, lse = dense.attend(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], tau)
    np.testing.assert_allclose(o, o_ref.detach().numpy(), rtol=0, atol=1e-12)
    # lse via a probe key with score 0 and a one-hot value: probe weight = 1 / (1 + e^lse)
    o_probe, _ = _sdpa(x, tau, extra_probe=True)
    w = o_probe.detach().numpy()[..., -1]
    np.testing.assert_allclose(lse, np.log(1.0 / w - 1.0), rtol=0, atol=1e-10)


@pytest.mark.parametrize("P,R,Hq,Hkv,d", [(37, 11, 4, 2, 8), (20, 13, 3, 1, 5)])
def test_backward_matches_library_autograd(P, R, Hq, Hkv, d):
    x = rand_problem(2, P, R, Hq, Hkv, d)
    tau = 0.41
    o_ref, (q, kp, vp, kr, vr) = _sdpa(x, tau)
    (o_ref * torch.tensor(x["d_o"])).sum().backward()
    g = dense.attend_bwd(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], x["d_o"], tau)
    np.testing.assert_allclose(g["dq"], q.grad[0].permute(1, 0, 2).numpy(), atol=1e-10, rtol=0)
    np.testing.assert_allclose(g["dk_r"], kr.grad.numpy(), atol=1e-10, rtol=0)
    np.testing.assert_allclose(g["dv_r"], vr.grad.numpy(), atol=1e-10, rtol=0)
    assert kp.grad is None and vp.grad is None      # stop-gradient resident state


def test_full_sequence_mode_differs_only_by_prompt_grads():
    x = rand_problem(3, 29, 10, 4, 2, 6)
    tau = 0.5
    o_ref, (q, kp, vp, kr, vr) = _sdpa(x, tau, full_grad=True)
    (o_ref * torch.tensor(x["d_o"])).sum().backward()
    full = dense.attend_bwd(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], x["d_o"], tau,
                            full_sequence=True)
    ronly = dense.attend_bwd(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], x["d_o"], tau)
    np.testing.assert_allclose(full["dk_p"], kp.grad.numpy(), atol=1e-10, rtol=0)
    np.testing.assert_allclose(full["dv_p"], vp.grad.numpy(), atol=1e-10, rtol=0)
    for key in ("dq", "dk_r", "dv_r"):
        np.testing.assert_array_equal(full[key], ronly[key])
    assert np.abs(full["dk_p"]).max() > 1e-3          # the dropped term is not trivially zero


def test_prompt_grads_given_stats_equal_full_sequence_mode():
    # two responses sharing the prompt: the conditional form over the stacked rows of both,
    # fed the exact O and lse, equals the sum of the two full-sequence prompt gradients
    x = rand_problem(31, 23, 9, 4, 2, 6)
    y = rand_problem(32, 23, 5, 4, 2, 6)
    y["k_p"], y["v_p"] = x["k_p"], x["v_p"]
    tau = 0.45
    rows_q, rows_do, rows_o, rows_lse = [], [], [], []
    ref_k = np.zeros_like(x["k_p"])
    ref_v = np.zeros_like(x["v_p"])
    for z in (x, y):
        o, lse = dense.attend(z["q"], z["k_p"], z["v_p"], z["k_r"], z["v_r"], tau)
        g = dense.attend_bwd(z["q"], z["k_p"], z["v_p"], z["k_r"], z["v_r"], z["d_o"], tau,
                             full_sequence=True)
        ref_k += g["dk_p"]
        ref_v += g["dv_p"]
        rows_q.append(z["q"]); rows_do.append(z["d_o"]); rows_o.append(o); rows_lse.append(lse)
    keys = np.array([0, 7, 22])
    dk, dv = dense.prompt_grads_given_stats(np.concatenate(rows_q), x["k_p"], x["v_p"],
                                            np.concatenate(rows_do), np.concatenate(rows_o),
                                            np.concatenate(rows_lse), tau, keys)
    np.testing.assert_allclose(dk, ref_k[keys], atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv, ref_v[keys], atol=1e-12, rtol=0)


def _loss(x, tau):
    o, _ = dense.attend(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], tau)
    return float(np.sum(o * x["d_o"]))


def test_backward_matches_finite_differences():
    x = rand_problem(4, 24, 8, 2, 1, 4)
    tau = 0.6
    g = dense.attend_bwd(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], x["d_o"], tau)
    h = 1e-6
    for name, grad in (("q", g["dq"]), ("k_r", g["dk_r"]), ("v_r", g["dv_r"])):
        fd = np.zeros_like(x[name])
        for idx in np.ndindex(*x[name].shape):
            xp = {k: v.copy() for k, v in x.items()}
            xm = {k: v.copy() for k, v in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            fd[idx] = (_loss(xp, tau) - _loss(xm, tau)) / (2 * h)
        err = np.abs(fd - grad)
        assert np.all(err <= 1e-6 * np.maximum(1.0, np.abs(grad))), (name, err.max())


def test_probabilities_sum_to_one_and_respect_causality():
    x = rand_problem(5, 17, 9, 2, 1, 8)
    o, lse, p = dense.attend(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], 0.3,
                             return_probs=True)
    np.testing.assert_allclose(p.sum(axis=2), 1.0, atol=1e-12)
    P, R = 17, 9
    for i in range(R):
        assert np.all(p[i, :, P + i + 1:] == 0.0)      # later response keys are invisible
        assert np.all(p[i, :, :P + i + 1] > 0.0)       # every prompt key and 0..i are visible


def test_closed_form_zero_queries():
    x = rand_problem(6, 13, 7, 4, 2, 8)
    x["q"][:] = 0.0
    o, lse = dense.attend(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], 0.9)
    P, R = 13, 7
    for i in range(R):
        np.testing.assert_allclose(lse[i], np.log(P + i + 1), atol=1e-13)
        for h in range(4):
            g = dense.kv_head(h, 4, 2)
            vis = np.concatenate([x["v_p"][:, g], x["v_r"][:i + 1, g]])
            np.testing.assert_allclose(o[i, h], vis.mean(axis=0), atol=1e-13)


def test_closed_form_constant_values_and_equal_keys():
    x = rand_problem(7, 11, 6, 2, 1, 5)
    c = np.array([0.5, -1.0, 2.0, 0.0, 3.0])
    x["v_p"][:] = c
    x["v_r"][:] = c
    o, _ = dense.attend(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], 0.7)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-13)
    g = dense.attend_bwd(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], x["d_o"], 0.7)
    assert np.abs(g["dq"]).max() < 1e-12 and np.abs(g["dk_r"]).max() < 1e-12
    # dv_r[j] = sum_{i >= j} p_ij d_o_i stays nonzero
    assert np.abs(g["dv_r"]).max() > 1e-3
    y = rand_problem(8, 11, 6, 2, 1, 5)
    y["k_p"][:] = y["k_p"][0]
    y["k_r"][:] = y["k_p"][0]
    g = dense.attend_bwd(y["q"], y["k_p"], y["v_p"], y["k_r"], y["v_r"], y["d_o"], 0.7)
    assert np.abs(g["dq"]).max() < 1e-12                # sum_j ds_ij = 0 and all k_j equal


def test_golden_two_key_example():
    gd = load_golden("two_key_closed_form.json")
    a = {k: np.array(gd[k], dtype=np.float64) for k in ("q", "k_p", "v_p", "k_r", "v_r", "d_o")}
    o, lse = dense.attend(a["q"], a["k_p"], a["v_p"], a["k_r"], a["v_r"], gd["tau"])
    g = dense.attend_bwd(a["q"], a["k_p"], a["v_p"], a["k_r"], a["v_r"], a["d_o"], gd["tau"],
                         full_sequence=True)
    e = gd["expect"]
    np.testing.assert_allclose(o, e["o"], atol=1e-14)
    np.testing.assert_allclose(lse, e["lse"], atol=1e-14)
    for key in ("dq", "dk_r", "dv_r", "dk_p", "dv_p"):
        np.testing.assert_allclose(g[key], e[key], atol=1e-14, err_msg=key)


def test_row_subsets_equal_full_rows():
    x = rand_problem(9, 30, 12, 4, 2, 8)
    rows = np.array([0, 5, 11])
    o, lse = dense.attend(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], 0.3)
    os_, ls = dense.attend(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], 0.3, rows=rows)
    np.testing.assert_allclose(os_, o[rows], atol=1e-14)
    np.testing.assert_allclose(ls, lse[rows], atol=1e-14)
    full = dense.attend_bwd(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], x["d_o"], 0.3)
    # rows j0..R-1 are exactly the rows that reach response keys >= j0
    tail = np.arange(7, 12)
    part = dense.attend_bwd(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], x["d_o"], 0.3,
                            rows=tail)
    np.testing.assert_allclose(part["dq"], full["dq"][tail], atol=1e-13)
    np.testing.assert_allclose(part["dk_r"][7:], full["dk_r"][7:], atol=1e-13)
    np.testing.assert_allclose(part["dv_r"][7:], full["dv_r"][7:], atol=1e-13)


def test_attend_rows_matches_library_autograd():
    """Individual (row, head) query rows: O, lse (through the probe key), dQ against torch's
    routine and its autograd; with every head of rows 9..R-1 included, the response keys
    from 9 on get their full gradients."""
    P, R, Hq, Hkv, d = 31, 14, 6, 2, 8
    x = rand_problem(12, P, R, Hq, Hkv, d)
    tau = 0.43
    o_ref, (q, kp, vp, kr, vr) = _sdpa(x, tau)
    (o_ref * torch.tensor(x["d_o"])).sum().backward()
    o_probe, _ = _sdpa(x, tau, extra_probe=True)
    g = np.random.default_rng(5)
    rows = np.concatenate([g.integers(0, 9, 10), np.repeat(np.arange(9, R), Hq)])
    heads = np.concatenate([g.integers(0, Hq, 10), np.tile(np.arange(Hq), R - 9)])
    out = dense.attend_rows(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], x["d_o"], tau, rows, heads)
    np.testing.assert_allclose(out["o"], o_ref.detach().numpy()[rows, heads], rtol=0, atol=1e-12)
    w = o_probe.detach().numpy()[rows, heads, -1]
    np.testing.assert_allclose(out["lse"], np.log(1.0 / w - 1.0), rtol=0, atol=1e-10)
    D = np.sum(o_ref.detach().numpy()[rows, heads] * x["d_o"][rows, heads], axis=1)
    np.testing.assert_allclose(out["D"], D, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["dq"], q.grad[0].permute(1, 0, 2).numpy()[rows, heads], atol=1e-10, rtol=0)
    np.testing.assert_allclose(out["dk_r"][9:], kr.grad.numpy()[9:], atol=1e-10, rtol=0)
    np.testing.assert_allclose(out["dv_r"][9:], vr.grad.numpy()[9:], atol=1e-10, rtol=0)
