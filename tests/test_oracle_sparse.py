"""Pins of the latent-page sparse oracle (CPU only): brute-force selection, the dense
special case k >= P, and torch fp64 attention / autograd under the selection mask."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import sparse


def _inputs(seed, P, R, H, dqk, dv, di):
    g = np.random.default_rng(seed)
    return dict(q=g.standard_normal((R, H, dqk)), latent_p=g.standard_normal((P, dqk)),
                latent_r=g.standard_normal((R, dqk)), d_o=g.standard_normal((R, H, dv)),
                q_idx=g.standard_normal((R, di)), k_idx=g.standard_normal((P, di)))


def test_topk_matches_brute_force_sort():
    g = np.random.default_rng(0)
    for P, k in [(50, 7), (64, 64), (33, 1), (40, 39)]:
        s = g.standard_normal((5, P))
        sel = sparse.topk_select(s, k)
        for i in range(5):
            order = sorted(range(P), key=lambda j: (-s[i, j], j))[:k]
            assert list(sel[i]) == sorted(order)


def test_topk_ties_break_toward_lower_position():
    s = np.array([[1.0, 3.0, 2.0, 3.0, 2.0, 2.0, 0.0]])
    assert list(sparse.topk_row(s[0], 3)) == [1, 2, 3]      # 3, 3, then the first 2.0
    assert list(sparse.topk_row(s[0], 4)) == [1, 2, 3, 4]
    assert list(sparse.topk_row(np.zeros(6), 2)) == [0, 1]
    assert list(sparse.topk_row(s[0], 10)) == list(range(7))


def test_index_scores_plain_dot():
    """fp32 scores: within the dot-product error bound n u sum|q_t k_t| (u = 2^-24) of the
    exact sum, and exact for small-integer data."""
    x = _inputs(1, 9, 4, 1, 3, 2, 5)
    s = sparse.index_scores(x["q_idx"], x["k_idx"])
    assert s.dtype == np.float32
    qf = x["q_idx"].astype(np.float32).astype(np.float64)
    kf = x["k_idx"].astype(np.float32).astype(np.float64)
    for i in range(4):
        for j in range(9):
            terms = [qf[i, t] * kf[j, t] for t in range(5)]
            bound = 5 * 2.0 ** -24 * sum(abs(v) for v in terms) / (1 - 5 * 2.0 ** -24)
            assert abs(float(s[i, j]) - sum(terms)) <= bound
    g = np.random.default_rng(3)
    qi, ki = g.integers(-3, 4, (6, 128)), g.integers(-3, 4, (50, 128))
    np.testing.assert_array_equal(sparse.index_scores(qi, ki), (qi @ ki.T).astype(np.float32))


def _torch_masked(x, idx, tau, dv, grad=False):
    """Attention over [prompt latent; response latent] with a mask that keeps the selected
    prompt rows and the causal response rows; every head reads the same latent row."""
    P, R, H = x["latent_p"].shape[0], x["latent_r"].shape[0], x["q"].shape[1]
    q = torch.tensor(x["q"]).permute(1, 0, 2)[None]
    lr = torch.tensor(x["latent_r"])
    if grad:
        q.requires_grad_(True)
        lr.requires_grad_(True)
    kv = torch.cat([torch.tensor(x["latent_p"]), lr], 0)
    mask = torch.zeros(R, P + R, dtype=torch.bool)
    for i in range(R):
        mask[i, torch.tensor(idx[i])] = True
    mask[:, P:] = torch.tril(torch.ones(R, R, dtype=torch.bool))
    k = kv[None, None].expand(1, H, P + R, kv.shape[1])
    v = kv[:, :dv][None, None].expand(1, H, P + R, dv)
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=tau)
    return o[0].permute(1, 0, 2), q, lr


@pytest.mark.parametrize("P,k", [(30, 8), (16, 16), (12, 40)])
def test_sparse_attention_matches_masked_library_attention(P, k):
    x = _inputs(2, P, 7, 3, 12, 8, 4)
    tau = 0.3
    idx = sparse.topk_select(sparse.index_scores(x["q_idx"], x["k_idx"]), k)
    o, lse = sparse.sparse_attend(x["q"], x["latent_p"], x["latent_r"], idx, tau, 8)
    o_ref, q, lr = _torch_masked(x, idx, tau, 8, grad=True)
    np.testing.assert_allclose(o, o_ref.detach().numpy(), atol=1e-12, rtol=0)
    (o_ref * torch.tensor(x["d_o"])).sum().backward()
    g = sparse.sparse_attend_bwd(x["q"], x["latent_p"], x["latent_r"], idx, x["d_o"], tau, 8)
    np.testing.assert_allclose(g["dq"], q.grad[0].permute(1, 0, 2).numpy(), atol=1e-10, rtol=0)
    # the response latent row's gradient = key part + value part (first d_v dims)
    dlat = g["dk_r"].copy()
    dlat[:, :8] += g["dv_r"]
    np.testing.assert_allclose(dlat, lr.grad.numpy(), atol=1e-10, rtol=0)
    # lse closed form: with all-zero queries every visible row has weight 1 / n_visible
    z = dict(x)
    z["q"] = np.zeros_like(x["q"])
    _, lz = sparse.sparse_attend(z["q"], x["latent_p"], x["latent_r"], idx, tau, 8)
    for i in range(7):
        np.testing.assert_allclose(lz[i], np.log(idx.shape[1] + i + 1), atol=1e-13)


def test_sparse_backward_finite_differences():
    x = _inputs(3, 10, 4, 2, 5, 3, 2)
    tau = 0.5
    idx = sparse.topk_select(sparse.index_scores(x["q_idx"], x["k_idx"]), 4)
    g = sparse.sparse_attend_bwd(x["q"], x["latent_p"], x["latent_r"], idx, x["d_o"], tau, 3)

    def loss(q, lat_r):
        o, _ = sparse.sparse_attend(q, x["latent_p"], lat_r, idx, tau, 3)
        return float(np.sum(o * x["d_o"]))

    h = 1e-6
    fdq = np.zeros_like(x["q"])
    for ix in np.ndindex(*x["q"].shape):
        a, b = x["q"].copy(), x["q"].copy()
        a[ix] += h
        b[ix] -= h
        fdq[ix] = (loss(a, x["latent_r"]) - loss(b, x["latent_r"])) / (2 * h)
    np.testing.assert_allclose(g["dq"], fdq, atol=1e-6)
    fdl = np.zeros_like(x["latent_r"])
    for ix in np.ndindex(*x["latent_r"].shape):
        a, b = x["latent_r"].copy(), x["latent_r"].copy()
        a[ix] += h
        b[ix] -= h
        fdl[ix] = (loss(x["q"], a) - loss(x["q"], b)) / (2 * h)
    dlat = g["dk_r"].copy()
    dlat[:, :3] += g["dv_r"]
    np.testing.assert_allclose(dlat, fdl, atol=1e-6)
