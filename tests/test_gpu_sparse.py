"""GPU parity of the latent-page sparse variant (needs an MI355X): fp32 index scores and
exact per-query top-k (ties toward the lower position), attention over the selected latent
rows plus the response's causal rows with 64 heads sharing each 576-wide row (value = its
first 512 dims), and the response-only backward (dq, dk_r, dv_r).

Where the GPU's fp32 scores and the oracle's fp64 scores could rank two near-equal
positions differently, several selections are correct: such rows are checked for validity
(every selected score >= every unselected score - eps) and their attention values are not
compared.  With small-integer index data every score is exact in fp32, the selection is
unique, and every output element is compared."""
import numpy as np
import pytest

from oracle import sparse
from resident_kv_response_amd import configs, synth
from tests._helpers import assert_bf16_close, assert_D_close

pytestmark = pytest.mark.gpu


def _data(seed, P, R, integer_index):
    g = np.random.default_rng(seed)
    bf = lambda shape: synth.f32_to_bf16_bits(g.standard_normal(shape, dtype=np.float32))
    d = dict(latent_p=bf((P, 576)), q=bf((R, 64, 576)), latent_r=bf((R, 576)), d_o=bf((R, 64, 512)))
    if integer_index:
        d["k_idx"] = g.integers(-3, 4, size=(P, 128)).astype(np.float32)
        d["q_idx"] = g.integers(-3, 4, size=(R, 128)).astype(np.float32)
    else:
        d["k_idx"] = g.standard_normal((P, 128), dtype=np.float32)
        d["q_idx"] = g.standard_normal((R, 128), dtype=np.float32)
    return d


def _oracle(d, topk, rows=None):
    f = lambda x: synth.as_f64(x, "bf16")
    R = d["q"].shape[0]
    rows = np.arange(R) if rows is None else np.asarray(rows)
    sig = sparse.index_scores(d["q_idx"][rows], d["k_idx"])
    sel = np.zeros((R, topk), dtype=np.int64)
    sel[rows] = sparse.topk_select(sig, topk)
    tau = 1.0 / np.sqrt(576)
    o, lse = sparse.sparse_attend(f(d["q"]), f(d["latent_p"]), f(d["latent_r"]), sel, tau, 512, rows=rows)
    gr = sparse.sparse_attend_bwd(f(d["q"]), f(d["latent_p"]), f(d["latent_r"]), sel, f(d["d_o"]), tau, 512,
                                  rows=rows)
    return sel, sig, o, lse, gr


def _run(d, P, R, topk, block):
    from tests import _gpu as G
    prob = G.latent_problem(P, R, topk, block)
    run = G.LatentRun(prob, d["latent_p"], d["k_idx"], d["q"][None], d["latent_r"][None], d["q_idx"][None],
                      d["d_o"][None], [R])
    return run.fwd().bwd().numpy()


@pytest.mark.parametrize("P,R,topk,block", [(3000, 96, 256, 32), (1500, 64, 1024, 64)])
def test_sparse_exact_selection_every_element(P, R, topk, block):
    d = _data(8000 + P, P, R, integer_index=True)
    print(f"[sparse] P={P} R={R} topk={topk}", flush=True)
    got = _run(d, P, R, topk, block)
    sel, sig, o, lse, gr = _oracle(d, topk)
    np.testing.assert_array_equal(got["idx"][0], sel)      # exact, ties toward the lower position
    assert_bf16_close("o", got["o"][0], o)
    assert np.max(np.abs(got["lse"][0] - lse)) <= 2e-2
    assert_bf16_close("dq", got["dq"][0], gr["dq"])
    assert_bf16_close("dk_r", got["dk"][0], gr["dk_r"])
    assert_bf16_close("dv_r", got["dv"][0], gr["dv_r"])
    # D = dO . O of the backward's preprocess, against the oracle's O
    assert_D_close("D", got["D"][0], np.sum(synth.as_f64(d["d_o"], "bf16") * o, axis=-1), "bf16")


def test_sparse_exact_selection_large_rows_with_ties():
    """Rows long enough for the sampled-threshold path; integer index data puts hundreds of
    positions on the k-th largest score, so the tie rule decides part of every row."""
    P, R, topk = 131072, 64, 2048
    d = _data(8100, P, R, integer_index=True)
    print(f"[sparse] large rows P={P} R={R} topk={topk}", flush=True)
    got = _run(d, P, R, topk, 32)
    sel, sig, o, lse, gr = _oracle(d, topk)
    kth = np.sort(sig, axis=1)[:, -topk]
    assert np.min(np.sum(sig == kth[:, None], axis=1)) > 1      # ties at the threshold exist
    np.testing.assert_array_equal(got["idx"][0], sel)
    assert_bf16_close("o", got["o"][0], o)
    assert_bf16_close("dq", got["dq"][0], gr["dq"])
    assert_bf16_close("dk_r", got["dk"][0], gr["dk_r"])


def _structured_index(kind, P, R, seed):
    """Index data whose scores are small exact integers with a chosen structure."""
    g = np.random.default_rng(seed)
    q_idx = np.zeros((R, 128), dtype=np.float32)
    q_idx[:, 0] = 1.0
    k_idx = np.zeros((P, 128), dtype=np.float32)
    if kind == "increasing":          # score = position: the top k are the last k positions
        k_idx[:, 0] = np.arange(P, dtype=np.float32)
        q_idx[1::2, 0] = -1.0         # odd rows: decreasing, the top k are the first k
    elif kind == "constant":          # every score equal: the k lowest positions
        k_idx[:, 0] = 5.0
    elif kind == "two_levels":        # 10% of positions score 1, far more than k tied at T
        k_idx[:, 0] = (g.random(P) < 0.1).astype(np.float32)
    return q_idx, k_idx


@pytest.mark.parametrize("kind", ["increasing", "constant", "two_levels"])
def test_sparse_selection_structured_scores(kind):
    P, R, topk = 131072, 8, 2048
    d = _data(8200, P, R, integer_index=True)
    d["q_idx"], d["k_idx"] = _structured_index(kind, P, R, 8201)
    print(f"[sparse] structured scores {kind}", flush=True)
    got = _run(d, P, R, topk, 8)
    sel, sig, o, lse, gr = _oracle(d, topk)
    np.testing.assert_array_equal(got["idx"][0], sel)
    assert_bf16_close("o", got["o"][0], o)


def test_sparse_latent_full_size_sampled_rows():
    w = configs.LATENT_P1M
    res = synth.resident(w)
    m = synth.member(w, 0)
    d = dict(latent_p=res["latent_p"], k_idx=res["k_idx"], q=m["q"], latent_r=m["latent_r"],
             q_idx=m["q_idx"], d_o=m["d_o"])
    print(f"[sparse] {w.name} full size", flush=True)
    got = _run(d, w.P, w.R, w.topk, w.block)
    # 512 seeded positions (every head of each: all 64 heads share a position's selection)
    rows = np.union1d(synth.sample_rows(w.seed, w.R, 512, w.block), np.arange(w.R - 4, w.R))
    print(f"[sparse] oracle over {rows.size} positions", flush=True)
    sel, sig, o, lse, gr = _oracle(d, w.topk, rows=rows)
    same = []
    for n, r in enumerate(rows):
        gsel = np.sort(got["idx"][0][r])
        assert gsel.size == w.topk and np.unique(gsel).size == w.topk and gsel.min() >= 0 and gsel.max() < w.P
        if np.array_equal(gsel, sel[r]):
            same.append(n)
            continue
        # a different selection must still be a valid top-k by the exact scores
        s = sig[n]
        mask = np.zeros(w.P, dtype=bool)
        mask[gsel] = True
        kth = np.sort(s)[-w.topk]
        eps = 1e-4 * max(1.0, abs(kth))
        assert s[mask].min() >= s[~mask].max() - eps, f"row {r}: invalid selection"
    assert len(same) >= len(rows) // 2, f"only {len(same)} of {len(rows)} rows have the unique selection"
    same = np.array(same)
    assert_bf16_close("o", got["o"][0][rows[same]], o[same])
    assert_bf16_close("dq", got["dq"][0][rows[same]], gr["dq"][same])
    assert np.max(np.abs(got["lse"][0][rows[same]] - lse[same])) <= 2e-2
    tail = np.arange(w.R - 4, w.R)
    if all(np.array_equal(np.sort(got["idx"][0][r]), sel[r]) for r in tail):
        assert_bf16_close("dk_r tail", got["dk"][0][w.R - 4:], gr["dk_r"][w.R - 4:])
        assert_bf16_close("dv_r tail", got["dv"][0][w.R - 4:], gr["dv_r"][w.R - 4:])
    assert np.all(np.isfinite(got["dk"][0])) and np.all(np.isfinite(got["dv"][0]))


def test_sparse_deterministic():
    """Two runs on the same inputs agree bit for bit (fixed-order reductions everywhere,
    including the chunked dK_r / dV_r partial sums)."""
    P, R, topk = 3000, 96, 256
    d = _data(8300, P, R, integer_index=False)
    print("[sparse] determinism", flush=True)
    a = _run(d, P, R, topk, 32)
    b = _run(d, P, R, topk, 32)
    for key in ("idx", "o", "lse", "dq", "dk", "dv"):
        assert np.array_equal(a[key], b[key], equal_nan=True), key


def test_sparse_varlen_microbatch():
    """Two responses in one call (K = 2), one shorter than R_max: the valid rows of each
    match the oracle exactly in selection and to the bf16 bounds in values; padding rows
    get O = 0, lse = -inf, selection -1 and zero gradients."""
    from tests import _gpu as G
    P, Rm, topk, lens = 3000, 64, 256, (64, 37)
    ds = [_data(8400 + n, P, Rm, integer_index=True) for n in range(2)]
    base = ds[0]
    stack = lambda key: np.stack([d[key] for d in ds])
    prob = G.latent_problem(P, Rm, topk, 32, K=2)
    run = G.LatentRun(prob, base["latent_p"], base["k_idx"], stack("q"), stack("latent_r"), stack("q_idx"),
                      stack("d_o"), lens)
    print("[sparse] varlen microbatch", flush=True)
    got = run.fwd().bwd().numpy()
    for kk, rl in enumerate(lens):
        d = dict(latent_p=base["latent_p"], k_idx=base["k_idx"], q=ds[kk]["q"][:rl],
                 latent_r=ds[kk]["latent_r"][:rl], q_idx=ds[kk]["q_idx"][:rl], d_o=ds[kk]["d_o"][:rl])
        sel, sig, o, lse, gr = _oracle(d, topk)
        np.testing.assert_array_equal(got["idx"][kk][:rl], sel)
        assert_bf16_close(f"o[{kk}]", got["o"][kk][:rl], o)
        assert_bf16_close(f"dq[{kk}]", got["dq"][kk][:rl], gr["dq"])
        assert_bf16_close(f"dk_r[{kk}]", got["dk"][kk][:rl], gr["dk_r"])
        assert_bf16_close(f"dv_r[{kk}]", got["dv"][kk][:rl], gr["dv_r"])
        if rl < Rm:
            assert np.all(got["idx"][kk][rl:] == -1)
            assert np.all(got["o"][kk][rl:] == 0) and np.all(np.isneginf(got["lse"][kk][rl:]))
            for key in ("dq", "dk", "dv"):
                assert np.all(got[key][kk][rl:] == 0), key


def test_sparse_caller_driven_reverse_walk():
    """The backward driven one block at a time (last block first, accumulating) equals the
    whole walk bit for bit, and after the call for block b the dK_r / dV_r rows of block b
    already hold their final values."""
    import torch
    from tests import _gpu as G
    P, R, topk, block = 3000, 96, 256, 32
    d = _data(8500, P, R, integer_index=False)
    prob = G.latent_problem(P, R, topk, block)
    run = G.LatentRun(prob, d["latent_p"], d["k_idx"], d["q"][None], d["latent_r"][None], d["q_idx"][None],
                      d["d_o"][None], [R])
    print("[sparse] caller-driven walk", flush=True)
    full = run.fwd().bwd().numpy()
    for t in (run.dq, run.dk, run.dv):
        t.zero_()
    nb = (R + block - 1) // block
    for b in reversed(range(nb)):
        run.bwd(accumulate=1, block_idx=b)
        torch.cuda.synchronize()
        lo, hi = b * block, min(R, (b + 1) * block)
        assert np.array_equal(run.dk[0, lo:hi].double().cpu().numpy(), full["dk"][0, lo:hi]), b
        assert np.array_equal(run.dv[0, lo:hi].double().cpu().numpy(), full["dv"][0, lo:hi]), b
    walked = run.numpy()
    for key in ("dq", "dk", "dv"):
        assert np.array_equal(walked[key], full[key]), key


def test_sparse_select_everything_and_empty_response():
    """top-k = P (every prompt position selected: attention becomes dense over the prompt)
    in a microbatch whose second response is empty (r_len = 0: all of its rows are
    padding)."""
    from tests import _gpu as G
    P, Rm, topk, lens = 512, 32, 512, (32, 0)
    ds = [_data(8600 + n, P, Rm, integer_index=False) for n in range(2)]
    base = ds[0]
    stack = lambda key: np.stack([d[key] for d in ds])
    prob = G.latent_problem(P, Rm, topk, 32, K=2)
    run = G.LatentRun(prob, base["latent_p"], base["k_idx"], stack("q"), stack("latent_r"), stack("q_idx"),
                      stack("d_o"), lens)
    print("[sparse] select everything + empty response", flush=True)
    got = run.fwd().bwd().numpy()
    sel, sig, o, lse, gr = _oracle(base, topk)
    np.testing.assert_array_equal(got["idx"][0], np.tile(np.arange(P), (Rm, 1)))
    np.testing.assert_array_equal(sel, np.tile(np.arange(P), (Rm, 1)))
    assert_bf16_close("o", got["o"][0], o)
    assert_bf16_close("dq", got["dq"][0], gr["dq"])
    assert_bf16_close("dk_r", got["dk"][0], gr["dk_r"])
    assert_bf16_close("dv_r", got["dv"][0], gr["dv_r"])
    assert np.all(got["idx"][1] == -1)
    assert np.all(got["o"][1] == 0) and np.all(np.isneginf(got["lse"][1]))
    for key in ("dq", "dk", "dv"):
        assert np.all(got[key][1] == 0), key
