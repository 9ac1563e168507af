"""GPU parity of the latent-page sparse variant (needs an MI355X): fp32 index scores and
exact per-query top-k (ties toward the lower position), attention over the selected latent
rows plus the response's causal rows with 64 heads sharing each 576-wide row (value = its
first 512 dims), and the response-only backward (dq, dk_r, dv_r).

The selection is decided by fp32 scores on both sides, summed in different orders, so
where two positions' scores lie within fp32 rounding of each other at the k-th place,
several selections are correct.  At full size each sampled row's selection is therefore
checked against the exact fp64 scores sigma and the fp32 bound e_j = g * sum |q_idx||k_idx_j|
(g = 128 * 2^-24 / (1 - 128 * 2^-24), the error of any fp32 evaluation of a 128-term dot
product): every position the GPU chose must score at least every position it left out,
within e; every difference from the oracle's selection must be a swap of positions within
e of each other; rows the oracle marks unambiguous (no position outside its selection
within e of one inside) must match it exactly; and at least 500 of the sampled rows must
match it exactly.  Attention values are compared on the rows whose selection matches.
With small-integer index data every score is exact in fp32, the selection is unique, and
every output element is compared."""
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


class _ExactScores:
    """Exact index scores (fp64 products of the fp32 values, whose 128-term sums are exact
    to far below the fp32 bound) and the fp32 evaluation bound e of each (row, position).
    e is formed in fp32 from |q_idx| |k_idx| and enlarged by 1e-4 relative, which covers
    that product's own rounding."""

    def __init__(self, k_idx):
        from tests._bounds import G128
        self.g = G128 * 1.0001
        self.kd = np.asarray(k_idx, np.float64)
        self.ka = np.abs(np.asarray(k_idx, np.float32))

    def batches(self, q_idx_rows, batch=32):
        """(first row, sigma [n][P], e [n][P]) per batch of rows."""
        for a in range(0, q_idx_rows.shape[0], batch):
            q = q_idx_rows[a:a + batch]
            sig = np.asarray(q, np.float64) @ self.kd.T
            err = np.abs(np.asarray(q, np.float32)) @ self.ka.T
            yield a, sig, self.g * err.astype(np.float64)


def _unambiguous(sig, err, sel):
    """No position outside sel within fp32 rounding of one inside it."""
    mask = np.zeros(sig.size, dtype=bool)
    mask[sel] = True
    return (sig[mask] - err[mask]).min() > (sig[~mask] + err[~mask]).max()


def test_sparse_latent_full_size_sampled_rows():
    w = configs.LATENT_P1M
    res = synth.resident(w)
    m = synth.member(w, 0)
    d = dict(latent_p=res["latent_p"], k_idx=res["k_idx"], q=m["q"], latent_r=m["latent_r"],
             q_idx=m["q_idx"], d_o=m["d_o"])
    from tests import _gpu as G
    prob = G.latent_problem(w.P, w.R, w.topk, w.block)
    run = G.LatentRun(prob, d["latent_p"], d["k_idx"], d["q"][None], d["latent_r"][None], d["q_idx"][None],
                      d["d_o"][None], [w.R])
    print(f"[sparse] {w.name} full size", flush=True)
    got = run.fwd().bwd().numpy()
    # 512 seeded positions (every head of each: all 64 heads share a position's selection)
    rows = np.union1d(synth.sample_rows(w.seed, w.R, 512, w.block), np.arange(w.R - 4, w.R))
    print(f"[sparse] oracle over {rows.size} positions", flush=True)
    sel, _, o, lse, gr = _oracle(d, w.topk, rows=rows)
    exact = _ExactScores(d["k_idx"])
    same, unamb = [], 0
    for n, s, e in ((a + i, sb[i], eb[i]) for a, sb, eb in exact.batches(d["q_idx"][rows]) for i in range(len(sb))):
        r = rows[n]
        gsel = np.sort(got["idx"][0][r])
        assert gsel.size == w.topk and np.unique(gsel).size == w.topk and gsel.min() >= 0 and gsel.max() < w.P
        mask = np.zeros(w.P, dtype=bool)
        mask[gsel] = True
        # a valid top-k by the exact scores, up to fp32 evaluation
        assert (s[mask] + e[mask]).min() >= (s[~mask] - e[~mask]).max(), f"row {r}: invalid selection"
        only_gpu = np.setdiff1d(gsel, sel[r])
        only_orc = np.setdiff1d(sel[r], gsel)
        assert only_gpu.size == only_orc.size
        for a_ in only_gpu:             # each difference: a swap within fp32 rounding
            assert np.all(np.abs(s[a_] - s[only_orc]) <= e[a_] + e[only_orc]), f"row {r}: swap outside the band"
        if _unambiguous(s, e, sel[r]):
            unamb += 1
            assert only_gpu.size == 0, f"row {r}: unambiguous row selected differently"
        if only_gpu.size == 0:
            same.append(n)
    print(f"[sparse] selection equal to the oracle's on {len(same)} of {rows.size} positions "
          f"({unamb} unambiguous by the fp32 bound)", flush=True)
    assert len(same) >= 500, f"only {len(same)} of {rows.size} positions have the oracle's selection"
    same = np.array(same)
    assert_bf16_close("o", got["o"][0][rows[same]], o[same])
    assert_bf16_close("dq", got["dq"][0][rows[same]], gr["dq"][same])
    assert np.max(np.abs(got["lse"][0][rows[same]] - lse[same])) <= 2e-2

    # dK_r / dV_r of the last response keys: key j collects rows i >= j, so the check needs
    # a run of consecutive rows whose selection is unambiguous.  The oracle finds the last
    # four such rows below R; the response is replayed with that length, and those rows'
    # selections must then equal the oracle's.
    t_end = None
    for t in range(w.R - 1, w.R - 257, -1):
        cand = np.arange(t - 3, t + 1)
        _, s4, e4 = next(exact.batches(d["q_idx"][cand]))
        sel4 = sparse.topk_select(sparse.index_scores(d["q_idx"][cand], d["k_idx"]), w.topk)
        if all(_unambiguous(s4[n], e4[n], sel4[n]) for n in range(4)):
            t_end = t + 1
            break
    assert t_end is not None, "no four consecutive unambiguous rows near the end"
    print(f"[sparse] tail check: response of {t_end} rows", flush=True)
    run.r_len = [t_end]
    got2 = run.fwd().bwd().numpy()
    tail = np.arange(t_end - 4, t_end)
    dt = dict(d, q=d["q"][:t_end], latent_r=d["latent_r"][:t_end], q_idx=d["q_idx"][:t_end], d_o=d["d_o"][:t_end])
    sel_t, _, _, _, gr_t = _oracle(dt, w.topk, rows=tail)
    for r in tail:
        np.testing.assert_array_equal(np.sort(got2["idx"][0][r]), sel_t[r])
    assert_bf16_close("dk_r tail", got2["dk"][0][tail], gr_t["dk_r"][tail])
    assert_bf16_close("dv_r tail", got2["dv"][0][tail], gr_t["dv_r"][tail])
    assert np.all(got2["idx"][0][t_end:] == -1)
    for key in ("dq", "dk", "dv"):
        assert np.all(got2[key][0][t_end:] == 0), key
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
