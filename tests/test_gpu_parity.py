"""GPU parity of the HIP path against the fp64 oracle (needs an MI355X).

Tolerances: fp32 inputs, max-abs <= 1e-5 on O, lse, dQ, dK, dV; bf16 inputs, rel-L2 <= 5e-3
and max-abs <= 2e-2 on O, dQ, dK, dV (lse max-abs <= 2e-2).  Padding rows (i >= r_len)
must hold O = 0, lse = -inf and zero gradients.
"""
import numpy as np
import pytest

from oracle import dense
from resident_kv_response_amd import configs, synth
from tests._helpers import assert_bf16_close, assert_D_close, assert_f32_close

pytestmark = pytest.mark.gpu


def _inputs(w, members_R):
    res = synth.resident(w)
    mem = [synth.member(w, g, R=rg) for g, rg in enumerate(members_R)]
    return res, mem


def _run_and_check(w, members_R, R_max=None, chunk=None, block=None, check_rows=None):
    from tests import _gpu as G
    R_max = R_max or max(members_R)
    chunk = chunk or w.chunk
    block = block or w.block
    res, mem = _inputs(w, members_R)
    st = G.stack_members(mem, R_max)
    prob = G.problem(w.P, R_max, w.Hq, w.Hkv, w.d_qk, chunk, block, w.dtype, K=len(members_R), tau=w.tau)
    print(f"[parity] {w.name} K={len(members_R)} R={members_R} chunk={chunk} block={block}", flush=True)
    run = G.Run(prob, w.dtype, res["k_p"], res["v_p"], st, members_R).fwd().bwd()
    got = run.numpy()
    for kk, rl in enumerate(members_R):
        rows = None if check_rows is None else check_rows
        ref = G.oracle_member(dense, w.dtype, res["k_p"], res["v_p"], st, kk, rl, w.tau, rows=rows)
        sel = slice(0, rl) if rows is None else rows
        pairs = [("o", got["o"][kk][sel], ref["o"]), ("dq", got["dq"][kk][sel], ref["dq"])]
        if rows is None:
            pairs += [("dk_r", got["dk"][kk][:rl], ref["dk_r"]), ("dv_r", got["dv"][kk][:rl], ref["dv_r"])]
        for name, a, b in pairs:
            if w.dtype == "f32":
                assert_f32_close(f"{name}[k={kk}]", a, b)
            else:
                assert_bf16_close(f"{name}[k={kk}]", a, b)
        lse_tol = 1e-5 if w.dtype == "f32" else 2e-2
        if rl > 0:
            assert np.max(np.abs(got["lse"][kk][sel] - ref["lse"])) <= lse_tol
            # D = dO . O of the backward's preprocess, against the oracle's O
            d_o = synth.as_f64(st["d_o"][kk, :rl], w.dtype)[sel]
            D_ref = np.sum(d_o * ref["o"], axis=-1)
            assert_D_close(f"D[k={kk}]", got["D"][kk][sel], D_ref, w.dtype)
        # padding rows
        assert np.all(got["o"][kk][rl:] == 0) and np.all(np.isneginf(got["lse"][kk][rl:]))
        assert np.all(got["dq"][kk][rl:] == 0)
        assert np.all(got["dk"][kk][rl:] == 0) and np.all(got["dv"][kk][rl:] == 0)
        assert np.all(got["D"][kk][rl:] == 0)
    return got


def test_tiny_f32_config():
    w = configs.TINY_F32
    _run_and_check(w, [w.R])


@pytest.mark.parametrize("chunk,block", [(1000, 64), (4096, 100), (4097, 256), (333, 17)])
def test_tiny_f32_partitions(chunk, block):
    w = configs.TINY_F32.with_(P=2500, R=200, seed=2001)
    _run_and_check(w, [w.R], chunk=chunk, block=block)


def test_f32_head_dim_128_gqa():
    # the fp32 kernels at d = 128 with two KV heads (the fp32 configuration itself is d = 64)
    w = configs.TINY_F32.with_(P=1300, R=100, Hq=4, Hkv=2, d_qk=128, d_v=128, seed=2101)
    _run_and_check(w, [100, 37], chunk=512, block=48)


def test_empty_prompt():
    # P = 0: the rows attend to their own causal keys only
    for base, seed in ((configs.SHARE_P256K, 2201), (configs.TINY_F32, 2202)):
        w = base.with_(P=0, R=150, chunk=64, block=64, seed=seed)
        _run_and_check(w, [150, 61])


@pytest.mark.parametrize("d,Hq,Hkv", [(128, 8, 2), (64, 8, 2), (128, 12, 2), (128, 4, 4)])
def test_bf16_multitile_ragged(d, Hq, Hkv):
    # several row tiles, ragged chunk and block tails, causal response across tiles
    w = configs.GQA_P128K.with_(P=5000, R=600, Hq=Hq, Hkv=Hkv, d_qk=d, d_v=d, chunk=2048, block=256,
                                seed=3000 + d + Hq)
    _run_and_check(w, [w.R])


@pytest.mark.parametrize("dtype,P,chunk", [("bf16", 1, 16), ("bf16", 33, 16), ("f32", 1, 4), ("f32", 45, 16)])
def test_tiny_prompts_and_chunks(dtype, P, chunk):
    # a one-position prompt, and prompts whose every chunk is shorter than a 32-key subtile
    base = configs.TINY_F32 if dtype == "f32" else configs.SHARE_P256K
    w = base.with_(P=P, R=70, chunk=chunk, block=32, seed=4100 + P)
    _run_and_check(w, [70, 41], R_max=72)


def test_bf16_varlen_microbatch():
    # K = 4 responses of different lengths in one call, including a one-row and an empty one
    w = configs.SHARE_P256K.with_(P=3000, R=400, chunk=1024, block=128, seed=4001)
    _run_and_check(w, [400, 263, 1, 0], R_max=400)


def test_f32_varlen_microbatch():
    w = configs.TINY_F32.with_(P=700, R=90, seed=4002)
    _run_and_check(w, [90, 33, 0], R_max=96, chunk=256, block=32)


@pytest.mark.parametrize("cfg", ["GQA_P128K", "SHARE_P256K", "FULL_P2M"])
def test_full_size_sampled_rows(cfg):
    """Full-size configurations: every output of the GPU path is produced; O, lse and dQ of
    512 seeded sampled query rows (a query row is one position of one head; both sides of
    every block boundary and the first and last rows of each response among them) are
    compared with the oracle.  The 2M group spreads them over its 8 members at their seeded
    lengths, 64 each.  dK/dV of the last 16 response keys (of the first member) are
    compared too: only the last 16 positions reach them, and every head of those is added
    to the sample."""
    from tests import _gpu as G
    w = getattr(configs, cfg)
    lens = [int(r) for r in synth.response_lengths(w)] if w.G > 1 else [w.R]
    n_tail = 16
    res = synth.resident(w)
    f = lambda x: synth.as_f64(x, w.dtype)
    kp, vp = f(res["k_p"]), f(res["v_p"])
    got_all = {k: [] for k in ("o", "lse", "D", "dq")}
    ref_all = {k: [] for k in ("o", "lse", "D", "dq")}
    for g, Rg in enumerate(lens):
        st = G.stack_members([synth.member(w, g, R=Rg)], Rg)
        prob = G.problem(w.P, Rg, w.Hq, w.Hkv, w.d_qk, w.chunk, w.block, w.dtype, tau=w.tau)
        print(f"[parity] {w.name} member {g} full size, R={Rg}", flush=True)
        got = G.Run(prob, w.dtype, res["k_p"], res["v_p"], st, [Rg]).fwd().bwd().numpy()
        assert np.all(np.isfinite(got["dk"])) and np.all(np.isfinite(got["dv"]))
        rows, heads = synth.sample_query_rows(w.seed + g, Rg, w.Hq, 512 // len(lens), w.block)
        if g == 0:
            tail = np.arange(Rg - n_tail, Rg)
            flat = np.union1d(rows * w.Hq + heads, (tail[:, None] * w.Hq + np.arange(w.Hq)).ravel())
            rows, heads = flat // w.Hq, flat % w.Hq
        print(f"[parity] oracle over {rows.size} query rows", flush=True)
        x = {n: f(st[n][0, :Rg]) for n in ("q", "k_r", "v_r", "d_o")}
        ref = dense.attend_rows(x["q"], kp, vp, x["k_r"], x["v_r"], x["d_o"], w.tau, rows, heads)
        for k in got_all:
            got_all[k].append(got[k][0][rows, heads])
            ref_all[k].append(ref[k])
        if g == 0:
            assert_bf16_close("dk_r tail", got["dk"][0][Rg - n_tail:], ref["dk_r"][Rg - n_tail:])
            assert_bf16_close("dv_r tail", got["dv"][0][Rg - n_tail:], ref["dv_r"][Rg - n_tail:])
    cat = lambda d, k: np.concatenate(d[k])
    assert_bf16_close("o", cat(got_all, "o"), cat(ref_all, "o"))
    assert_bf16_close("dq", cat(got_all, "dq"), cat(ref_all, "dq"))
    assert_D_close("D", cat(got_all, "D"), cat(ref_all, "D"), w.dtype)
    assert np.max(np.abs(cat(got_all, "lse") - cat(ref_all, "lse"))) <= 2e-2


@pytest.fixture(scope="module")
def gqa_full():
    """The GQA configuration (P = 131,072, R = 4096, 32/8 heads) run once through the GPU
    path, with the oracle's fp64 inputs."""
    from tests import _gpu as G
    w = configs.GQA_P128K
    res, mem = _inputs(w, [w.R])
    st = G.stack_members(mem, w.R)
    prob = G.problem(w.P, w.R, w.Hq, w.Hkv, w.d_qk, w.chunk, w.block, w.dtype, tau=w.tau)
    print(f"[parity] {w.name} full run", flush=True)
    got = G.Run(prob, w.dtype, res["k_p"], res["v_p"], st, [w.R]).fwd().bwd().numpy()
    f = lambda x: synth.as_f64(x, w.dtype)
    x = {n: f(st[n][0]) for n in ("q", "k_r", "v_r", "d_o")}
    x["k_p"], x["v_p"] = f(res["k_p"]), f(res["v_p"])
    return w, x, got


@pytest.mark.parametrize("g", range(8))
def test_gqa_full_size_every_row(gqa_full, g):
    """Every row of the GQA configuration, one KV head per case: O, lse and dQ of all 4096
    positions of its 4 query heads, and, since every query row that reaches them is
    included, the full dK_r, dV_r of that KV head."""
    w, x, got = gqa_full
    grp = w.Hq // w.Hkv
    print(f"[parity] {w.name} every row of KV head {g}", flush=True)
    rows = np.repeat(np.arange(w.R), grp)
    heads = np.tile(np.arange(g * grp, (g + 1) * grp), w.R)
    ref = dense.attend_rows(x["q"], x["k_p"], x["v_p"], x["k_r"], x["v_r"], x["d_o"], w.tau, rows, heads)
    assert_bf16_close("o", got["o"][0][rows, heads], ref["o"])
    assert_bf16_close("dq", got["dq"][0][rows, heads], ref["dq"])
    assert_D_close("D", got["D"][0][rows, heads], ref["D"], w.dtype)
    assert np.max(np.abs(got["lse"][0][rows, heads] - ref["lse"])) <= 2e-2
    assert_bf16_close("dk_r", got["dk"][0][:, g], ref["dk_r"][:, g])
    assert_bf16_close("dv_r", got["dv"][0][:, g], ref["dv_r"][:, g])


@pytest.mark.parametrize("slope", [6.0, 40.0, 400.0])
def test_bf16_growing_scores(slope):
    """Scores that rise along the prompt (a ramp in one key dimension that every query
    reads), so a row's running maximum keeps moving: the forward's pipelined subtiles
    keep exceeding their row-sum bound and are redone against the new maximum (every few
    subtiles at the steepest slope).  O and lse are checked at the bf16 bounds for every
    slope, the gradients at those bounds for the mild slope.  With a ramp of height 40 or
    400 in one key dimension, dQ = tau sum_j dS_j k_j relies on sum_j dS_j = 0 to cancel
    the common ramp, which rounding dS to bf16 before the dQ product (reading 9) leaves
    incomplete; there every element of dQ, dK_r and dV_r is held to the bound of the
    bf16 rounding model (tests/_bounds.py), computed from the oracle's exact values."""
    from tests import _gpu as G
    from tests._bounds import bwd_bounds, worst_ratio
    w = configs.GQA_P128K.with_(P=6000, R=300, Hq=8, Hkv=2, chunk=2048, block=128, seed=4300)
    res, mem = _inputs(w, [w.R])
    kp = synth.bf16_bits_to_f32(res["k_p"]).copy()
    kp[:, :, 0] = slope * np.linspace(-1.0, 1.0, w.P, dtype=np.float32)[:, None]
    res["k_p"] = synth.f32_to_bf16_bits(kp)
    q = synth.bf16_bits_to_f32(mem[0]["q"]).copy()
    q[:, :, 0] = 4.0
    mem[0]["q"] = synth.f32_to_bf16_bits(q)
    st = G.stack_members(mem, w.R)
    prob = G.problem(w.P, w.R, w.Hq, w.Hkv, w.d_qk, w.chunk, w.block, w.dtype, tau=w.tau)
    print(f"[parity] growing scores slope={slope}", flush=True)
    got = G.Run(prob, w.dtype, res["k_p"], res["v_p"], st, [w.R]).fwd().bwd().numpy()
    ref = G.oracle_member(dense, w.dtype, res["k_p"], res["v_p"], st, 0, w.R, w.tau)
    assert_bf16_close("o", got["o"][0], ref["o"])
    assert np.max(np.abs(got["lse"][0] - ref["lse"])) <= 2e-2
    if slope <= 6.0:
        for name, a, b in [("dq", got["dq"][0], ref["dq"]), ("dk_r", got["dk"][0], ref["dk_r"]),
                           ("dv_r", got["dv"][0], ref["dv_r"])]:
            assert_bf16_close(name, a, b)
    f = lambda x: synth.as_f64(x, w.dtype)
    x = [f(st[n][0]) for n in ("q",)] + [f(res["k_p"]), f(res["v_p"])] + [f(st[n][0]) for n in ("k_r", "v_r", "d_o")]
    bounds = bwd_bounds(*x, w.tau, ref["dq"], ref["dk_r"], ref["dv_r"])
    for name, a, b, bnd in [("dq", got["dq"][0], ref["dq"], bounds[0]), ("dk_r", got["dk"][0], ref["dk_r"], bounds[1]),
                            ("dv_r", got["dv"][0], ref["dv_r"], bounds[2])]:
        ratio = worst_ratio(a, b, bnd)
        rel = float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
        print(f"[parity] slope={slope} {name}: worst |err|/bound {ratio:.3f}, rel-L2 {rel:.2e}", flush=True)
        assert ratio <= 1.0, f"{name}: error exceeds the bf16 rounding-model bound ({ratio:.3f})"
