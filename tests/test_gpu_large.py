"""GPU parity past 32-bit offsets (needs an MI355X): a resident prompt of 16,778,216
positions with one KV head of 128 dims holds 2^31 + 128,000 elements (4.3 GB) per K and V
tensor, so key offsets pass 2^31 elements and 2^32 bytes.  The oracle receives the same
values widened exactly to fp32 and gathers each KV head in fp64.
"""
import numpy as np
import pytest
import torch

from oracle import dense
from resident_kv_response_amd import configs, rr_attn as R, synth
from tests._helpers import assert_bf16_close, assert_D_close

pytestmark = pytest.mark.gpu

BIG = configs.GQA_P128K.with_(P=(1 << 24) + 1000, R=96, Hq=8, Hkv=1, chunk=1 << 20, block=64, seed=5100)


@pytest.fixture(scope="module")
def big_resident():
    res = synth.resident(BIG)
    f32 = {n: synth.bf16_bits_to_f32(res[n]) for n in ("k_p", "v_p")}
    return res, f32


def test_forward_backward_sampled_rows(big_resident):
    """O, lse, D and dQ of 64 sampled query rows (every row sees every key, those past the
    boundary included), and dK_r, dV_r of the last 4 response keys."""
    from tests import _gpu as G
    res, f32 = big_resident
    w = BIG
    st = G.stack_members([synth.member(w, 0)], w.R)
    prob = G.problem(w.P, w.R, w.Hq, w.Hkv, w.d_qk, w.chunk, w.block, w.dtype, tau=w.tau)
    print(f"[large] P={w.P} R={w.R} Hq={w.Hq} Hkv={w.Hkv}", flush=True)
    got = G.Run(prob, w.dtype, res["k_p"], res["v_p"], st, [w.R]).fwd().bwd().numpy()
    rows, heads = synth.sample_query_rows(w.seed, w.R, w.Hq, 64, w.block)
    n_tail = 4
    tail = np.arange(w.R - n_tail, w.R)
    flat = np.union1d(rows * w.Hq + heads, (tail[:, None] * w.Hq + np.arange(w.Hq)).ravel())
    rows, heads = flat // w.Hq, flat % w.Hq
    print(f"[large] oracle over {rows.size} query rows", flush=True)
    x = {n: synth.as_f64(st[n][0], w.dtype) for n in ("q", "k_r", "v_r", "d_o")}
    ref = dense.attend_rows(x["q"], f32["k_p"], f32["v_p"], x["k_r"], x["v_r"], x["d_o"], w.tau, rows, heads,
                            batch_bytes=16 << 30)
    assert_bf16_close("o", got["o"][0][rows, heads], ref["o"])
    assert_bf16_close("dq", got["dq"][0][rows, heads], ref["dq"])
    assert_D_close("D", got["D"][0][rows, heads], ref["D"], w.dtype)
    assert np.max(np.abs(got["lse"][0][rows, heads] - ref["lse"])) <= 2e-2
    assert_bf16_close("dk_r tail", got["dk"][0][w.R - n_tail:], ref["dk_r"][w.R - n_tail:])
    assert_bf16_close("dv_r tail", got["dv"][0][w.R - n_tail:], ref["dv_r"][w.R - n_tail:])


def test_prompt_grads_across_the_boundary(big_resident):
    """Full-sequence prompt gradients of a 4-row response at keys on both sides of the
    2^31-element boundary (key 2^24), of each chunk boundary near it, and at the end."""
    from tests import _gpu as G
    res, f32 = big_resident
    w = BIG.with_(R=4)
    st = G.stack_members([synth.member(w, 0)], w.R)
    prob = G.problem(w.P, w.R, w.Hq, w.Hkv, w.d_qk, w.chunk, w.block, w.dtype, tau=w.tau)
    print(f"[large] prompt grads P={w.P} R={w.R}", flush=True)
    run = G.Run(prob, w.dtype, res["k_p"], res["v_p"], st, [w.R]).fwd()
    dk = torch.empty((w.P, w.Hkv, w.d_qk), device="cuda")
    dv = torch.empty((w.P, w.Hkv, w.d_v), device="cuda")
    R.rr_attn_prompt_grads(prob, run.kv, run.q, run.r_len, run.o, run.lse, run.d_o, dk, dv,
                           ws=R.workspace(prob, R.RR_OP_PROMPT_GRADS, "cuda"))
    torch.cuda.synchronize()
    b = 1 << 24
    keys = np.array([0, 1, 15 * w.chunk - 1, 15 * w.chunk, b - 129, b - 128, b - 2, b - 1, b, b + 1,
                     b + 127, b + 128, w.P - 2, w.P - 1])
    x = {n: synth.as_f64(st[n][0], w.dtype) for n in ("q", "k_r", "v_r", "d_o")}
    rows = np.repeat(np.arange(w.R), w.Hq)
    heads = np.tile(np.arange(w.Hq), w.R)
    ref = dense.attend_rows(x["q"], f32["k_p"], f32["v_p"], x["k_r"], x["v_r"], x["d_o"], w.tau, rows, heads,
                            batch_bytes=16 << 30)
    o = ref["o"].reshape(w.R, w.Hq, w.d_v)
    lse = ref["lse"].reshape(w.R, w.Hq)
    ref_k, ref_v = dense.prompt_grads_given_stats(x["q"], f32["k_p"], f32["v_p"], x["d_o"], o, lse, w.tau, keys)
    at = torch.as_tensor(keys, device="cuda")
    assert_bf16_close("dk_p", dk[at].double().cpu().numpy(), ref_k)
    assert_bf16_close("dv_p", dv[at].double().cpu().numpy(), ref_v)
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all()
