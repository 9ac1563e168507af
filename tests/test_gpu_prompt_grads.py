"""GPU parity of the full-sequence differential mode (needs an MI355X): dk_p, dv_p of the
resident prompt K/V, the term the response-only contract drops, against the fp64 oracle.

Small problems compare every element with the full-sequence oracle (bf16: rel-L2 <= 5e-3
and max-abs <= 2e-2; fp32: max-abs <= 1e-5).  At the full 2,097,152-position prompt,
sampled positions of a short response are compared with the oracle, and the full-length
member is checked through two identities of the exact gradients over all keys.
"""
import numpy as np
import pytest
import torch

from oracle import dense
from resident_kv_response_amd import configs, rr_attn as R, synth
from tests._helpers import assert_bf16_close, assert_f32_close

pytestmark = pytest.mark.gpu


def _setup(w, lens, chunk=None, block=None):
    from tests import _gpu as G
    res = synth.resident(w)
    mem = [synth.member(w, g, R=r) for g, r in enumerate(lens)]
    st = G.stack_members(mem, max(lens))
    prob = G.problem(w.P, max(lens), w.Hq, w.Hkv, w.d_qk, chunk or w.chunk, block or w.block, w.dtype,
                     K=len(lens), tau=w.tau)
    run = G.Run(prob, w.dtype, res["k_p"], res["v_p"], st, lens).fwd()
    return G, res, mem, st, prob, run


def _prompt_grads(run, prob, accumulate=0, out=None):
    dk, dv = out if out is not None else (
        torch.full((prob.P, prob.Hkv, prob.d_qk), float("nan"), device="cuda"),
        torch.full((prob.P, prob.Hkv, prob.d_v), float("nan"), device="cuda"))
    ws = R.workspace(prob, R.RR_OP_PROMPT_GRADS, "cuda")
    R.rr_attn_prompt_grads(prob, run.kv, run.q, run.r_len, run.o, run.lse, run.d_o, dk, dv,
                           accumulate=accumulate, ws=ws)
    torch.cuda.synchronize()
    return dk, dv


def _oracle_sum(w, res, mem, lens):
    f = lambda x: synth.as_f64(x, w.dtype)
    dk = np.zeros((w.P, w.Hkv, w.d_qk))
    dv = np.zeros((w.P, w.Hkv, w.d_v))
    for m, rl in zip(mem, lens):
        if rl == 0:
            continue
        g = dense.attend_bwd(f(m["q"][:rl]), f(res["k_p"]), f(res["v_p"]), f(m["k_r"][:rl]),
                             f(m["v_r"][:rl]), f(m["d_o"][:rl]), w.tau, full_sequence=True)
        dk += g["dk_p"]
        dv += g["dv_p"]
    return dk, dv


@pytest.mark.parametrize("d,Hq,Hkv,P,lens", [
    (128, 24, 4, 4100, [520, 77]),      # ragged last key tile, two responses, ragged stages
    (64, 8, 2, 3000, [300, 1, 0]),      # d = 64, a one-row and an empty response
    (128, 8, 8, 1000, [200]),           # one query head per KV head
])
def test_bf16_every_element(d, Hq, Hkv, P, lens):
    w = configs.SHARE_P256K.with_(P=P, R=max(lens), Hq=Hq, Hkv=Hkv, d_qk=d, d_v=d, chunk=1024,
                                  block=128, seed=7001 + d + Hq)
    print(f"[prompt_grads] bf16 d={d} Hq={Hq} Hkv={Hkv} P={P} R={lens}", flush=True)
    G, res, mem, st, prob, run = _setup(w, lens)
    dk, dv = _prompt_grads(run, prob)
    ref_k, ref_v = _oracle_sum(w, res, mem, lens)
    assert_bf16_close("dk_p", dk.double().cpu().numpy(), ref_k)
    assert_bf16_close("dv_p", dv.double().cpu().numpy(), ref_v)


@pytest.mark.parametrize("d,Hkv", [(64, 1), (128, 2)])
def test_f32_every_element(d, Hkv):
    w = configs.TINY_F32.with_(P=1500, R=90, Hkv=Hkv, d_qk=d, d_v=d, seed=7101 + d)
    lens = [90, 33]
    print(f"[prompt_grads] f32 d={d} P={w.P} R={lens}", flush=True)
    G, res, mem, st, prob, run = _setup(w, lens, chunk=512, block=32)
    dk, dv = _prompt_grads(run, prob)
    ref_k, ref_v = _oracle_sum(w, res, mem, lens)
    assert_f32_close("dk_p", dk.double().cpu().numpy(), ref_k)
    assert_f32_close("dv_p", dv.double().cpu().numpy(), ref_v)


def test_accumulate_adds_and_response_grads_unchanged():
    """accumulate = 1 adds to what is there (exactly 2x after two calls), and the
    response-only backward gives the same bits whether or not the prompt gradients were
    formed."""
    w = configs.SHARE_P256K.with_(P=2100, R=300, chunk=1024, block=128, seed=7201)
    lens = [300]
    G, res, mem, st, prob, run = _setup(w, lens)
    a = run.bwd().numpy()
    dk1, dv1 = _prompt_grads(run, prob)
    dk2, dv2 = _prompt_grads(run, prob, accumulate=1, out=(dk1.clone(), dv1.clone()))
    assert torch.equal(dk2, 2 * dk1) and torch.equal(dv2, 2 * dv1)
    b = run.bwd().numpy()
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def _sampled_keys(w, n):
    """The first and last prompt positions, both sides of the 128-key workgroup boundaries
    next to them and of every chunk boundary, and n seeded positions."""
    rng = np.random.default_rng(w.seed + 77)
    return np.unique(np.concatenate([
        [0, 1, 127, 128, w.P - 129, w.P - 128, w.P - 1],
        np.arange(1, w.n_chunks) * w.chunk, np.arange(1, w.n_chunks) * w.chunk - 1,
        rng.choice(w.P, n, replace=False)]))


def test_full_prompt_short_response_sampled_keys():
    """Every one of the 2,097,152 prompt positions is a key of the launch; a 24-row
    response (144 rows of the packed row stream: two full 64-row stages and a ragged one)
    keeps the oracle's forward over all its rows and heads short.  Sampled positions are
    compared with the oracle, whose O and lse are its own."""
    w = configs.FULL_P2M
    Rs = 24
    print(f"[prompt_grads] {w.name} full prompt, R={Rs}", flush=True)
    G, res, mem, st, prob, run = _setup(w, [Rs])
    dk, dv = _prompt_grads(run, prob)
    keys = _sampled_keys(w, 200)
    f = lambda x: synth.as_f64(x, w.dtype)
    x = {n: f(st[n][0, :Rs]) for n in ("q", "k_r", "v_r", "d_o")}
    kp, vp = f(res["k_p"]), f(res["v_p"])
    o, lse = dense.attend(x["q"], kp, vp, x["k_r"], x["v_r"], w.tau)
    ref_k, ref_v = dense.prompt_grads_given_stats(x["q"], kp, vp, x["d_o"], o, lse, w.tau, keys)
    assert_bf16_close("dk_p sampled", dk[keys].double().cpu().numpy(), ref_k)
    assert_bf16_close("dv_p sampled", dv[keys].double().cpu().numpy(), ref_v)
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all()


def test_full_size_key_sums():
    """The 2M configuration's first member at its seeded length, as the full-sequence
    benchmark launches it, checked through two identities of the exact gradients that need
    no oracle forward over 2M keys.  Per KV head g, over all keys j (prompt and response):
      sum_j dV[j, g] = sum over rows i and heads h of g of dO[i, h]   (each row of P sums to 1)
      sum_j dK[j, g] = 0                                              (each row of dS sums to 0)
    The first is held to the bf16 bounds.  For the second the bf16 rounding of dS before
    its product leaves a residue of about 1e-3 of |dK|; a term dropped over one prompt chunk
    leaves about the square root of the chunk's share of the keys (0.25 for 131,072 of 2M
    keys, 0.125 for 32,768), so the bound is 2e-2 of the norm of all dK rows."""
    w = configs.FULL_P2M
    Rg = int(synth.response_lengths(w)[0])
    print(f"[prompt_grads] {w.name} key sums, R={Rg}", flush=True)
    G, res, mem, st, prob, run = _setup(w, [Rg])
    dk, dv = _prompt_grads(run, prob)
    got = run.bwd().numpy()
    grp = w.Hq // w.Hkv
    d_o = synth.as_f64(st["d_o"][0, :Rg], w.dtype)
    want_v = d_o.reshape(Rg, w.Hkv, grp, w.d_v).sum(axis=(0, 2))
    sum_v = dv.double().sum(0).cpu().numpy() + got["dv"][0][:Rg].sum(0)
    sum_k = dk.double().sum(0).cpu().numpy() + got["dk"][0][:Rg].sum(0)
    assert_bf16_close("sum of dV over all keys", sum_v, want_v)
    norm_k = np.sqrt(float((dk.double() ** 2).sum()) + float(np.sum(got["dk"][0][:Rg] ** 2)))
    resid = float(np.linalg.norm(sum_k)) / norm_k
    print(f"[prompt_grads] |sum dK| / |dK| = {resid:.2e}", flush=True)
    assert resid <= 2e-2
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all()
