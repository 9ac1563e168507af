"""GPU parity of the full-sequence differential mode (needs an MI355X): dk_p, dv_p of the
resident prompt K/V, the term the response-only contract drops, against the fp64 oracle.

Small problems compare every element with the full-sequence oracle (bf16: rel-L2 <= 5e-3
and max-abs <= 2e-2; fp32: max-abs <= 1e-5).  At the full 2,097,152-position size, sampled
prompt positions are compared with the oracle's conditional form, fed the device's O and
lse (which the full-size forward tests validate on sampled rows).
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


def test_full_size_sampled_keys():
    """The 2M configuration's first member at its seeded length: sampled prompt positions
    (the first and last, both sides of every 128-key workgroup boundary nearby and of the
    chunk boundaries) against the conditional oracle over every row of the response."""
    w = configs.FULL_P2M
    Rg = int(synth.response_lengths(w)[0])
    print(f"[prompt_grads] {w.name} full size, R={Rg}", flush=True)
    G, res, mem, st, prob, run = _setup(w, [Rg])
    dk, dv = _prompt_grads(run, prob)
    rng = np.random.default_rng(w.seed + 77)
    keys = np.unique(np.concatenate([
        [0, 1, 127, 128, w.P - 129, w.P - 128, w.P - 1],
        np.arange(1, w.n_chunks) * w.chunk, np.arange(1, w.n_chunks) * w.chunk - 1,
        rng.choice(w.P, 24, replace=False)]))
    f = lambda x: synth.as_f64(x, w.dtype)
    o = run.o[0, :Rg].double().cpu().numpy()
    lse = run.lse[0, :Rg].double().cpu().numpy()
    ref_k, ref_v = dense.prompt_grads_given_stats(f(st["q"][0, :Rg]), f(res["k_p"]), f(res["v_p"]),
                                                  f(st["d_o"][0, :Rg]), o, lse, w.tau, keys)
    assert_bf16_close("dk_p sampled", dk[keys].double().cpu().numpy(), ref_k)
    assert_bf16_close("dv_p sampled", dv[keys].double().cpu().numpy(), ref_v)
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all()
