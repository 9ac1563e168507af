"""rr_attn_fwd_static, the forward for callers that cannot allocate (needs an MI355X): its
workspace is the library's static device scratch.  Two calls in a row, the second on a
smaller problem (so the scratch still holds the first call's bytes), each equal bit for
bit to rr_attn_fwd with a caller workspace; then a small latent-page call."""
import numpy as np
import pytest
import torch

from resident_kv_response_amd import configs, rr_attn as R, synth

pytestmark = pytest.mark.gpu


def _dense_case(w, lens):
    from tests import _gpu as G
    res = synth.resident(w)
    mem = [synth.member(w, g, R=r) for g, r in enumerate(lens)]
    st = G.stack_members(mem, max(lens))
    prob = G.problem(w.P, max(lens), w.Hq, w.Hkv, w.d_qk, w.chunk, w.block, w.dtype, K=len(lens), tau=w.tau)
    return G.Run(prob, w.dtype, res["k_p"], res["v_p"], st, lens)


def _static_matches(run, extra=None):
    from tests import _gpu as G
    assert R.rr_workspace_bytes(run.p, R.RR_OP_FWD) <= R.RR_STATIC_SCRATCH_BYTES
    ref = run.fwd(**(extra or {}))
    torch.cuda.synchronize()
    want = {"o": run.o.clone(), "lse": run.lse.clone()}
    gd = G.Guarded()
    o = gd.alloc("o", tuple(run.o.shape), torch.float32, float("nan"))
    lse = gd.alloc("lse", tuple(run.lse.shape), torch.float32, float("nan"))
    R.rr_attn_fwd_static(run.p, run.kv, run.q, getattr(run, "k_r", None), getattr(run, "v_r", None), run.r_len,
                         o=o, lse=lse, **(extra or {}))
    gd.check()
    assert torch.equal(o, want["o"]) or np.array_equal(o.cpu().numpy(), want["o"].cpu().numpy(), equal_nan=True)
    assert np.array_equal(lse.cpu().numpy(), want["lse"].cpu().numpy(), equal_nan=True)
    return ref


def test_static_scratch_forward_equals_workspace_forward():
    big = configs.GQA_P128K.with_(P=5000, R=300, Hq=8, Hkv=2, chunk=2048, block=128, seed=4500)
    small = configs.SHARE_P256K.with_(P=1500, R=130, Hq=4, Hkv=1, d_qk=64, d_v=64, chunk=512, block=64,
                                      seed=4501)
    print("[static] first call: bf16 P=5000 R=300", flush=True)
    _static_matches(_dense_case(big, [300]))
    print("[static] second, smaller call: bf16 d=64 K=2 R=[130, 77]", flush=True)
    _static_matches(_dense_case(small, [130, 77]))
    print("[static] third call: fp32 P=700 R=90", flush=True)
    _static_matches(_dense_case(configs.TINY_F32.with_(P=700, R=90, seed=4502), [90]))


def test_static_scratch_latent_forward():
    from tests import _gpu as G
    from tests.test_gpu_sparse import _data
    P, Rr, topk = 2048, 64, 256
    d = _data(4503, P, Rr, integer_index=True)
    prob = G.latent_problem(P, Rr, topk, 32)
    run = G.LatentRun(prob, d["latent_p"], d["k_idx"], d["q"][None], d["latent_r"][None], d["q_idx"][None],
                      d["d_o"][None], [Rr])
    print("[static] latent P=2048 R=64 top-256", flush=True)
    run.fwd()
    torch.cuda.synchronize()
    gd = G.Guarded()
    o = gd.alloc("o", tuple(run.o.shape), torch.float32, float("nan"))
    lse = gd.alloc("lse", tuple(run.lse.shape), torch.float32, float("nan"))
    idx = gd.alloc("topk_idx", tuple(run.idx.shape), torch.int32, -7)
    R.rr_attn_fwd_static(prob, run.kv, run.q, run.latent_r, None, run.r_len, o=o, lse=lse, q_idx=run.q_idx,
                         topk_idx=idx)
    gd.check()
    assert torch.equal(idx, run.idx)
    assert torch.equal(o, run.o) and torch.equal(lse, run.lse)
