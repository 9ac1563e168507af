"""Context-parallel composition on one GPU (needs an MI355X): the prompt split into two
shards, each attended by its own call, partials exported and merged by rr_lse_merge
(the rank-local softmax statistics composed into the exact global output); the backward
run per shard with the merged statistics, dQ summed over shards, and the response dK/dV
formed once by the shard that owns the response keys."""
import numpy as np
import pytest
import torch

from oracle import dense
from resident_kv_response_amd import configs, rr_attn as R, synth
from tests._helpers import assert_bf16_close

pytestmark = pytest.mark.gpu


def _shard_run(w, rows_check=None):
    from tests import _gpu as G
    res = synth.resident(w)
    m = synth.member(w, 0)
    st = G.stack_members([m], w.R)
    full_p = G.problem(w.P, w.R, w.Hq, w.Hkv, w.d_qk, w.chunk, w.block, w.dtype, tau=w.tau)
    full = G.Run(full_p, w.dtype, res["k_p"], res["v_p"], st, [w.R]).fwd().bwd()
    ref_full = full.numpy()
    cut = w.P // 2 + 123                      # uneven shards
    shards = [(0, cut, R.RR_FLAG_SHARD_NO_RESPONSE), (cut, w.P, 0)]
    runs, parts_o, parts_l = [], [], []
    for lo, hi, flags in shards:
        p = G.problem(hi - lo, w.R, w.Hq, w.Hkv, w.d_qk, w.chunk, w.block, w.dtype, tau=w.tau)
        p.flags = flags
        run = G.Run(p, w.dtype, res["k_p"][lo:hi], res["v_p"][lo:hi], st, [w.R])
        n = R.rr_num_parts(p)
        po = torch.empty((n, 1, w.R, w.Hq, w.d_v), device="cuda")
        pl = torch.empty((n, 1, w.R, w.Hq), device="cuda")
        R.rr_attn_fwd(p, run.kv, run.q, run.k_r, run.v_r, [w.R], part_o=po, part_lse=pl, ws=run.ws_f)
        parts_o.append(po)
        parts_l.append(pl)
        runs.append((p, run))
    po = torch.cat(parts_o)
    pl = torch.cat(parts_l)
    o = torch.empty((1, w.R, w.Hq, w.d_v), device="cuda")
    lse = torch.empty((1, w.R, w.Hq), device="cuda")
    R.rr_lse_merge(po, pl, o, lse)
    dq_sum = torch.zeros((1, w.R, w.Hq, w.d_qk), device="cuda")
    dk = dv = None
    for (p, run), (lo, hi, flags) in zip(runs, shards):
        dq = torch.empty_like(dq_sum)
        if flags:
            R.rr_attn_bwd(p, run.kv, run.q, run.k_r, run.v_r, [w.R], o, lse, run.d_o, dq, None, None,
                          ws=run.ws_b)
        else:
            dk = torch.empty((1, w.R, w.Hkv, w.d_qk), device="cuda")
            dv = torch.empty((1, w.R, w.Hkv, w.d_v), device="cuda")
            R.rr_attn_bwd(p, run.kv, run.q, run.k_r, run.v_r, [w.R], o, lse, run.d_o, dq, dk, dv,
                          ws=run.ws_b)
        dq_sum += dq
    torch.cuda.synchronize()
    got = {"o": o.double().cpu().numpy(), "lse": lse.double().cpu().numpy(),
           "dq": dq_sum.double().cpu().numpy(), "dk": dk.double().cpu().numpy(),
           "dv": dv.double().cpu().numpy()}
    # against the single-call path
    for key in ("o", "dq", "dk", "dv"):
        assert_bf16_close(f"shards vs single {key}", got[key], ref_full[key], rl2=2e-3, mabs=1e-2)
    assert np.max(np.abs(got["lse"] - ref_full["lse"])) < 1e-3
    # against the oracle
    ref = G.oracle_member(dense, w.dtype, res["k_p"], res["v_p"], st, 0, w.R, w.tau, rows=rows_check)
    sel = slice(None) if rows_check is None else rows_check
    assert_bf16_close("o", got["o"][0][sel], ref["o"])
    assert_bf16_close("dq", got["dq"][0][sel], ref["dq"])
    if rows_check is None:
        assert_bf16_close("dk", got["dk"][0], ref["dk_r"])
        assert_bf16_close("dv", got["dv"][0], ref["dv_r"])


def test_two_shards_compose_exactly_small():
    w = configs.SHARE_P256K.with_(P=6000, R=700, chunk=1024, block=256, seed=7001)
    print("[shards] small", flush=True)
    _shard_run(w)


def test_two_shards_compose_exactly_one_rank_share():
    w = configs.SHARE_P256K
    rows = synth.sample_rows(w.seed, w.R, 16, w.block)
    print("[shards] one-rank share, full size", flush=True)
    _shard_run(w, rows_check=rows)
