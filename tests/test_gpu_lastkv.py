"""GPU parity of LastKV chunk recurrence with previous-chunk blending (needs an MI355X).

A sequence is processed chunk by chunk through the C ABI, as replay does: for chunk c the
blend (rr_lastkv_blend) writes K~, V~ of chunk c-1 behind the last-layer history, the
chunk's rows attend with rr_attn_fwd (history = resident keys, the chunk's own K/V =
causal part), and the backward takes rr_attn_bwd (dQ and the chunk's own dK, dV),
rr_attn_prompt_grads over the key range of K~ (and, for the longer gradient path, of the
older history) and rr_lastkv_blend_bwd (both sources of the blend and the gate).
Compared with oracle/lastkv.py on every element: bf16 rel-L2 <= 5e-3 and max-abs <= 2e-2,
fp32 max-abs <= 1e-5.  Sequence lengths C - 1, C, C + 1 and a ragged last chunk cover the
chunk boundaries, including a sequence that ends inside a chunk.
"""
import numpy as np
import pytest
import torch

from oracle import lastkv
from resident_kv_response_amd import rr_attn as R, synth
from tests._helpers import assert_bf16_close, assert_f32_close, rel_l2

pytestmark = pytest.mark.gpu


def _dev(x, dtype):
    from tests import _gpu as G
    return G.to_dev(x, dtype)


class Seq:
    """Device copies of one layer's sequence and the history buffer the chunks read."""

    def __init__(self, x, dtype, tau):
        self.dtype, self.tau = dtype, tau
        self.t = {k: _dev(v, dtype) for k, v in x.items() if k != "alpha"}
        self.alpha = torch.tensor(x["alpha"], device="cuda", dtype=torch.float32)
        self.N, self.Hq, self.d = x["q"].shape
        self.Hkv = x["k_layer"].shape[1]
        # last-layer history with the previous chunk's slot overwritten by its blend
        self.hk = self.t["k_last"].clone()
        self.hv = self.t["v_last"].clone()

    def problem(self, P, n, chunk):
        return R.Problem(P=P, R_max=n, Hq=self.Hq, Hkv=self.Hkv, d_qk=self.d, d_v=self.d, chunk=chunk,
                         block=max(1, min(n, 64)), tau=self.tau,
                         dtype=R.RR_BF16 if self.dtype == "bf16" else R.RR_F32)

    def chunk(self, c, C, chunk=96):
        """Forward of chunk c; returns (problem, resident, row slice, o, lse, ws)."""
        lo, hi = max(c - 1, 0) * C, c * C
        n = min(self.N, hi + C) - hi
        if c >= 1:   # K~, V~ of chunk c-1 into its slot of the history
            R.rr_lastkv_blend(self.alpha, self.t["k_layer"][lo:hi], self.t["k_last"][lo:hi], self.hk[lo:hi])
            R.rr_lastkv_blend(self.alpha, self.t["v_layer"][lo:hi], self.t["v_last"][lo:hi], self.hv[lo:hi])
        prob = self.problem(hi, n, chunk)
        kv = R.resident(self.hk[:hi], self.hv[:hi])
        rows = slice(hi, hi + n)
        o = torch.empty(1, n, self.Hq, self.d, device="cuda")
        lse = torch.empty(1, n, self.Hq, device="cuda")
        ws = R.workspace(prob, R.RR_OP_FWD, "cuda")
        R.rr_attn_fwd(prob, kv, self.q(rows), self.k(rows), self.v(rows), [n], o=o, lse=lse, ws=ws)
        return prob, kv, rows, o, lse

    def restore(self, c, C):
        lo, hi = max(c - 1, 0) * C, c * C
        self.hk[lo:hi].copy_(self.t["k_last"][lo:hi])
        self.hv[lo:hi].copy_(self.t["v_last"][lo:hi])

    def q(self, rows):
        return self.t["q"][rows][None].contiguous()

    def k(self, rows):
        return self.t["k_layer"][rows][None].contiguous()

    def v(self, rows):
        return self.t["v_layer"][rows][None].contiguous()


def _f64(x, dtype):
    return {k: (v.astype(np.float64) if k == "alpha" else synth.as_f64(v, dtype)) for k, v in x.items()}


@pytest.mark.parametrize("dtype,N,C,Hq,Hkv,d", [
    ("bf16", 255, 256, 8, 2, 128),    # C - 1: one partial chunk, no history
    ("bf16", 256, 256, 8, 2, 128),    # C
    ("bf16", 257, 256, 8, 2, 128),    # C + 1: one row after the first boundary
    ("bf16", 805, 256, 8, 2, 128),    # three boundaries, ragged last chunk
    ("bf16", 700, 192, 12, 4, 64),    # d = 64, GQA 3
    ("f32", 63, 64, 4, 1, 64),
    ("f32", 65, 64, 4, 1, 64),
    ("f32", 230, 64, 4, 2, 64),
])
def test_sequence_chunk_by_chunk(dtype, N, C, Hq, Hkv, d):
    x = synth.lastkv_sequence(8000 + N + C + d, N, Hq, Hkv, d, dtype)
    tau = 1.0 / np.sqrt(d)
    s = Seq(x, dtype, tau)
    print(f"[lastkv] {dtype} N={N} C={C} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
    o = np.zeros((N, Hq, d))
    lse = np.zeros((N, Hq))
    for c in range(-(-N // C)):
        prob, kv, rows, oc, lc = s.chunk(c, C)
        torch.cuda.synchronize()
        o[rows] = oc[0].double().cpu().numpy()
        lse[rows] = lc[0].double().cpu().numpy()
        s.restore(c, C)
    xf = _f64(x, dtype)
    ro, rl = lastkv.sequence_attend(xf["q"], xf["k_layer"], xf["v_layer"], xf["k_last"], xf["v_last"],
                                    xf["alpha"], C, tau)
    if dtype == "f32":
        assert_f32_close("o", o, ro)
        assert_f32_close("lse", lse, rl)
    else:
        assert_bf16_close("o", o, ro)
        assert np.max(np.abs(lse - rl)) <= 2e-2


@pytest.mark.parametrize("dtype,N,C,c,Hq,Hkv,d", [
    ("bf16", 805, 256, 3, 8, 2, 128),   # ragged last chunk, two older chunks of history
    ("bf16", 600, 192, 1, 12, 4, 64),   # the first chunk with a blended predecessor
    ("f32", 230, 64, 2, 4, 2, 64),
])
def test_chunk_backward(dtype, N, C, c, Hq, Hkv, d):
    x = synth.lastkv_sequence(9000 + N + c, N, Hq, Hkv, d, dtype)
    tau = 1.0 / np.sqrt(d)
    s = Seq(x, dtype, tau)
    print(f"[lastkv bwd] {dtype} N={N} C={C} c={c}", flush=True)
    prob, kv, rows, o, lse = s.chunk(c, C)
    n = rows.stop - rows.start
    lo, hi = max(c - 1, 0) * C, c * C
    f32 = dict(device="cuda", dtype=torch.float32)
    d_o = s.t["d_o"][rows][None].contiguous()
    dq = torch.empty(1, n, Hq, d, **f32)
    dk = torch.empty(1, n, Hkv, d, **f32)
    dv = torch.empty(1, n, Hkv, d, **f32)
    R.rr_attn_bwd(prob, kv, s.q(rows), s.k(rows), s.v(rows), [n], o, lse, d_o, dq, dk, dv,
                  ws=R.workspace(prob, R.RR_OP_BWD, "cuda"))
    ws_pg = R.workspace(prob, R.RR_OP_PROMPT_GRADS, "cuda")
    dkb = torch.empty(hi - lo, Hkv, d, **f32)
    dvb = torch.empty(hi - lo, Hkv, d, **f32)
    R.rr_attn_prompt_grads(prob, kv, s.q(rows), [n], o, lse, d_o, dkb, dvb, key_range=(lo, hi), ws=ws_pg)
    dkh = torch.empty(max(lo, 1), Hkv, d, **f32)
    dvh = torch.empty(max(lo, 1), Hkv, d, **f32)
    R.rr_attn_prompt_grads(prob, kv, s.q(rows), [n], o, lse, d_o, dkh, dvh, key_range=(0, lo), ws=ws_pg)
    grads = {k: torch.zeros(hi - lo, Hkv, d, **f32) for k in ("dk_prev_layer", "dk_prev_last",
                                                              "dv_prev_layer", "dv_prev_last")}
    d_alpha = torch.zeros(Hkv, **f32)
    R.rr_lastkv_blend_bwd(s.alpha, s.t["k_layer"][lo:hi], s.t["k_last"][lo:hi], dkb, grads["dk_prev_layer"],
                          grads["dk_prev_last"], d_alpha, accumulate=1)
    R.rr_lastkv_blend_bwd(s.alpha, s.t["v_layer"][lo:hi], s.t["v_last"][lo:hi], dvb, grads["dv_prev_layer"],
                          grads["dv_prev_last"], d_alpha, accumulate=1)
    torch.cuda.synchronize()
    xf = _f64(x, dtype)
    ref = lastkv.chunk_attend_bwd(xf["q"][rows], xf["d_o"][rows], xf["k_layer"], xf["v_layer"], xf["k_last"],
                                  xf["v_last"], xf["alpha"], C, c, tau)
    got = {"dq": dq[0], "dk_c": dk[0], "dv_c": dv[0], "dk_hist": dkh[:lo], "dv_hist": dvh[:lo], **grads}
    close = assert_f32_close if dtype == "f32" else assert_bf16_close
    for key, val in got.items():
        close(key, val.double().cpu().numpy(), ref[key])
    da = d_alpha.double().cpu().numpy()
    assert rel_l2(da, ref["d_alpha"]) <= (1e-5 if dtype == "f32" else 5e-3), (da, ref["d_alpha"])


def test_blend_matches_its_definition():
    """Every element of the blend: fp32 arithmetic rounded once to the stored dtype, within
    one rounding of the exact blend plus the fp32 error of the two products."""
    for dtype in ("bf16", "f32"):
        x = synth.lastkv_sequence(9901, 300, 4, 4, 128, dtype)
        s = Seq(x, dtype, 0.1)
        out = torch.empty_like(s.t["k_layer"])
        R.rr_lastkv_blend(s.alpha, s.t["k_layer"], s.t["k_last"], out)
        torch.cuda.synchronize()
        xf = _f64(x, dtype)
        ref = lastkv.blend(xf["k_layer"], xf["k_last"], xf["alpha"])
        got = out.double().cpu().numpy()
        # one rounding of the stored value plus fp32 arithmetic error (cancellation near 0)
        scale = np.abs(xf["k_layer"]) + np.abs(xf["k_last"])
        tol = np.abs(ref) * (2.0 ** -8 if dtype == "bf16" else 2.0 ** -22) + 2.0 ** -20 * scale
        assert np.all(np.abs(got - ref) <= tol)
