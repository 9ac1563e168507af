"""GPU-side helpers for the parity tests: numpy inputs -> device tensors -> the C ABI.

Everything here is marshalling; the computation runs in librr_attn.so.
"""
from __future__ import annotations

import numpy as np
import torch

from resident_kv_response_amd import rr_attn as R
from resident_kv_response_amd.synth import as_f64

DEV = "cuda"


GUARD = 64 << 10        # bytes of canary before and after every guarded output
CANARY = 0xA5


class Guarded:
    """Output buffers placed between canary regions: each tensor is a view into a larger
    byte buffer whose GUARD bytes before and after it hold CANARY.  check() fails if any
    kernel wrote outside its output."""

    def __init__(self):
        self.bufs = []

    def alloc(self, name, shape, dtype, fill=None):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        raw = torch.full((n + 2 * GUARD,), CANARY, dtype=torch.uint8, device=DEV)
        t = raw[GUARD:GUARD + n].view(dtype).view(shape)
        if fill is not None:
            t.fill_(fill)
        self.bufs.append((name, raw, n))
        return t

    def workspace(self, p, op):
        return self.alloc(f"ws{op}", (max(1, R.rr_workspace_bytes(p, op)),), torch.uint8)

    def check(self):
        torch.cuda.synchronize()
        for name, raw, n in self.bufs:
            head, tail = raw[:GUARD], raw[GUARD + n:]
            assert bool(torch.all(head == CANARY)) and bool(torch.all(tail == CANARY)), \
                f"a kernel wrote outside {name}"


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def stack_members(members, R_max, keys=("q", "k_r", "v_r", "d_o")):
    """Stack per-member arrays [R_g][...] into [K][R_max][...], zero-padded."""
    out = {}
    for key in keys:
        first = members[0][key]
        arr = np.zeros((len(members), R_max) + first.shape[1:], dtype=first.dtype)
        for i, m in enumerate(members):
            arr[i, :m[key].shape[0]] = m[key]
        out[key] = arr
    return out


def problem(P, R_max, Hq, Hkv, d, chunk, block, dtype, K=1, tau=None):
    return R.Problem(P=P, R_max=R_max, Hq=Hq, Hkv=Hkv, d_qk=d, d_v=d, chunk=chunk, block=block,
                     tau=float(tau if tau is not None else 1.0 / np.sqrt(d)),
                     dtype=R.RR_BF16 if dtype == "bf16" else R.RR_F32, K=K)


def ws_D(ws, p):
    """D = dO . O [K][R_max][Hq] fp32, which rr_attn_bwd leaves at the head of its workspace."""
    n = p.K * p.R_max * p.Hq
    return ws[:4 * n].view(torch.float32).reshape(p.K, p.R_max, p.Hq).double().cpu().numpy()


class Run:
    """Device copies of one problem's inputs plus its outputs."""

    def __init__(self, prob: R.Problem, dtype: str, k_p, v_p, stacked, r_len, version=0, dev_resident=None):
        self.p, self.dtype, self.r_len = prob, dtype, [int(x) for x in r_len]
        if dev_resident is not None:     # device copies shared with other runs (one prompt group)
            self.k_p, self.v_p = dev_resident
        else:
            self.k_p, self.v_p = to_dev(k_p, dtype), to_dev(v_p, dtype)
        self.q = to_dev(stacked["q"], dtype)
        self.k_r = to_dev(stacked["k_r"], dtype)
        self.v_r = to_dev(stacked["v_r"], dtype)
        self.d_o = to_dev(stacked["d_o"], dtype)
        self.kv = R.resident(self.k_p, self.v_p, version=version)
        K, Rm, Hq, d = prob.K, prob.R_max, prob.Hq, prob.d_qk
        self.guard = gd = Guarded()
        nan, f = float("nan"), torch.float32
        self.o = gd.alloc("o", (K, Rm, Hq, prob.d_v), f, nan)
        self.lse = gd.alloc("lse", (K, Rm, Hq), f, nan)
        self.dq = gd.alloc("dq", (K, Rm, Hq, d), f, nan)
        self.dk = gd.alloc("dk_r", (K, Rm, prob.Hkv, d), f, nan)
        self.dv = gd.alloc("dv_r", (K, Rm, prob.Hkv, prob.d_v), f, nan)
        self.ws_f = gd.workspace(prob, R.RR_OP_FWD)
        self.ws_b = gd.workspace(prob, R.RR_OP_BWD)

    def fwd(self, **kw):
        R.rr_attn_fwd(self.p, self.kv, self.q, self.k_r, self.v_r, self.r_len, o=self.o, lse=self.lse,
                      ws=self.ws_f, **kw)
        return self

    def bwd(self, accumulate=0, block_idx=-1):
        self.tag = R.rr_attn_bwd(self.p, self.kv, self.q, self.k_r, self.v_r, self.r_len, self.o, self.lse,
                                 self.d_o, self.dq, self.dk, self.dv, accumulate=accumulate,
                                 block_idx=block_idx, ws=self.ws_b)
        return self

    def numpy(self):
        """Outputs, and D = dO . O [K][R_max][Hq] from the head of the backward's workspace;
        first checks that no kernel wrote outside an output or a workspace."""
        self.guard.check()
        out = {k: getattr(self, k).double().cpu().numpy() for k in ("o", "lse", "dq", "dk", "dv")}
        out["D"] = ws_D(self.ws_b, self.p)
        return out


def oracle_member(dense, dtype, k_p, v_p, stacked, kk, rl, tau, rows=None, grads=True):
    """Oracle of member kk (its first rl rows) in fp64 from the identical stored values."""
    f = lambda x: as_f64(x, dtype)
    q, kr, vr, do = (f(stacked[n][kk, :rl]) for n in ("q", "k_r", "v_r", "d_o"))
    kp, vp = f(k_p), f(v_p)
    o, lse = dense.attend(q, kp, vp, kr, vr, tau, rows=rows)
    out = {"o": o, "lse": lse}
    if grads:
        out.update(dense.attend_bwd(q, kp, vp, kr, vr, do, tau, rows=rows))
    return out


class LatentRun:
    """Device copies of a latent-page problem (one or more responses) and its outputs."""

    def __init__(self, prob, latent_p, k_idx, q, latent_r, q_idx, d_o, r_len):
        self.p, self.r_len = prob, [int(x) for x in r_len]
        self.latent_p = to_dev(latent_p, "bf16")
        self.k_idx = to_dev(k_idx, "f32")
        self.q, self.latent_r, self.d_o = to_dev(q, "bf16"), to_dev(latent_r, "bf16"), to_dev(d_o, "bf16")
        self.q_idx = to_dev(q_idx, "f32")
        self.kv = R.resident(self.latent_p, None, version=0, k_idx=self.k_idx)
        K, Rm = prob.K, prob.R_max
        self.guard = gd = Guarded()
        nan, f = float("nan"), torch.float32
        self.o = gd.alloc("o", (K, Rm, prob.Hq, prob.d_v), f, nan)
        self.lse = gd.alloc("lse", (K, Rm, prob.Hq), f, nan)
        self.idx = gd.alloc("topk_idx", (K, Rm, prob.topk), torch.int32, -7)
        self.dq = gd.alloc("dq", (K, Rm, prob.Hq, prob.d_qk), f, nan)
        self.dk = gd.alloc("dk_r", (K, Rm, prob.d_qk), f, nan)
        self.dv = gd.alloc("dv_r", (K, Rm, prob.d_v), f, nan)
        self.ws_f = gd.workspace(prob, R.RR_OP_FWD)
        self.ws_b = gd.workspace(prob, R.RR_OP_BWD)

    def fwd(self):
        R.rr_attn_fwd(self.p, self.kv, self.q, self.latent_r, None, self.r_len, o=self.o, lse=self.lse,
                      q_idx=self.q_idx, topk_idx=self.idx, ws=self.ws_f)
        return self

    def bwd(self, accumulate=0, block_idx=-1):
        self.tag = R.rr_attn_bwd(self.p, self.kv, self.q, self.latent_r, None, self.r_len, self.o, self.lse,
                                 self.d_o, self.dq, self.dk, self.dv, accumulate=accumulate,
                                 block_idx=block_idx, topk_idx=self.idx, ws=self.ws_b)
        return self

    def numpy(self):
        self.guard.check()
        out = {k: getattr(self, k).double().cpu().numpy() for k in ("o", "lse", "dq", "dk", "dv")}
        out["idx"] = self.idx.cpu().numpy()
        out["D"] = ws_D(self.ws_b, self.p)
        return out


def latent_problem(P, R_max, topk, block, K=1):
    return R.Problem(P=P, R_max=R_max, Hq=64, Hkv=1, d_qk=576, d_v=512, chunk=P, block=block,
                     tau=float(1.0 / np.sqrt(576)), dtype=R.RR_BF16, K=K, topk=topk, idx_dim=128, latent=1)
