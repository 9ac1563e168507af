"""ctypes binding of librr_attn.so (include/rr_attn.h).

Argument marshalling only: torch tensors become device pointers, the current HIP stream
becomes the stream handle, and a non-zero return code becomes an RRError carrying the
library's message.  Every computation runs in the library's HIP kernels; there is no
fallback: if the library is not built, loading it raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librr_attn.so")

RR_OK = 0
RR_E_NULL, RR_E_SHAPE, RR_E_UNSUPPORTED, RR_E_WORKSPACE = -1, -2, -3, -4
RR_E_RANGE, RR_E_DUPLICATE, RR_E_STALE, RR_E_MISSING, RR_E_HIP, RR_E_PTR = -5, -6, -7, -8, -9, -10
RR_E_POISONED = -11
RR_F32, RR_BF16 = 0, 1
RR_OP_FWD, RR_OP_BWD, RR_OP_PROMPT_GRADS = 0, 1, 2
RR_MAX_K, RR_MAX_ACC = 64, 8
RR_FLAG_SHARD_NO_RESPONSE = 1

RR_STATIC_SCRATCH_BYTES = 64 << 20

EXPORTS = ["rr_workspace_bytes", "rr_num_parts", "rr_attn_fwd", "rr_lse_merge", "rr_attn_bwd",
           "rr_attn_prompt_grads", "rr_lastkv_blend", "rr_lastkv_blend_bwd", "rr_grad_accum",
           "rr_accum_check_complete", "rr_attn_fwd_static", "rr_last_error", "rr_profile_begin",
           "rr_profile_end"]


class RRError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"rr_attn error {code}: {msg}")
        self.code = code


class CProblem(ctypes.Structure):
    _fields_ = [("P", ctypes.c_int64), ("chunk", ctypes.c_int64), ("R_max", ctypes.c_int32),
                ("K", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32), ("block", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("idx_dim", ctypes.c_int32), ("latent", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("tau", ctypes.c_float), ("flags", ctypes.c_int32)]


class CResident(ctypes.Structure):
    _fields_ = [("k_p", ctypes.c_void_p), ("v_p", ctypes.c_void_p), ("k_idx", ctypes.c_void_p),
                ("P", ctypes.c_int64), ("version", ctypes.c_uint64)]


class CGradTag(ctypes.Structure):
    _fields_ = [("version", ctypes.c_uint64), ("resident", ctypes.c_void_p), ("P", ctypes.c_int64),
                ("seal", ctypes.c_uint64)]


class CAccum(ctypes.Structure):
    _fields_ = [("n_bufs", ctypes.c_int32), ("buf", ctypes.c_void_p * RR_MAX_ACC),
                ("n", ctypes.c_int64 * RR_MAX_ACC), ("G", ctypes.c_int32),
                ("version", ctypes.c_uint64), ("seen", ctypes.POINTER(ctypes.c_uint8)),
                ("resident", ctypes.c_void_p), ("resident_P", ctypes.c_int64), ("poisoned", ctypes.c_int32)]


class CProfileEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load librr_attn.so (built in-tree by resident_kv_response_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m resident_kv_response_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.rr_workspace_bytes.argtypes = [ctypes.POINTER(CProblem), ctypes.c_int]
        L.rr_workspace_bytes.restype = sz
        L.rr_num_parts.argtypes = [ctypes.POINTER(CProblem)]
        L.rr_num_parts.restype = i32
        L.rr_attn_fwd.argtypes = [ctypes.POINTER(CProblem), ctypes.POINTER(CResident), vp, vp, vp,
                                  ctypes.POINTER(i32), vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.rr_attn_fwd.restype = ctypes.c_int
        L.rr_attn_fwd_static.argtypes = [ctypes.POINTER(CProblem), ctypes.POINTER(CResident), vp, vp, vp,
                                         ctypes.POINTER(i32), vp, vp, vp, vp, vp, vp, vp]
        L.rr_attn_fwd_static.restype = ctypes.c_int
        L.rr_lse_merge.argtypes = [i32, i64, i32, vp, vp, vp, vp, vp]
        L.rr_lse_merge.restype = ctypes.c_int
        L.rr_attn_bwd.argtypes = [ctypes.POINTER(CProblem), ctypes.POINTER(CResident), vp, vp, vp,
                                  ctypes.POINTER(i32), vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, sz,
                                  ctypes.POINTER(CGradTag), vp]
        L.rr_attn_bwd.restype = ctypes.c_int
        L.rr_attn_prompt_grads.argtypes = [ctypes.POINTER(CProblem), ctypes.POINTER(CResident), vp,
                                           ctypes.POINTER(i32), vp, vp, vp, i64, i64, vp, vp, i32, vp, sz,
                                           vp]
        L.rr_attn_prompt_grads.restype = ctypes.c_int
        L.rr_lastkv_blend.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp, vp]
        L.rr_lastkv_blend.restype = ctypes.c_int
        L.rr_lastkv_blend_bwd.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp]
        L.rr_lastkv_blend_bwd.restype = ctypes.c_int
        L.rr_grad_accum.argtypes = [ctypes.POINTER(CAccum), i32, ctypes.POINTER(CGradTag),
                                    ctypes.POINTER(vp), ctypes.POINTER(i64), ctypes.c_float, vp]
        L.rr_grad_accum.restype = ctypes.c_int
        L.rr_accum_check_complete.argtypes = [ctypes.POINTER(CAccum)]
        L.rr_accum_check_complete.restype = ctypes.c_int
        L.rr_last_error.argtypes = []
        L.rr_last_error.restype = ctypes.c_char_p
        L.rr_profile_begin.argtypes = []
        L.rr_profile_begin.restype = ctypes.c_int
        L.rr_profile_end.argtypes = [ctypes.POINTER(CProfileEntry), i32, ctypes.POINTER(i32)]
        L.rr_profile_end.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != RR_OK:
        raise RRError(rc, lib().rr_last_error().decode(errors="replace"))


@dataclasses.dataclass
class Problem:
    """Mirror of rr_problem."""
    P: int
    R_max: int
    Hq: int
    Hkv: int
    d_qk: int
    d_v: int
    chunk: int
    block: int
    tau: float
    dtype: int = RR_BF16
    K: int = 1
    topk: int = 0
    idx_dim: int = 0
    latent: int = 0
    flags: int = 0

    def c(self) -> CProblem:
        return CProblem(P=self.P, chunk=self.chunk, R_max=self.R_max, K=self.K, Hq=self.Hq,
                        Hkv=self.Hkv, d_qk=self.d_qk, d_v=self.d_v, block=self.block, topk=self.topk,
                        idx_dim=self.idx_dim, latent=self.latent, dtype=self.dtype, tau=self.tau,
                        flags=self.flags)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("rr_attn tensors must be GPU tensors (a host pointer would fault in a kernel)")
    if not t.is_contiguous():
        raise ValueError("rr_attn tensors must be contiguous")
    return t.data_ptr()


def _need(name: str, t: Optional[torch.Tensor], dtype: torch.dtype, numel: int) -> None:
    """Refuse a tensor whose dtype differs from the layout the library reads or writes for
    it (include/rr_attn.h), or that holds fewer elements than the layout: a kernel would
    read or write past its end.  NULL (None) is left to the library's own checks."""
    if t is None:
        return
    if t.dtype != dtype:
        raise ValueError(f"rr_attn: {name} has dtype {t.dtype}, the layout needs {dtype}")
    if t.numel() < numel:
        raise ValueError(f"rr_attn: {name} has {t.numel()} elements, the layout needs {numel}")


def _elem(p: "Problem") -> torch.dtype:
    return torch.bfloat16 if p.dtype == RR_BF16 else torch.float32


def _need_r_len(p: "Problem", r_len) -> None:
    if len(r_len) != p.K:
        raise ValueError(f"rr_attn: r_len has {len(r_len)} entries, the problem has K = {p.K}")


def _need_resident(p: "Problem", kv: "CResident") -> None:
    """Resident tensors built by resident(): element type and row width against p."""
    meta = getattr(kv, "_meta", None)
    if meta is None:
        return
    rows = max(int(kv.P), 0)

    def need(name, got, dtype, n):
        if got is not None and (got[0] != dtype or got[1] < n):
            raise ValueError(f"rr_attn: resident {name} has {got[1]} elements of {got[0]}, "
                             f"the layout needs {n} of {dtype}")

    need("k_p", meta[0], _elem(p), rows * (p.d_qk if p.latent else p.Hkv * p.d_qk))
    if not p.latent:
        need("v_p", meta[1], _elem(p), rows * p.Hkv * p.d_v)
    if p.topk > 0:
        need("k_idx", meta[2], torch.float32, rows * p.idx_dim)


def _need_rows(p: "Problem", q=None, k_r=None, v_r=None, d_o=None, o=None, lse=None, dq=None, dk_r=None,
               dv_r=None, q_idx=None, topk_idx=None) -> None:
    KR = p.K * p.R_max
    et = _elem(p)
    kw = p.d_qk if p.latent else p.Hkv * p.d_qk
    vw = p.d_v if p.latent else p.Hkv * p.d_v
    _need("q", q, et, KR * p.Hq * p.d_qk)
    _need("k_r", k_r, et, KR * kw)
    if not p.latent:
        _need("v_r", v_r, et, KR * vw)
    _need("d_o", d_o, et, KR * p.Hq * p.d_v)
    _need("o", o, torch.float32, KR * p.Hq * p.d_v)
    _need("lse", lse, torch.float32, KR * p.Hq)
    _need("dq", dq, torch.float32, KR * p.Hq * p.d_qk)
    _need("dk_r", dk_r, torch.float32, KR * kw)
    _need("dv_r", dv_r, torch.float32, KR * vw)
    _need("q_idx", q_idx, torch.float32, KR * p.idx_dim)
    _need("topk_idx", topk_idx, torch.int32, KR * p.topk)


def _need_ws(ws: Optional[torch.Tensor]) -> int:
    if ws is None:
        return 0
    if ws.dtype != torch.uint8:
        raise ValueError(f"rr_attn: workspace has dtype {ws.dtype}, expected torch.uint8")
    return ws.numel()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _r_len(r_len: Sequence[int]):
    arr = (ctypes.c_int32 * len(r_len))(*[int(x) for x in r_len])
    return arr


def resident(k_p: torch.Tensor, v_p: Optional[torch.Tensor], version: int = 0,
             k_idx: Optional[torch.Tensor] = None) -> CResident:
    kv = CResident(k_p=_ptr(k_p), v_p=_ptr(v_p), k_idx=_ptr(k_idx), P=k_p.shape[0], version=version)
    kv._meta = ((k_p.dtype, k_p.numel()), None if v_p is None else (v_p.dtype, v_p.numel()),
                None if k_idx is None else (k_idx.dtype, k_idx.numel()))
    return kv


def rr_workspace_bytes(p: Problem, op: int) -> int:
    cp = p.c()
    n = lib().rr_workspace_bytes(ctypes.byref(cp), op)
    if n == 0:
        msg = lib().rr_last_error().decode()
        if msg:
            raise RRError(RR_E_SHAPE, msg)
    return int(n)


def rr_num_parts(p: Problem) -> int:
    cp = p.c()
    n = lib().rr_num_parts(ctypes.byref(cp))
    if n == 0:
        raise RRError(RR_E_SHAPE, lib().rr_last_error().decode())
    return int(n)


def workspace(p: Problem, op: int, device) -> torch.Tensor:
    return torch.empty(max(1, rr_workspace_bytes(p, op)), dtype=torch.uint8, device=device)


def rr_attn_fwd(p: Problem, kv: CResident, q, k_r, v_r, r_len, o=None, lse=None, part_o=None,
                part_lse=None, q_idx=None, topk_idx=None, ws=None, stream=None) -> None:
    _need_r_len(p, r_len)
    _need_resident(p, kv)
    _need_rows(p, q=q, k_r=k_r, v_r=v_r, o=o, lse=lse, q_idx=q_idx, topk_idx=topk_idx)
    if part_o is not None or part_lse is not None:
        n = rr_num_parts(p) * p.K * p.R_max * p.Hq
        _need("part_o", part_o, torch.float32, n * p.d_v)
        _need("part_lse", part_lse, torch.float32, n)
    cp = p.c()
    nbytes = _need_ws(ws)
    _check(lib().rr_attn_fwd(ctypes.byref(cp), ctypes.byref(kv), _ptr(q), _ptr(k_r), _ptr(v_r),
                             _r_len(r_len), _ptr(q_idx), _ptr(o), _ptr(lse), _ptr(part_o),
                             _ptr(part_lse), _ptr(topk_idx), _ptr(ws), nbytes, _stream(stream)))


def rr_attn_fwd_static(p: Problem, kv: CResident, q, k_r, v_r, r_len, o=None, lse=None, part_o=None,
                       part_lse=None, q_idx=None, topk_idx=None, stream=None) -> None:
    """rr_attn_fwd with the library's static device scratch as workspace (allocates
    nothing; problems whose workspace exceeds RR_STATIC_SCRATCH_BYTES are refused)."""
    _need_r_len(p, r_len)
    _need_resident(p, kv)
    _need_rows(p, q=q, k_r=k_r, v_r=v_r, o=o, lse=lse, q_idx=q_idx, topk_idx=topk_idx)
    if part_o is not None or part_lse is not None:
        n = rr_num_parts(p) * p.K * p.R_max * p.Hq
        _need("part_o", part_o, torch.float32, n * p.d_v)
        _need("part_lse", part_lse, torch.float32, n)
    cp = p.c()
    _check(lib().rr_attn_fwd_static(ctypes.byref(cp), ctypes.byref(kv), _ptr(q), _ptr(k_r), _ptr(v_r),
                                    _r_len(r_len), _ptr(q_idx), _ptr(o), _ptr(lse), _ptr(part_o),
                                    _ptr(part_lse), _ptr(topk_idx), _stream(stream)))


def rr_lse_merge(part_o, part_lse, o, lse, stream=None) -> None:
    n_parts, rows, d_v = part_o.shape[0], part_lse[0].numel(), part_o.shape[-1]
    _need("part_o", part_o, torch.float32, n_parts * rows * d_v)
    _need("part_lse", part_lse, torch.float32, n_parts * rows)
    _need("o", o, torch.float32, rows * d_v)
    _need("lse", lse, torch.float32, rows)
    _check(lib().rr_lse_merge(n_parts, rows, d_v, _ptr(part_o), _ptr(part_lse), _ptr(o), _ptr(lse),
                              _stream(stream)))


def rr_attn_bwd(p: Problem, kv: CResident, q, k_r, v_r, r_len, o, lse, d_o, dq, dk_r, dv_r,
                accumulate: int = 0, block_idx: int = -1, topk_idx=None, ws=None,
                stream=None) -> CGradTag:
    """Response-only backward.  Returns the gradient tag (the identity of kv) that
    rr_grad_accum checks against its window."""
    _need_r_len(p, r_len)
    _need_resident(p, kv)
    _need_rows(p, q=q, k_r=k_r, v_r=v_r, d_o=d_o, o=o, lse=lse, dq=dq, dk_r=dk_r, dv_r=dv_r,
               topk_idx=topk_idx)
    cp = p.c()
    nbytes = _need_ws(ws)
    tag = CGradTag()
    _check(lib().rr_attn_bwd(ctypes.byref(cp), ctypes.byref(kv), _ptr(q), _ptr(k_r), _ptr(v_r),
                             _r_len(r_len), _ptr(topk_idx), _ptr(o), _ptr(lse), _ptr(d_o), _ptr(dq),
                             _ptr(dk_r), _ptr(dv_r), int(accumulate), int(block_idx), _ptr(ws),
                             nbytes, ctypes.byref(tag), _stream(stream)))
    return tag


def rr_attn_prompt_grads(p: Problem, kv: CResident, q, r_len, o, lse, d_o, dk_p, dv_p,
                         accumulate: int = 0, key_range=None, ws=None, stream=None) -> None:
    """Full-sequence differential mode: dk_p, dv_p [key_hi - key_lo][Hkv][d] fp32 of the
    resident positions in key_range (default: the whole prompt), the prompt-side term
    that rr_attn_bwd drops."""
    _need_r_len(p, r_len)
    _need_resident(p, kv)
    _need_rows(p, q=q, d_o=d_o, o=o, lse=lse)
    lo, hi = key_range if key_range is not None else (0, p.P)
    _need("dk_p", dk_p, torch.float32, max(hi - lo, 0) * p.Hkv * p.d_qk)
    _need("dv_p", dv_p, torch.float32, max(hi - lo, 0) * p.Hkv * p.d_v)
    cp = p.c()
    nbytes = _need_ws(ws)
    _check(lib().rr_attn_prompt_grads(ctypes.byref(cp), ctypes.byref(kv), _ptr(q), _r_len(r_len),
                                      _ptr(o), _ptr(lse), _ptr(d_o), int(lo), int(hi), _ptr(dk_p),
                                      _ptr(dv_p), int(accumulate), _ptr(ws), nbytes, _stream(stream)))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return RR_BF16
    if t.dtype == torch.float32:
        return RR_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def rr_lastkv_blend(alpha, x_layer, x_last, x_out, stream=None) -> None:
    """x_out = (1 - alpha_g) x_layer + alpha_g x_last over [rows][Hkv][d] (LastKV
    previous-chunk blending)."""
    rows, Hkv, d = x_layer.shape
    n = rows * Hkv * d
    _need("alpha", alpha, torch.float32, Hkv)
    _need("x_last", x_last, x_layer.dtype, n)
    _need("x_out", x_out, x_layer.dtype, n)
    _check(lib().rr_lastkv_blend(rows, Hkv, d, _dtype_code(x_layer), _ptr(alpha), _ptr(x_layer),
                                 _ptr(x_last), _ptr(x_out), _stream(stream)))


def rr_lastkv_blend_bwd(alpha, x_layer, x_last, d_out, d_layer, d_last, d_alpha, accumulate: int = 0,
                        stream=None) -> None:
    rows, Hkv, d = x_layer.shape
    n = rows * Hkv * d
    _need("alpha", alpha, torch.float32, Hkv)
    _need("x_last", x_last, x_layer.dtype, n)
    _need("d_out", d_out, torch.float32, n)
    _need("d_layer", d_layer, torch.float32, n)
    _need("d_last", d_last, torch.float32, n)
    _need("d_alpha", d_alpha, torch.float32, Hkv)
    _check(lib().rr_lastkv_blend_bwd(rows, Hkv, d, _dtype_code(x_layer), _ptr(alpha), _ptr(x_layer),
                                     _ptr(x_last), _ptr(d_out), _ptr(d_layer), _ptr(d_last), _ptr(d_alpha),
                                     int(accumulate), _stream(stream)))


class Accum:
    """Host handle of an rr_accum window: device accumulators plus the seen-mask."""

    def __init__(self, bufs: Sequence[torch.Tensor], G: int, version: int):
        self.bufs = list(bufs)
        self.seen = (ctypes.c_uint8 * G)()
        self.c = CAccum()
        self.c.n_bufs = len(self.bufs)
        for i, b in enumerate(self.bufs):
            self.c.buf[i] = _ptr(b)
            self.c.n[i] = b.numel()
        self.c.G = G
        self.c.version = version
        self.c.seen = ctypes.cast(self.seen, ctypes.POINTER(ctypes.c_uint8))
        for b in self.bufs:
            if b.dtype != torch.float32:
                raise ValueError(f"rr_accum buffers must be torch.float32 (got {b.dtype})")


def rr_grad_accum(acc: Accum, member_g: int, tag: CGradTag, grads: Sequence[torch.Tensor],
                  scale: float = 1.0, n_elems: Optional[Sequence[int]] = None, stream=None) -> None:
    """acc += scale * grads of member member_g; tag is what rr_attn_bwd returned for them."""
    n = len(grads)
    if n != acc.c.n_bufs:
        raise ValueError(f"rr_grad_accum: {n} gradients for a window of {acc.c.n_bufs} buffers")
    if n_elems is not None and len(n_elems) != n:
        raise ValueError(f"rr_grad_accum: {len(n_elems)} element counts for {n} gradients")
    for i, g in enumerate(grads):
        if g.dtype != torch.float32:
            raise ValueError(f"rr_grad_accum: gradient {i} has dtype {g.dtype}, expected torch.float32")
        if n_elems is not None and not 0 <= int(n_elems[i]) <= g.numel():
            raise ValueError(f"rr_grad_accum: n_elems[{i}] = {n_elems[i]} outside [0, {g.numel()}]")
    ptrs = (ctypes.c_void_p * n)(*[_ptr(g) for g in grads])
    ns = (ctypes.c_int64 * n)(*[(g.numel() if n_elems is None else int(n_elems[i])) for i, g in enumerate(grads)])
    _check(lib().rr_grad_accum(ctypes.byref(acc.c), member_g, ctypes.byref(tag) if tag is not None else None,
                               ptrs, ns, scale, _stream(stream)))


def rr_accum_check_complete(acc: Accum) -> None:
    _check(lib().rr_accum_check_complete(ctypes.byref(acc.c)))


def rr_profile_begin() -> None:
    _check(lib().rr_profile_begin())


def rr_profile_end() -> dict:
    arr = (CProfileEntry * 64)()
    n = ctypes.c_int32(0)
    _check(lib().rr_profile_end(arr, 64, ctypes.byref(n)))
    return {arr[i].name.decode(): (int(arr[i].launches), float(arr[i].total_ms)) for i in range(n.value)}
