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
RR_F32, RR_BF16 = 0, 1
RR_OP_FWD, RR_OP_BWD, RR_OP_PROMPT_GRADS = 0, 1, 2
RR_MAX_K, RR_MAX_ACC = 64, 8
RR_FLAG_SHARD_NO_RESPONSE = 1

EXPORTS = ["rr_workspace_bytes", "rr_num_parts", "rr_attn_fwd", "rr_lse_merge", "rr_attn_bwd",
           "rr_attn_prompt_grads", "rr_lastkv_blend", "rr_lastkv_blend_bwd", "rr_grad_accum", "rr_accum_check_complete", "rr_last_error", "rr_profile_begin",
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


class CAccum(ctypes.Structure):
    _fields_ = [("n_bufs", ctypes.c_int32), ("buf", ctypes.c_void_p * RR_MAX_ACC),
                ("n", ctypes.c_int64 * RR_MAX_ACC), ("G", ctypes.c_int32),
                ("version", ctypes.c_uint64), ("seen", ctypes.POINTER(ctypes.c_uint8))]


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
        L.rr_lse_merge.argtypes = [i32, i64, i32, vp, vp, vp, vp, vp]
        L.rr_lse_merge.restype = ctypes.c_int
        L.rr_attn_bwd.argtypes = [ctypes.POINTER(CProblem), ctypes.POINTER(CResident), vp, vp, vp,
                                  ctypes.POINTER(i32), vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, sz, vp]
        L.rr_attn_bwd.restype = ctypes.c_int
        L.rr_attn_prompt_grads.argtypes = [ctypes.POINTER(CProblem), ctypes.POINTER(CResident), vp,
                                           ctypes.POINTER(i32), vp, vp, vp, i64, i64, vp, vp, i32, vp, sz,
                                           vp]
        L.rr_attn_prompt_grads.restype = ctypes.c_int
        L.rr_lastkv_blend.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp, vp]
        L.rr_lastkv_blend.restype = ctypes.c_int
        L.rr_lastkv_blend_bwd.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp]
        L.rr_lastkv_blend_bwd.restype = ctypes.c_int
        L.rr_grad_accum.argtypes = [ctypes.POINTER(CAccum), i32, ctypes.c_uint64,
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


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _r_len(r_len: Sequence[int]):
    arr = (ctypes.c_int32 * len(r_len))(*[int(x) for x in r_len])
    return arr


def resident(k_p: torch.Tensor, v_p: Optional[torch.Tensor], version: int = 0,
             k_idx: Optional[torch.Tensor] = None) -> CResident:
    return CResident(k_p=_ptr(k_p), v_p=_ptr(v_p), k_idx=_ptr(k_idx), P=k_p.shape[0],
                     version=version)


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
    cp = p.c()
    wsp = _ptr(ws)
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().rr_attn_fwd(ctypes.byref(cp), ctypes.byref(kv), _ptr(q), _ptr(k_r), _ptr(v_r),
                             _r_len(r_len), _ptr(q_idx), _ptr(o), _ptr(lse), _ptr(part_o),
                             _ptr(part_lse), _ptr(topk_idx), wsp, nbytes, _stream(stream)))


def rr_lse_merge(part_o, part_lse, o, lse, stream=None) -> None:
    n_parts, rows, d_v = part_o.shape[0], part_lse[0].numel(), part_o.shape[-1]
    _check(lib().rr_lse_merge(n_parts, rows, d_v, _ptr(part_o), _ptr(part_lse), _ptr(o), _ptr(lse),
                              _stream(stream)))


def rr_attn_bwd(p: Problem, kv: CResident, q, k_r, v_r, r_len, o, lse, d_o, dq, dk_r, dv_r,
                accumulate: int = 0, block_idx: int = -1, topk_idx=None, ws=None,
                stream=None) -> None:
    cp = p.c()
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().rr_attn_bwd(ctypes.byref(cp), ctypes.byref(kv), _ptr(q), _ptr(k_r), _ptr(v_r),
                             _r_len(r_len), _ptr(topk_idx), _ptr(o), _ptr(lse), _ptr(d_o), _ptr(dq),
                             _ptr(dk_r), _ptr(dv_r), int(accumulate), int(block_idx), _ptr(ws),
                             nbytes, _stream(stream)))


def rr_attn_prompt_grads(p: Problem, kv: CResident, q, r_len, o, lse, d_o, dk_p, dv_p,
                         accumulate: int = 0, key_range=None, ws=None, stream=None) -> None:
    """Full-sequence differential mode: dk_p, dv_p [key_hi - key_lo][Hkv][d] fp32 of the
    resident positions in key_range (default: the whole prompt), the prompt-side term
    that rr_attn_bwd drops."""
    cp = p.c()
    lo, hi = key_range if key_range is not None else (0, p.P)
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
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
    _check(lib().rr_lastkv_blend(rows, Hkv, d, _dtype_code(x_layer), _ptr(alpha), _ptr(x_layer),
                                 _ptr(x_last), _ptr(x_out), _stream(stream)))


def rr_lastkv_blend_bwd(alpha, x_layer, x_last, d_out, d_layer, d_last, d_alpha, accumulate: int = 0,
                        stream=None) -> None:
    rows, Hkv, d = x_layer.shape
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


def rr_grad_accum(acc: Accum, member_g: int, version: int, grads: Sequence[torch.Tensor],
                  scale: float = 1.0, n_elems: Optional[Sequence[int]] = None, stream=None) -> None:
    n = len(grads)
    ptrs = (ctypes.c_void_p * n)(*[_ptr(g) for g in grads])
    ns = (ctypes.c_int64 * n)(*[(g.numel() if n_elems is None else n_elems[i]) for i, g in enumerate(grads)])
    _check(lib().rr_grad_accum(ctypes.byref(acc.c), member_g, version, ptrs, ns, scale, _stream(stream)))


def rr_accum_check_complete(acc: Accum) -> None:
    _check(lib().rr_accum_check_complete(ctypes.byref(acc.c)))


def rr_profile_begin() -> None:
    _check(lib().rr_profile_begin())


def rr_profile_end() -> dict:
    arr = (CProfileEntry * 64)()
    n = ctypes.c_int32(0)
    _check(lib().rr_profile_end(arr, 64, ctypes.byref(n)))
    return {arr[i].name.decode(): (int(arr[i].launches), float(arr[i].total_ms)) for i in range(n.value)}
