"""The C ABI on the CPU: the library loads, exports every entry point the header declares,
and rejects invalid calls on the host before any launch (no GPU needed: every call here
fails validation, so nothing reaches HIP)."""
import ctypes
import os
import re

import pytest

from resident_kv_response_amd import rr_attn as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rr_attn.h")
FAKE = 0x100000   # a 16-byte aligned stand-in device address; never dereferenced here


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(rr_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(R.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = R.lib()
    for name in _declared():
        assert hasattr(L, name), name


def _prob(**kw):
    base = dict(P=4096, R_max=256, Hq=4, Hkv=1, d_qk=64, d_v=64, chunk=1024, block=256, tau=0.125,
                dtype=R.RR_F32)
    base.update(kw)
    return R.Problem(**base)


def _fwd(p, r_len=(256,), q=FAKE, kv=None, o=FAKE, lse=FAKE, part_o=None, part_lse=None, ws=FAKE,
         ws_bytes=1 << 40):
    L = R.lib()
    kv = kv or R.CResident(k_p=FAKE, v_p=FAKE, k_idx=None, P=p.P, version=0)
    cp = p.c()
    arr = (ctypes.c_int32 * len(r_len))(*r_len)
    rc = L.rr_attn_fwd(ctypes.byref(cp), ctypes.byref(kv), q, FAKE, FAKE, arr, None, o, lse, part_o,
                       part_lse, None, ws, ws_bytes, None)
    return rc, L.rr_last_error().decode()


@pytest.mark.parametrize("kw,code,frag", [
    (dict(Hq=5, Hkv=2), R.RR_E_SHAPE, "multiple"),
    (dict(P=-1), R.RR_E_SHAPE, "P must"),
    (dict(R_max=0), R.RR_E_SHAPE, "R_max"),
    (dict(K=0), R.RR_E_SHAPE, "K must"),
    (dict(K=65), R.RR_E_SHAPE, "K must"),
    (dict(chunk=0), R.RR_E_SHAPE, "chunk"),
    (dict(block=0), R.RR_E_SHAPE, "block"),
    (dict(tau=0.0), R.RR_E_SHAPE, "tau"),
    (dict(tau=float("inf")), R.RR_E_SHAPE, "tau"),
    (dict(dtype=7), R.RR_E_SHAPE, "dtype"),
    (dict(d_qk=96, d_v=96), R.RR_E_UNSUPPORTED, "head dims"),
    (dict(d_qk=128, d_v=64), R.RR_E_UNSUPPORTED, "head dims"),
])
def test_fwd_rejects_bad_problems(kw, code, frag):
    rc, msg = _fwd(_prob(**kw))
    assert rc == code and frag in msg, (rc, msg)


def test_fwd_rejects_bad_arguments():
    p = _prob()
    assert _fwd(p, r_len=(257,))[0] == R.RR_E_SHAPE
    assert _fwd(p, r_len=(-1,))[0] == R.RR_E_SHAPE
    assert _fwd(p, q=None)[0] == R.RR_E_NULL
    assert _fwd(p, q=FAKE + 2)[0] == R.RR_E_SHAPE          # misaligned
    assert _fwd(p, o=None)[0] == R.RR_E_NULL                # o without lse
    assert _fwd(p, o=None, lse=None)[0] == R.RR_E_NULL      # no output at all
    assert _fwd(p, ws=None)[0] == R.RR_E_WORKSPACE
    assert _fwd(p, ws_bytes=R.rr_workspace_bytes(p, R.RR_OP_FWD) - 1)[0] == R.RR_E_WORKSPACE
    bad_kv = R.CResident(k_p=FAKE, v_p=FAKE, k_idx=None, P=p.P + 1, version=0)
    assert _fwd(p, kv=bad_kv)[0] == R.RR_E_SHAPE
    null_kv = R.CResident(k_p=None, v_p=FAKE, k_idx=None, P=p.P, version=0)
    assert _fwd(p, kv=null_kv)[0] == R.RR_E_NULL


def test_bwd_rejects_bad_arguments():
    L = R.lib()
    p = _prob()
    cp = p.c()
    kv = R.CResident(k_p=FAKE, v_p=FAKE, k_idx=None, P=p.P, version=0)
    arr = (ctypes.c_int32 * 1)(256)

    def call(accumulate=0, block_idx=-1, ws=FAKE, ws_bytes=1 << 40, dq=FAKE):
        return L.rr_attn_bwd(ctypes.byref(cp), ctypes.byref(kv), FAKE, FAKE, FAKE, arr, None, FAKE,
                             FAKE, FAKE, dq, FAKE, FAKE, accumulate, block_idx, ws, ws_bytes, None, None)

    assert call(block_idx=1) == R.RR_E_SHAPE          # one block of 256 rows only
    assert call(block_idx=-2) == R.RR_E_SHAPE
    assert call(accumulate=2) == R.RR_E_SHAPE
    assert call(dq=None) == R.RR_E_NULL
    assert call(ws=None) == R.RR_E_WORKSPACE
    assert call(ws_bytes=R.rr_workspace_bytes(p, R.RR_OP_BWD) - 1) == R.RR_E_WORKSPACE


def test_prompt_grads_rejects_bad_arguments():
    L = R.lib()
    p = _prob()
    kv = R.CResident(k_p=FAKE, v_p=FAKE, k_idx=None, P=p.P, version=0)

    def call(prob=p, r_len=(256,), accumulate=0, ws=FAKE, ws_bytes=1 << 40, dk_p=FAKE, kv_=kv, keys=None):
        cp = prob.c()
        arr = (ctypes.c_int32 * len(r_len))(*r_len)
        lo, hi = keys if keys is not None else (0, prob.P)
        return L.rr_attn_prompt_grads(ctypes.byref(cp), ctypes.byref(kv_), FAKE, arr, FAKE, FAKE, FAKE, lo, hi,
                                      dk_p, FAKE, accumulate, ws, ws_bytes, None)

    assert call(r_len=(257,)) == R.RR_E_SHAPE
    assert call(accumulate=2) == R.RR_E_SHAPE
    assert call(keys=(-1, 10)) == R.RR_E_SHAPE
    assert call(keys=(10, 9)) == R.RR_E_SHAPE
    assert call(keys=(0, p.P + 1)) == R.RR_E_SHAPE
    assert call(dk_p=None) == R.RR_E_NULL
    assert call(dk_p=FAKE + 4) == R.RR_E_SHAPE                      # misaligned
    assert call(ws=None) == R.RR_E_WORKSPACE
    assert call(ws_bytes=R.rr_workspace_bytes(p, R.RR_OP_PROMPT_GRADS) - 1) == R.RR_E_WORKSPACE
    assert call(kv_=R.CResident(k_p=FAKE, v_p=None, k_idx=None, P=p.P, version=0)) == R.RR_E_NULL
    lat = R.Problem(P=4096, R_max=64, Hq=64, Hkv=1, d_qk=576, d_v=512, chunk=4096, block=64, tau=0.04,
                    dtype=R.RR_BF16, topk=256, idx_dim=128, latent=1)
    assert call(prob=lat, r_len=(64,)) == R.RR_E_UNSUPPORTED


def test_prompt_grads_workspace_formula():
    # rows of each KV head, every response at R_max rows, padded to 64 per response
    p = _prob(P=2097152, R_max=7666, Hq=24, Hkv=4, d_qk=128, d_v=128, chunk=131072, dtype=R.RR_BF16, K=3)
    up = lambda x: -(-x // 256) * 256
    rows = 4 * 3 * (-(-7666 * 6 // 64) * 64)
    assert R.rr_workspace_bytes(p, R.RR_OP_PROMPT_GRADS) == 2 * up(rows * 128 * 2) + up(rows * 8)
    p32 = _prob()
    rows = 1 * 1 * 256 * 4
    assert R.rr_workspace_bytes(p32, R.RR_OP_PROMPT_GRADS) == 2 * up(rows * 64 * 4) + up(rows * 8)


def test_merge_rejects_bad_arguments():
    L = R.lib()
    assert L.rr_lse_merge(0, 10, 64, FAKE, FAKE, FAKE, FAKE, None) == R.RR_E_SHAPE
    assert L.rr_lse_merge(2, -1, 64, FAKE, FAKE, FAKE, FAKE, None) == R.RR_E_SHAPE
    assert L.rr_lse_merge(2, 10, 0, FAKE, FAKE, FAKE, FAKE, None) == R.RR_E_SHAPE
    assert L.rr_lse_merge(2, 10, 64, None, FAKE, FAKE, FAKE, None) == R.RR_E_NULL


def test_workspace_and_parts_formulas():
    p = _prob(P=2097152, R_max=8192, Hq=24, Hkv=4, d_qk=128, d_v=128, chunk=131072, dtype=R.RR_BF16)
    assert R.rr_num_parts(p) == 17
    rows = 8192 * 24
    up = lambda x: -(-x // 256) * 256
    assert R.rr_workspace_bytes(p, R.RR_OP_FWD) == up(17 * rows * 128 * 4) + up(17 * rows * 4)
    stream = 4 * 8192 * 6          # packed rows of the response dK/dV kernel: Hkv * R_max * grp
    assert R.rr_workspace_bytes(p, R.RR_OP_BWD) == (up(rows * 4) + up(17 * rows * 128 * 4)
                                                    + 2 * up(stream * 128 * 2) + up(stream * 8))
    with pytest.raises(R.RRError):
        R.rr_workspace_bytes(_prob(Hq=3, Hkv=2), R.RR_OP_FWD)


def test_bwd_workspace_holds_the_key_gradient_slots():
    # bf16: the dQ partials' region is reused, once dQ is reduced, for the partial slots
    # ([128 keys][d_qk + d_v] fp32) of the response dK/dV kernel's later segments: per
    # response min(1024, Hkv * key tiles * 64-row stages / 8); a small problem with a short
    # prompt needs the slots' size, a large one the partials'
    up = lambda x: -(-x // 256) * 256
    p = _prob(P=64, R_max=2048, Hq=4, Hkv=1, d_qk=64, d_v=64, chunk=64, dtype=R.RR_BF16)
    rows = 2048 * 4
    slots = min(1024, 1 * 16 * 128 // 8) * 128 * (64 + 64) * 4
    assert 2 * rows * 64 * 4 < slots
    stream = 1 * 2048 * 4
    assert R.rr_workspace_bytes(p, R.RR_OP_BWD) == (up(rows * 4) + up(slots) + 2 * up(stream * 64 * 2)
                                                    + up(stream * 8))
    # K responses: K times the slots
    pk = _prob(P=64, R_max=2048, Hq=4, Hkv=1, d_qk=64, d_v=64, chunk=64, dtype=R.RR_BF16, K=3)
    assert R.rr_workspace_bytes(pk, R.RR_OP_BWD) == (up(3 * rows * 4) + up(3 * slots) + 2 * up(3 * stream * 64 * 2)
                                                     + up(3 * stream * 8))
    # fp32 runs no segmented kernel: D and the dQ partials only
    p32 = _prob(P=64, R_max=2048, Hq=4, Hkv=1, d_qk=64, d_v=64, chunk=64, dtype=R.RR_F32)
    assert R.rr_workspace_bytes(p32, R.RR_OP_BWD) == up(rows * 4) + up(2 * rows * 64 * 4)


def _accum(G=8, version=5):
    acc = R.CAccum()
    seen = (ctypes.c_uint8 * G)()
    acc.n_bufs = 2
    acc.buf[0], acc.buf[1] = FAKE, FAKE
    acc.n[0], acc.n[1] = 100, 50
    acc.G, acc.version = G, version
    acc.seen = ctypes.cast(seen, ctypes.POINTER(ctypes.c_uint8))
    return acc, seen


def _accum_call(acc, g, tag, n=(100, 50)):
    L = R.lib()
    ptrs = (ctypes.c_void_p * 2)(FAKE, FAKE)
    ns = (ctypes.c_int64 * 2)(*n)
    return L.rr_grad_accum(ctypes.byref(acc), g, ctypes.byref(tag) if tag is not None else None, ptrs, ns,
                           1.0, None)


def test_accumulator_hazards_are_rejected_before_launch():
    # Only rr_attn_bwd writes a valid tag (sealed over the resident's version, k_p and P);
    # here every tag is hand-made, so each call stops at a check before any launch.  The
    # accepting path, the version and the prompt-group checks with real tags are covered by
    # tests/native/host_checks.cpp and tests/test_gpu_invariants.py.
    acc, seen = _accum()
    tag = R.CGradTag(version=5, resident=FAKE, P=4096, seal=1234)
    assert _accum_call(acc, 8, tag) == R.RR_E_RANGE            # member outside the window
    assert _accum_call(acc, -1, tag) == R.RR_E_RANGE
    assert _accum_call(acc, 3, None) == R.RR_E_NULL            # no tag
    L = R.lib()
    assert _accum_call(acc, 3, tag) == R.RR_E_STALE            # a tag no backward wrote
    assert "not written by rr_attn_bwd" in L.rr_last_error().decode()
    assert bytes(seen) == bytes(8)                              # rejections leave the mask alone
    assert L.rr_accum_check_complete(ctypes.byref(acc)) == R.RR_E_MISSING
    assert "member 0" in L.rr_last_error().decode()
    for g in range(8):
        seen[g] = 1
    assert L.rr_accum_check_complete(ctypes.byref(acc)) == R.RR_OK
    acc.poisoned = 1                                            # after a failed partial launch
    assert _accum_call(acc, 3, tag) == R.RR_E_POISONED
    assert L.rr_accum_check_complete(ctypes.byref(acc)) == R.RR_E_POISONED


def test_binding_checks_layouts_before_any_call():
    """The binding refuses tensors whose dtype or element count differs from the layout
    of include/rr_attn.h before calling the library (host tensors reach this check first,
    so no GPU is needed; a correctly shaped host tensor is then refused as a host
    pointer)."""
    import torch
    p = _prob(P=64, R_max=16, Hq=4, Hkv=1, d_qk=64, d_v=64, chunk=32, block=16, dtype=R.RR_BF16)
    kv = R.CResident(k_p=FAKE, v_p=FAKE, k_idx=None, P=p.P, version=0)
    bf = lambda *sh: torch.zeros(*sh, dtype=torch.bfloat16)
    f32 = lambda *sh: torch.zeros(*sh, dtype=torch.float32)
    q, kr, vr = bf(1, 16, 4, 64), bf(1, 16, 1, 64), bf(1, 16, 1, 64)
    o, lse = f32(1, 16, 4, 64), f32(1, 16, 4)
    with pytest.raises(ValueError, match="q has dtype"):
        R.rr_attn_fwd(p, kv, f32(1, 16, 4, 64), kr, vr, [16], o=o, lse=lse)
    with pytest.raises(ValueError, match="k_r has 512 elements"):
        R.rr_attn_fwd(p, kv, q, bf(1, 8, 1, 64), vr, [16], o=o, lse=lse)
    with pytest.raises(ValueError, match="o has 2048 elements"):
        R.rr_attn_fwd(p, kv, q, kr, vr, [16], o=f32(1, 16, 4, 32), lse=lse)
    with pytest.raises(ValueError, match="lse has dtype"):
        R.rr_attn_fwd(p, kv, q, kr, vr, [16], o=o, lse=bf(1, 16, 4))
    with pytest.raises(ValueError, match="r_len has 2 entries"):
        R.rr_attn_fwd(p, kv, q, kr, vr, [16, 16], o=o, lse=lse)
    with pytest.raises(ValueError, match="workspace has dtype"):
        R.rr_attn_fwd(p, kv, q, kr, vr, [16], o=o, lse=lse, ws=f32(10))
    with pytest.raises(ValueError, match="dq has 2048 elements"):
        R.rr_attn_bwd(p, kv, q, kr, vr, [16], o, lse, bf(1, 16, 4, 64), f32(1, 8, 4, 64), f32(1, 16, 1, 64),
                      f32(1, 16, 1, 64))
    with pytest.raises(ValueError, match="d_o has dtype"):
        R.rr_attn_bwd(p, kv, q, kr, vr, [16], o, lse, f32(1, 16, 4, 64), f32(1, 16, 4, 64), f32(1, 16, 1, 64),
                      f32(1, 16, 1, 64))
    with pytest.raises(ValueError, match="dk_p has"):
        R.rr_attn_prompt_grads(p, kv, q, [16], o, lse, bf(1, 16, 4, 64), f32(63, 1, 64), f32(64, 1, 64))
    with pytest.raises(ValueError, match="part_lse has"):
        R.rr_lse_merge(f32(3, 16, 64), f32(2, 16), f32(16, 64), f32(16))
    with pytest.raises(ValueError, match="x_out has"):
        R.rr_lastkv_blend(f32(2), bf(8, 2, 16), bf(8, 2, 16), bf(7, 2, 16))
    with pytest.raises(ValueError, match="d_alpha has"):
        R.rr_lastkv_blend_bwd(f32(2), bf(8, 2, 16), bf(8, 2, 16), f32(8, 2, 16), None, None, f32(1))
    # a correctly laid out call gets past the layout checks and stops at the host pointer
    with pytest.raises(ValueError, match="GPU tensors"):
        R.rr_attn_fwd(p, kv, q, kr, vr, [16], o=o, lse=lse)


def test_binding_accumulator_arguments():
    import torch
    acc = R.Accum.__new__(R.Accum)           # a window handle without device buffers
    acc.c = R.CAccum()
    acc.c.n_bufs = 3
    g = [torch.zeros(10)] * 2
    with pytest.raises(ValueError, match="2 gradients for a window of 3"):
        R.rr_grad_accum(acc, 0, R.CGradTag(), g)
    acc.c.n_bufs = 2
    with pytest.raises(ValueError, match="n_elems"):
        R.rr_grad_accum(acc, 0, R.CGradTag(), g, n_elems=[10, 11])
    with pytest.raises(ValueError, match="dtype"):
        R.rr_grad_accum(acc, 0, R.CGradTag(), [torch.zeros(10, dtype=torch.float64)] * 2)


def _latent(**kw):
    base = dict(P=1048576, R_max=4096, Hq=64, Hkv=1, d_qk=576, d_v=512, chunk=65536, block=2048,
                tau=1.0 / 24.0, dtype=R.RR_BF16, topk=2048, idx_dim=128, latent=1)
    base.update(kw)
    return R.Problem(**base)


def _latent_fwd(p, q_idx=FAKE, k_idx=FAKE, topk_idx=FAKE, ws=FAKE, ws_bytes=1 << 40, part_o=None):
    L = R.lib()
    kv = R.CResident(k_p=FAKE, v_p=None, k_idx=k_idx, P=p.P, version=0)
    cp = p.c()
    arr = (ctypes.c_int32 * 1)(min(p.R_max, 8))
    rc = L.rr_attn_fwd(ctypes.byref(cp), ctypes.byref(kv), FAKE, FAKE, None, arr, q_idx, FAKE, FAKE, part_o,
                       FAKE if part_o else None, topk_idx, ws, ws_bytes, None)
    return rc, L.rr_last_error().decode()


@pytest.mark.parametrize("kw,code,frag", [
    (dict(dtype=R.RR_F32), R.RR_E_UNSUPPORTED, "bf16"),
    (dict(Hq=32), R.RR_E_UNSUPPORTED, "Hq=64"),
    (dict(d_qk=512), R.RR_E_UNSUPPORTED, "d_qk=576"),
    (dict(topk=2000), R.RR_E_SHAPE, "multiple of 32"),
    (dict(topk=0), R.RR_E_SHAPE, "multiple of 32"),
    (dict(topk=8192), R.RR_E_SHAPE, "4096"),
    (dict(P=1000, topk=1024), R.RR_E_SHAPE, "multiple of 32"),
    (dict(idx_dim=64), R.RR_E_UNSUPPORTED, "128 wide"),
    (dict(R_max=4092), R.RR_E_SHAPE, "R_max"),
    (dict(flags=R.RR_FLAG_SHARD_NO_RESPONSE), R.RR_E_UNSUPPORTED, "shard"),
])
def test_latent_problem_limits(kw, code, frag):
    rc, msg = _latent_fwd(_latent(**kw))
    assert rc == code and frag in msg, (rc, msg)


def test_latent_fwd_arguments_and_workspace():
    p = _latent()
    assert _latent_fwd(p, q_idx=None)[0] == R.RR_E_NULL
    assert _latent_fwd(p, k_idx=None)[0] == R.RR_E_NULL
    assert _latent_fwd(p, topk_idx=None)[0] == R.RR_E_NULL
    assert _latent_fwd(p, part_o=FAKE)[0] == R.RR_E_UNSUPPORTED
    assert _latent_fwd(p, ws=FAKE + 8)[0] == R.RR_E_SHAPE            # misaligned workspace
    need = R.rr_workspace_bytes(p, R.RR_OP_FWD)
    assert _latent_fwd(p, ws_bytes=need - 1)[0] == R.RR_E_WORKSPACE
    # per row a threshold and a candidate count, the key-norm maximum of each of the
    # screen's key ranges, then one region holding first the sample scores [K*R][8192] and
    # then the candidates (keys and positions [K*R][cap], cap = 2 * expected + 1024,
    # expected = rank * P / 8192, rank = 3k * 8192 / P): no [K*R][P] score matrix
    up = lambda x: -(-x // 256) * 256
    rank = max(32, -(-3 * 2048 * 8192 // 1048576))
    cap = up(2 * (rank * 1048576 // 8192) + 1024)
    n_kt = 1048576 // 32
    per = -(-n_kt // 128)
    n_splits = -(-n_kt // per)
    region = max(4096 * 8192 * 4, 2 * up(4096 * cap * 4))
    assert need == 2 * up(4096 * 4) + up(n_splits * 4) + up(region)
    assert need < 4096 * 1048576 // 8          # far below the 16 GiB a score matrix would take
    # backward: D, then P and dS of the response pairs [K][R][64][R] bf16 (+ one padded
    # segment), then the dK_r / dV_r chunk partials [16 chunks of 256 rows][K][R][576] fp32
    assert R.rr_workspace_bytes(p, R.RR_OP_BWD) == (up(4096 * 64 * 4) + 2 * up((4096 * 64 * 4096 + 128) * 2)
                                                   + up(16 * 4096 * 576 * 4))
    # short rows take the exact full-row path and need only the per-row arrays
    small = _latent(P=3000, R_max=96, topk=256)
    assert R.rr_workspace_bytes(small, R.RR_OP_FWD) == 2 * up(96 * 4) + up(4)


def test_blend_rejects_bad_arguments():
    L = R.lib()
    assert L.rr_lastkv_blend(10, 2, 12, R.RR_BF16, FAKE, FAKE, FAKE, FAKE, None) == R.RR_E_SHAPE   # d % 8
    assert L.rr_lastkv_blend(-1, 2, 16, R.RR_BF16, FAKE, FAKE, FAKE, FAKE, None) == R.RR_E_SHAPE
    assert L.rr_lastkv_blend(10, 2, 16, 5, FAKE, FAKE, FAKE, FAKE, None) == R.RR_E_SHAPE
    assert L.rr_lastkv_blend(10, 2, 16, R.RR_BF16, None, FAKE, FAKE, FAKE, None) == R.RR_E_NULL
    assert L.rr_lastkv_blend(10, 2, 16, R.RR_BF16, FAKE, FAKE + 2, FAKE, FAKE, None) == R.RR_E_SHAPE
    assert L.rr_lastkv_blend_bwd(10, 2, 16, R.RR_F32, FAKE, FAKE, FAKE, FAKE, None, None, None, 0,
                                 None) == R.RR_E_NULL                                   # d_alpha
    assert L.rr_lastkv_blend_bwd(10, 2, 16, R.RR_F32, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 3,
                                 None) == R.RR_E_SHAPE                                  # accumulate


def test_empty_prompt_is_accepted_without_resident_pointers():
    # P = 0: rows attend to their own causal keys only; k_p / v_p may be NULL
    p = _prob(P=0)
    assert R.rr_num_parts(p) == 1
    kv = R.CResident(k_p=None, v_p=None, k_idx=None, P=0, version=0)
    rc, msg = _fwd(p, kv=kv, ws=None, ws_bytes=0)
    assert rc == R.RR_E_WORKSPACE, msg          # passes every check up to the workspace


def test_binding_rejects_host_tensors():
    # a host pointer handed to a kernel would fault: the binding refuses it before any call
    import torch
    x = torch.zeros(8, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensors"):
        R.resident(x, x)
    with pytest.raises(ValueError, match="GPU tensors"):
        R.rr_lse_merge(torch.zeros(2, 4, 64), torch.zeros(2, 4), torch.zeros(4, 64), torch.zeros(4))


def _gpu_present():
    import torch
    return torch.cuda.device_count() > 0


@pytest.mark.skipif(_gpu_present(), reason="passes made-up pointers past validation; CPU hosts only")
def test_pointer_check_runs_before_any_launch():
    # valid shapes with pointers the GPU cannot access: the call stops at the pointer check
    # (RR_E_PTR), never at a launch
    p = _prob()
    rc, msg = _fwd(p, ws_bytes=R.rr_workspace_bytes(p, R.RR_OP_FWD))
    assert rc == R.RR_E_PTR, (rc, msg)
    assert "not memory the GPU can access" in msg


def test_static_scratch_forward_refuses_oversized_problems():
    # the workspace check runs before the scratch is looked up: no device is touched
    L = R.lib()
    p = _prob(P=131072, R_max=4096, Hq=32, Hkv=8, d_qk=128, d_v=128, chunk=8192, dtype=R.RR_BF16)
    assert R.rr_workspace_bytes(p, R.RR_OP_FWD) > R.RR_STATIC_SCRATCH_BYTES
    kv = R.CResident(k_p=FAKE, v_p=FAKE, k_idx=None, P=p.P, version=0)
    cp = p.c()
    arr = (ctypes.c_int32 * 1)(4096)
    rc = L.rr_attn_fwd_static(ctypes.byref(cp), ctypes.byref(kv), FAKE, FAKE, FAKE, arr, None, FAKE, FAKE,
                              None, None, None, None)
    assert rc == R.RR_E_WORKSPACE
    assert "static scratch" in L.rr_last_error().decode()
    cp = _prob(R_max=0).c()          # invalid problems are refused the same way as rr_attn_fwd
    rc = L.rr_attn_fwd_static(ctypes.byref(cp), ctypes.byref(kv), FAKE, FAKE, FAKE, arr, None, FAKE, FAKE,
                              None, None, None, None)
    assert rc == R.RR_E_SHAPE
