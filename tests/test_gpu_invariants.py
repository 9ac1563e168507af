"""GPU invariants of the method (needs an MI355X): chunking and blocking do not change the
result, the reverse block walk finalises block b at step b, exported partials merged by
rr_lse_merge equal the fused output, results are bitwise deterministic, the resident
prompt KV is never written, and serial accumulation equals the sum of replays."""
import numpy as np
import pytest
import torch

from oracle import dense
from resident_kv_response_amd import configs, rr_attn as R, synth
from tests._helpers import assert_bf16_close

pytestmark = pytest.mark.gpu

W = configs.SHARE_P256K.with_(P=4100, R=520, chunk=1024, block=128, seed=5001)


def _setup(w=W, R_list=None, chunk=None, block=None):
    from tests import _gpu as G
    R_list = R_list or [w.R]
    res = synth.resident(w)
    mem = [synth.member(w, g, R=r) for g, r in enumerate(R_list)]
    st = G.stack_members(mem, max(R_list))
    prob = G.problem(w.P, max(R_list), w.Hq, w.Hkv, w.d_qk, chunk or w.chunk, block or w.block,
                     w.dtype, K=len(R_list), tau=w.tau)
    return G, res, st, prob, R_list


def test_chunk_and_block_invariance():
    outs = []
    for chunk, block in [(4100, 520), (1024, 128), (333, 77), (64, 64)]:
        G, res, st, prob, rl = _setup(chunk=chunk, block=block)
        print(f"[invariance] chunk={chunk} block={block}", flush=True)
        outs.append(G.Run(prob, W.dtype, res["k_p"], res["v_p"], st, rl).fwd().bwd().numpy())
    for o in outs[1:]:
        for key in ("o", "dq", "dk", "dv"):
            assert_bf16_close(key, o[key], outs[0][key])


def test_deterministic_and_prompt_untouched():
    G, res, st, prob, rl = _setup()
    a = G.Run(prob, W.dtype, res["k_p"], res["v_p"], st, rl)
    kp0, vp0 = a.k_p.clone(), a.v_p.clone()
    x = a.fwd().bwd().numpy()
    y = a.fwd().bwd().numpy()
    for key in x:
        np.testing.assert_array_equal(x[key], y[key])
    assert torch.equal(a.k_p.view(torch.int16), kp0.view(torch.int16))
    assert torch.equal(a.v_p.view(torch.int16), vp0.view(torch.int16))


@pytest.mark.parametrize("block,R_list", [(128, None), (77, [520, 301, 1]), (200, [520, 77])])
def test_caller_driven_reverse_walk(block, R_list):
    """Blocks driven one call at a time, last first, equal the whole walk; after step b the
    dQ, dK, dV rows of block b are final.  Block sizes whose row boundaries fall inside a
    64-row stage of the packed stream (77 and 200 rows with 6 heads per KV head), and
    responses that end before, inside or after a block."""
    G, res, st, prob, rl = _setup(R_list=R_list, block=block)
    full = G.Run(prob, W.dtype, res["k_p"], res["v_p"], st, rl).fwd().bwd().numpy()
    run = G.Run(prob, W.dtype, res["k_p"], res["v_p"], st, rl).fwd()
    run.dq.zero_()
    run.dk.zero_()
    run.dv.zero_()
    R_max = max(rl)
    nb = -(-R_max // block)
    print(f"[walk] block={block} R={rl}", flush=True)
    for b in range(nb - 1, -1, -1):
        run.bwd(accumulate=1, block_idx=b)
        now = run.numpy()
        lo, hi = b * block, min(R_max, (b + 1) * block)
        # after step b, the rows of block b are final
        for key in ("dk", "dv", "dq"):
            np.testing.assert_allclose(now[key][:, lo:hi], full[key][:, lo:hi], rtol=0, atol=1e-6,
                                       err_msg=f"{key} block {b}")


def test_exported_partials_merge():
    G, res, st, prob, rl = _setup()
    run = G.Run(prob, W.dtype, res["k_p"], res["v_p"], st, rl)
    n_parts = R.rr_num_parts(prob)
    po = torch.empty((n_parts, 1, W.R, W.Hq, W.d_v), device="cuda", dtype=torch.float32)
    pl = torch.empty((n_parts, 1, W.R, W.Hq), device="cuda", dtype=torch.float32)
    run.fwd(part_o=po, part_lse=pl)
    o2 = torch.empty_like(run.o)
    l2 = torch.empty_like(run.lse)
    R.rr_lse_merge(po, pl, o2, l2)
    torch.cuda.synchronize()
    np.testing.assert_allclose(o2.cpu().numpy(), run.o.cpu().numpy(), rtol=0, atol=1e-6)
    np.testing.assert_allclose(l2.cpu().numpy(), run.lse.cpu().numpy(), rtol=0, atol=1e-6)
    # Exported partials are part-major, workspace partials row-major: the same arithmetic at
    # other addresses, so the forward without export gives the same bits.
    o_exp, l_exp = run.o.clone(), run.lse.clone()
    run.fwd()
    torch.cuda.synchronize()
    assert torch.equal(run.o, o_exp) and torch.equal(run.lse, l_exp), "workspace and export layouts differ"
    run.guard.check()
    # per-part statistics against the oracle's chunk partials (rows 0 and R-1)
    f = lambda x: synth.as_f64(x, W.dtype)
    rows = np.array([0, 255, W.R - 1])
    ref_o, ref_l = dense.chunk_partials(f(st["q"][0]), f(res["k_p"]), f(res["v_p"]), f(st["k_r"][0]),
                                        f(st["v_r"][0]), W.tau, dense.chunk_bounds(W.P, W.chunk), rows=rows)
    got_o = po.cpu().numpy()[:, 0][:, rows]
    got_l = pl.cpu().numpy()[:, 0][:, rows]
    assert_bf16_close("part_o", got_o, ref_o)
    assert np.max(np.abs(got_l - ref_l)) <= 2e-2


def test_merge_handles_empty_parts():
    po = torch.randn(3, 5, 8, device="cuda")
    pl = torch.randn(3, 5, device="cuda")
    pl[1] = float("-inf")
    pl[:, 4] = float("-inf")
    o = torch.empty(5, 8, device="cuda")
    lse = torch.empty(5, device="cuda")
    R.rr_lse_merge(po, pl, o, lse)
    ro, rl_ = dense.merge(po.double().cpu().numpy(), pl.double().cpu().numpy())
    np.testing.assert_allclose(o.cpu().numpy(), ro, atol=1e-6)
    assert np.isneginf(lse[4].item()) and np.all(o[4].cpu().numpy() == 0)
    np.testing.assert_allclose(lse.cpu().numpy()[:4], rl_[:4], atol=1e-6)


@pytest.mark.parametrize("n_parts,d_v", [(150, 512), (70, 70), (17, 128), (1, 64)])
def test_merge_many_parts_and_widths(n_parts, d_v):
    """rr_lse_merge over more parts than a wave has lanes, head dims that take several
    column passes or no 16-byte vectors, and one part: every element against the
    oracle's merge (fp32 inputs, fp64 reference), with -inf parts and an all-empty row."""
    g = torch.Generator().manual_seed(900 + n_parts)
    rows = 37
    po = torch.randn(n_parts, rows, d_v, generator=g)
    pl = 4.0 * torch.randn(n_parts, rows, generator=g)
    pl[::3, 5] = float("-inf")
    pl[:, 9] = float("-inf")
    if n_parts > 1:
        pl[1] = float("-inf")
    ref_o, ref_l = dense.merge(po.double().numpy(), pl.double().numpy())
    o = torch.full((rows, d_v), float("nan"), device="cuda")
    lse = torch.full((rows,), float("nan"), device="cuda")
    R.rr_lse_merge(po.cuda(), pl.cuda(), o, lse)
    torch.cuda.synchronize()
    np.testing.assert_allclose(o.cpu().numpy(), ref_o, rtol=0, atol=2e-5 * max(1.0, float(np.abs(ref_o).max())))
    assert np.isneginf(lse[9].item()) and np.all(o[9].cpu().numpy() == 0)
    keep = np.isfinite(ref_l)
    np.testing.assert_allclose(lse.cpu().numpy()[keep], ref_l[keep], rtol=0,
                               atol=2e-5 * (1.0 + float(np.abs(ref_l[keep]).max())))


def _group_runs(w, seed_version=7):
    """The members of a small group, each replayed against one shared resident prompt
    state (one device copy of K_p, V_p with one version), plus the oracle's gradients."""
    from tests import _gpu as G
    res = synth.resident(w)
    lens = [int(x) for x in synth.response_lengths(w)]
    shared = (G.to_dev(res["k_p"], w.dtype), G.to_dev(res["v_p"], w.dtype))
    runs, refs = [], []
    f = lambda x: synth.as_f64(x, w.dtype)
    for g, rg in enumerate(lens):
        m = synth.member(w, g, R=rg)
        st = G.stack_members([m], rg)
        prob = G.problem(w.P, rg, w.Hq, w.Hkv, w.d_qk, w.chunk, w.block, w.dtype, tau=w.tau)
        runs.append(G.Run(prob, w.dtype, None, None, st, [rg], version=seed_version, dev_resident=shared))
        refs.append(dense.attend_bwd(f(m["q"]), f(res["k_p"]), f(res["v_p"]), f(m["k_r"]), f(m["v_r"]),
                                     f(m["d_o"]), w.tau))
    return res, lens, shared, runs, refs


def _window(w, Rm, version=7):
    bufs = [torch.zeros(Rm, w.Hq, w.d_qk, device="cuda"), torch.zeros(Rm, w.Hkv, w.d_qk, device="cuda"),
            torch.zeros(Rm, w.Hkv, w.d_v, device="cuda")]
    return bufs, R.Accum(bufs, G=w.G, version=version)


def test_serial_group_accumulation():
    """G = 8 members replayed one at a time against one resident prompt state, accumulated
    into position-aligned fp32 buffers; equals the oracle's sum of 8 independent replays.
    Rejected before any launch: a retried member, gradients computed against a resident
    of another model version, gradients computed against another prompt group's resident,
    a tag that no backward wrote; a missing member is reported."""
    from tests import _gpu as G
    w = configs.FULL_P2M.with_(P=2048, R=192, r_min=64, chunk=512, block=64, seed=6001)
    res, lens, shared, runs, refs = _group_runs(w)
    bufs, win = _window(w, w.R)
    for g, run in enumerate(runs):
        run.fwd().bwd()
        grads = [run.dq[0], run.dk[0], run.dv[0]]
        R.rr_grad_accum(win, g, run.tag, grads)
        if g == 0:
            with pytest.raises(R.RRError) as e:
                R.rr_grad_accum(win, 0, run.tag, grads)
            assert e.value.code == R.RR_E_DUPLICATE
            with pytest.raises(R.RRError) as e:
                R.rr_accum_check_complete(win)
            assert e.value.code == R.RR_E_MISSING
        if g == 1:
            # the same member recomputed against the resident of a newer model version
            st2 = G.stack_members([synth.member(w, 2, R=lens[2])], lens[2])
            newer = G.Run(runs[2].p, w.dtype, None, None, st2, [lens[2]], version=8, dev_resident=shared)
            newer.fwd().bwd()
            with pytest.raises(R.RRError) as e:
                R.rr_grad_accum(win, 2, newer.tag, [newer.dq[0], newer.dk[0], newer.dv[0]])
            assert e.value.code == R.RR_E_STALE and "version" in str(e.value)
            # ... against another prompt group's resident state (same version, other buffers)
            other = G.Run(runs[2].p, w.dtype, res["k_p"], res["v_p"], st2, [lens[2]], version=7)
            other.fwd().bwd()
            with pytest.raises(R.RRError) as e:
                R.rr_grad_accum(win, 2, other.tag, [other.dq[0], other.dk[0], other.dv[0]])
            assert e.value.code == R.RR_E_STALE and "resident" in str(e.value)
            # ... and a tag no backward wrote
            forged = R.CGradTag(version=7, resident=run.tag.resident, P=run.tag.P, seal=0)
            with pytest.raises(R.RRError) as e:
                R.rr_grad_accum(win, 2, forged, [other.dq[0], other.dk[0], other.dv[0]])
            assert e.value.code == R.RR_E_STALE
            assert bytes(win.seen) == bytes([1, 1] + [0] * (w.G - 2))   # rejections leave the mask alone
    R.rr_accum_check_complete(win)
    torch.cuda.synchronize()
    assert_bf16_close("acc dq", bufs[0].cpu().numpy(), dense.accumulate([r["dq"] for r in refs], w.R))
    assert_bf16_close("acc dk", bufs[1].cpu().numpy(), dense.accumulate([r["dk_r"] for r in refs], w.R))
    assert_bf16_close("acc dv", bufs[2].cpu().numpy(), dense.accumulate([r["dv_r"] for r in refs], w.R))


def test_accumulation_replay_order_and_microbatch():
    """The update-boundary sum does not depend on the schedule that produced it: the same
    G = 8 members replayed in a permuted order, and replayed as two microbatches of
    K = 4 stacked responses each (other call sizes, other padding), accumulate to the
    in-order serial result up to fp32 addition order, and to the oracle's sum."""
    from tests import _gpu as G
    w = configs.FULL_P2M.with_(P=2048, R=192, r_min=64, chunk=512, block=64, seed=6002)
    res, lens, shared, runs, refs = _group_runs(w)
    bufs_a, win_a = _window(w, w.R)
    for g, run in enumerate(runs):
        run.fwd().bwd()
        R.rr_grad_accum(win_a, g, run.tag, [run.dq[0], run.dk[0], run.dv[0]])
    order = [5, 2, 7, 0, 3, 6, 1, 4]
    bufs_b, win_b = _window(w, w.R)
    for g in order:
        run = runs[g].fwd().bwd()
        R.rr_grad_accum(win_b, g, run.tag, [run.dq[0], run.dk[0], run.dv[0]])
    bufs_c, win_c = _window(w, w.R)
    for b0 in (4, 0):                       # the later microbatch first
        gs = list(range(b0, b0 + 4))
        rm = max(lens[g] for g in gs)
        mem = [synth.member(w, g, R=lens[g]) for g in gs]
        prob = G.problem(w.P, rm, w.Hq, w.Hkv, w.d_qk, w.chunk, w.block, w.dtype, K=4, tau=w.tau)
        mb = G.Run(prob, w.dtype, None, None, G.stack_members(mem, rm), [lens[g] for g in gs], version=7,
                   dev_resident=shared).fwd().bwd()
        for i, g in enumerate(gs):
            rg = lens[g]
            R.rr_grad_accum(win_c, g, mb.tag, [mb.dq[i, :rg], mb.dk[i, :rg], mb.dv[i, :rg]])
    for win in (win_a, win_b, win_c):
        R.rr_accum_check_complete(win)
    torch.cuda.synchronize()
    for n, key in enumerate(("dq", "dk_r", "dv_r")):
        a = bufs_a[n].double().cpu().numpy()
        scale = max(1.0, float(np.abs(a).max()))
        for other in (bufs_b, bufs_c):
            assert np.max(np.abs(other[n].double().cpu().numpy() - a)) <= 1e-5 * scale, key
        assert_bf16_close(f"permuted acc {key}", bufs_b[n].cpu().numpy(),
                          dense.accumulate([r[key] for r in refs], w.R))
        assert_bf16_close(f"microbatch acc {key}", bufs_c[n].cpu().numpy(),
                          dense.accumulate([r[key] for r in refs], w.R))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_microbatch_equals_single_calls(dtype):
    """A call over K stacked, zero-padded responses gives, for each response, exactly the
    bits that a call over that response alone gives: responses never read one another,
    and the per-row arithmetic does not depend on K, on the padded length or on where in
    the batch a response sits."""
    from tests import _gpu as G
    base = W if dtype == "bf16" else configs.TINY_F32.with_(P=700, R=90, seed=5002)
    lens = [520, 300, 65, 1] if dtype == "bf16" else [90, 41, 7]
    w = base.with_(R=max(lens))
    res = synth.resident(w)
    mem = [synth.member(w, g, R=r) for g, r in enumerate(lens)]
    chunk, block = (1024, 128) if dtype == "bf16" else (256, 32)
    st = G.stack_members(mem, max(lens))
    prob = G.problem(w.P, max(lens), w.Hq, w.Hkv, w.d_qk, chunk, block, w.dtype, K=len(lens),
                     tau=w.tau)
    print(f"[microbatch] {dtype} K={len(lens)} R={lens}", flush=True)
    many = G.Run(prob, w.dtype, res["k_p"], res["v_p"], st, lens).fwd().bwd().numpy()
    for kk, rl in enumerate(lens):
        st1 = G.stack_members([mem[kk]], rl)
        p1 = G.problem(w.P, rl, w.Hq, w.Hkv, w.d_qk, chunk, block, w.dtype, tau=w.tau)
        one = G.Run(p1, w.dtype, res["k_p"], res["v_p"], st1, [rl]).fwd().bwd().numpy()
        for key in ("o", "lse", "dq", "dk", "dv", "D"):
            np.testing.assert_array_equal(many[key][kk][:rl], one[key][0], err_msg=f"{key}[k={kk}]")


def test_microbatch_full_size_group():
    """The 2M group (P = 2,097,152, members of 2159 to 7666 rows) as one call with K = 8
    gives every member exactly the bits of its own call, D included, and zeros in each
    member's padding rows."""
    from tests import _gpu as G
    w = configs.FULL_P2M
    lens = [int(r) for r in synth.response_lengths(w)]
    res = synth.resident(w)
    mem = [synth.member(w, g, R=r) for g, r in enumerate(lens)]
    st = G.stack_members(mem, w.R)
    prob = G.problem(w.P, w.R, w.Hq, w.Hkv, w.d_qk, w.chunk, w.block, w.dtype, K=len(lens), tau=w.tau)
    print(f"[microbatch] full size K={len(lens)} R={lens}", flush=True)
    many = G.Run(prob, w.dtype, res["k_p"], res["v_p"], st, lens).fwd().bwd().numpy()
    for kk, rl in enumerate(lens):
        print(f"[microbatch] member {kk} alone", flush=True)
        p1 = G.problem(w.P, rl, w.Hq, w.Hkv, w.d_qk, w.chunk, w.block, w.dtype, tau=w.tau)
        one = G.Run(p1, w.dtype, res["k_p"], res["v_p"], G.stack_members([mem[kk]], rl), [rl]).fwd().bwd().numpy()
        for key in ("o", "lse", "dq", "dk", "dv", "D"):
            np.testing.assert_array_equal(many[key][kk][:rl], one[key][0], err_msg=f"{key}[k={kk}]")
        assert np.all(many["o"][kk][rl:] == 0) and np.all(np.isneginf(many["lse"][kk][rl:]))
        for key in ("dq", "dk", "dv", "D"):
            assert np.all(many[key][kk][rl:] == 0), key

