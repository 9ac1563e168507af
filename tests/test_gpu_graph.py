"""The entry points launch asynchronously on the caller's stream with no allocation and no
synchronisation, so a caller can capture them into a HIP graph (needs an MI355X).

One member's forward, backward and update-boundary accumulation are captured once and
replayed several times, with eager work between the replays (clearing the accumulators,
poisoning the outputs with NaN); every replay must give, bit for bit, what the same calls
give when run eagerly."""
import numpy as np
import pytest
import torch

from resident_kv_response_amd import configs, rr_attn as R, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_graph_replays_equal_eager(dtype):
    from tests import _gpu as G
    base = configs.GQA_P128K.with_(P=5000, R=300, Hq=8, Hkv=2, chunk=2048, block=128, seed=4400)
    w = base if dtype == "bf16" else configs.TINY_F32.with_(P=700, R=90, seed=4401)
    res = synth.resident(w)
    st = G.stack_members([synth.member(w, 0)], w.R)
    prob = G.problem(w.P, w.R, w.Hq, w.Hkv, w.d_qk, w.chunk, w.block, w.dtype, tau=w.tau)
    shared = (G.to_dev(res["k_p"], w.dtype), G.to_dev(res["v_p"], w.dtype))

    def window(run):
        bufs = [torch.zeros_like(run.dq[0]), torch.zeros_like(run.dk[0]), torch.zeros_like(run.dv[0])]
        return bufs, R.Accum(bufs, G=1, version=3)

    print(f"[graph] {dtype} eager", flush=True)
    eager = G.Run(prob, w.dtype, None, None, st, [w.R], version=3, dev_resident=shared)
    eager.fwd().bwd()
    acc_e, win_e = window(eager)
    R.rr_grad_accum(win_e, 0, eager.tag, [eager.dq[0], eager.dk[0], eager.dv[0]])
    ref = eager.numpy()
    ref_acc = [t.cpu().numpy() for t in acc_e]

    run = G.Run(prob, w.dtype, None, None, st, [w.R], version=3, dev_resident=shared)
    acc_g, win_g = window(run)
    graph = torch.cuda.CUDAGraph()
    print(f"[graph] {dtype} capture", flush=True)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run.fwd().bwd()
        R.rr_grad_accum(win_g, 0, run.tag, [run.dq[0], run.dk[0], run.dv[0]])
    for rep in range(3):
        for t in acc_g:
            t.zero_()
        for t in (run.o, run.lse, run.dq, run.dk, run.dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        print(f"[graph] {dtype} replay {rep}", flush=True)
        graph.replay()
        got = run.numpy()
        for key in ("o", "lse", "dq", "dk", "dv", "D"):
            np.testing.assert_array_equal(got[key], ref[key], err_msg=f"replay {rep}: {key}")
        for n, t in enumerate(acc_g):
            np.testing.assert_array_equal(t.cpu().numpy(), ref_acc[n], err_msg=f"replay {rep}: accumulator {n}")
