"""Benchmark: response-replay attention fwd + response-only bwd at a 2,097,152-position
resident prompt (one GPU).

One step = one group of G = 8 members replayed serially, K members per call (replay
microbatch K, default 1; --microbatch K stacks K consecutive members, zero-padded to the
longest of them, into one call).  Each call runs rr_attn_fwd (chunk partials + exact
merge) and rr_attn_bwd (D, dQ partials + ordered reduction, reverse block walk for
response dK/dV); each member's dQ, dK, dV then go through rr_grad_accum into
position-aligned fp32 accumulators (zeroed at the start of the group).  All inputs are
synthetic (seeded N(0,1), rounded to bf16) and resident in HBM before timing starts.

With --full-sequence every call also forms the prompt K/V gradients (rr_attn_prompt_grads,
summed over the group): the term the response-only contract drops, for differential
comparison.  `value` then counts its flops too, and the line reports the gradient norms
and the cosine between the response-only and the full gradient at the attention boundary.

With --workload bf16_lastkv_P2097152_C8192 a step is one layer's current chunk of a LastKV
recurrence (8192 positions after 2,097,152 of history): the previous chunk's blend,
forward, response-only backward, the blended chunk's gradient and the blend's backward.

With --workload bf16_latent_P1048576_R4096_top2048 a step is one response of the
latent-page top-k variant: fp32 index scores, exact top-2048 selection, sparse attention
forward and response-only backward (64 heads sharing 576-wide latent rows).

Prints one JSON line.  `value` is algorithmic TFLOP/s of the whole step; `roofline` is
measured live for the kernel with the largest device time, from HIP events the library
records around every launch in the timed region.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="bf16_full_P2097152_G8")
    ap.add_argument("--cpu-rows", type=int, default=24, help="oracle sample rows (0 = skip)")
    ap.add_argument("--microbatch", type=int, default=1,
                    help="replay microbatch K: the group's members run as calls of K responses each")
    ap.add_argument("--full-sequence", action="store_true",
                    help="full-sequence differential mode: every call also forms the prompt K/V "
                         "gradients (rr_attn_prompt_grads), summed over the group")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device copy and exit: the reference kernel for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes")
    return ap.parse_args()


def copy_calibration() -> int:
    """One device copy of 2^28 fp32 (1 GiB read, 1 GiB written), for the counter scale."""
    import torch

    x = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": x.numel() * 4}))
    return 0


def kernel_flops(w, R: int) -> dict:
    """Algorithmic flops of each launch kind for one member of length R (d_qk = d_v = d).
    dq_partials: S, dP and dQ over every visible pair; fwd_partials: S and PV over every
    visible pair; dkdv: S, dP, dK and dV over the response pairs; prompt_dkdv (full-sequence
    mode only): S, dP, dK and dV over every (row, prompt key) pair.  Each is the set of
    contractions that kernel performs (without stored scores, a key-parallel gradient kernel
    recomputes S and dP).  These are per-kernel figures: the step's value counts every pair's
    S and dP once (configs.flops_dense), so the recomputation in dkdv adds nothing to it."""
    d, Hq = w.d_qk, w.Hq
    n_p, n_r = R * w.P, R * (R + 1) // 2
    return {"fwd_partials": 4.0 * d * Hq * (n_p + n_r),
            "dq_partials": 6.0 * d * Hq * (n_p + n_r),
            "dkdv": 8.0 * d * Hq * n_r,
            "prompt_dkdv": 8.0 * d * Hq * n_p}


def traffic_from_profiles(kernel: str, workload: str, src_sha: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != src_sha:
        return None
    try:
        return float(fields["hbm_bytes_per_launch_for_bench_member_mean"])
    except (KeyError, ValueError):
        return None


KERNEL_SOURCES = {
    "fwd_partials": ["k_fwd_bf16.hip", "k_ring.h", "k_lds.h", "k_addr.h", "k_attn_tile.h", "k_common.h"],
    "dq_partials": ["k_dq_bf16.hip", "k_ring.h", "k_lds.h", "k_addr.h", "k_attn_tile.h", "k_common.h"],
    "dkdv": ["k_kv_grads.hip", "k_split.h", "k_ring.h", "k_lds.h", "k_addr.h", "k_attn_tile.h", "k_common.h"],
    "prompt_dkdv": ["k_kv_grads.hip", "k_split.h", "k_ring.h", "k_lds.h", "k_addr.h", "k_attn_tile.h",
                    "k_common.h"],
}


def source_sha(files) -> str:
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "resident_kv_response_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def main() -> int:
    a = _args()
    if a.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU (no path across GPUs); --gpus must be 1",
                          "n_gpus_requested": a.gpus}))
        return 2
    if a.copy_calibration:
        return copy_calibration()
    from resident_kv_response_amd import configs

    w = configs.BY_NAME[a.workload]
    if w.latent:
        return run_latent(a, w)
    if "lastkv" in w.name:
        return run_lastkv(a, w)
    return run_dense(a, w)


def run_dense(a, w) -> int:
    import torch

    from resident_kv_response_amd import configs, rr_attn as R, synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    lens = synth.response_lengths(w) if w.G > 1 else np.array([w.R])
    Rmax = int(lens.max())

    t0 = time.time()
    res = synth.resident(w)

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)

    k_p, v_p = up(res["k_p"]), up(res["v_p"])
    members = []
    host_m0 = None
    for g, rg in enumerate(lens):
        m = synth.member(w, g, R=int(rg))
        if g == 0:
            host_m0 = m
        members.append({k: up(v)[None] for k, v in m.items()})
    gen_s = time.time() - t0

    kv = R.resident(k_p, v_p, version=1)
    Kmb = max(1, min(int(a.microbatch), len(lens)))
    # microbatches: consecutive members, K per call; inputs stacked [K][R_max][...] and
    # zero-padded (rows past a member's length are padding rows of the call)
    mbs = []
    for b0 in range(0, len(lens), Kmb):
        gs = list(range(b0, min(b0 + Kmb, len(lens))))
        rmax_b = int(max(lens[g] for g in gs))
        st = {}
        for key in ("q", "k_r", "v_r", "d_o"):
            t = torch.zeros((len(gs), rmax_b) + tuple(members[0][key].shape[2:]), device=dev,
                            dtype=torch.bfloat16)
            for i, g in enumerate(gs):
                t[i, :int(lens[g])] = members[g][key][0]
            st[key] = t
        prob = R.Problem(P=w.P, R_max=rmax_b, Hq=w.Hq, Hkv=w.Hkv, d_qk=w.d_qk, d_v=w.d_v,
                         chunk=w.chunk, block=w.block, tau=w.tau, K=len(gs))
        mbs.append((gs, [int(lens[g]) for g in gs], st, prob))
    members = None   # the stacked copies are the resident inputs now
    pmax = R.Problem(P=w.P, R_max=Rmax, Hq=w.Hq, Hkv=w.Hkv, d_qk=w.d_qk, d_v=w.d_v, chunk=w.chunk,
                     block=w.block, tau=w.tau, K=Kmb)
    ws_f = R.workspace(pmax, R.RR_OP_FWD, dev)
    ws_b = R.workspace(pmax, R.RR_OP_BWD, dev)
    f32 = dict(device=dev, dtype=torch.float32)
    # flat output buffers; a call of K responses of stride R_max uses their leading part
    row_elems = {"o": w.Hq * w.d_v, "lse": w.Hq, "dq": w.Hq * w.d_qk, "dk": w.Hkv * w.d_qk, "dv": w.Hkv * w.d_v}
    flat = {n: torch.empty(Kmb * Rmax * e, **f32) for n, e in row_elems.items()}
    shape = {"o": (w.Hq, w.d_v), "lse": (w.Hq,), "dq": (w.Hq, w.d_qk), "dk": (w.Hkv, w.d_qk),
             "dv": (w.Hkv, w.d_v)}

    def outs(K, rm):
        return [flat[n][:K * rm * row_elems[n]].view((K, rm) + shape[n]) for n in ("o", "lse", "dq", "dk", "dv")]
    acc = [torch.zeros(Rmax, w.Hq, w.d_qk, **f32), torch.zeros(Rmax, w.Hkv, w.d_qk, **f32),
           torch.zeros(Rmax, w.Hkv, w.d_v, **f32)]
    full = bool(a.full_sequence)
    if full:   # the group's prompt K/V gradients, summed over its members
        dk_p = torch.empty(w.P, w.Hkv, w.d_qk, **f32)
        dv_p = torch.empty(w.P, w.Hkv, w.d_v, **f32)
        ws_pg = R.workspace(pmax, R.RR_OP_PROMPT_GRADS, dev)

    def mb_pass(b, win=None):
        gs, rls, st, prob = mbs[b]
        og, lg, dqg, dkg, dvg = outs(len(gs), prob.R_max)
        R.rr_attn_fwd(prob, kv, st["q"], st["k_r"], st["v_r"], rls, o=og, lse=lg, ws=ws_f)
        tag = R.rr_attn_bwd(prob, kv, st["q"], st["k_r"], st["v_r"], rls, og, lg, st["d_o"], dqg, dkg, dvg,
                            ws=ws_b)
        if full:
            R.rr_attn_prompt_grads(prob, kv, st["q"], rls, og, lg, st["d_o"], dk_p, dv_p,
                                   accumulate=1 if b > 0 else 0, ws=ws_pg)
        if win is not None:
            for i, g in enumerate(gs):
                rg = rls[i]
                R.rr_grad_accum(win, g, tag, [dqg[i, :rg], dkg[i, :rg], dvg[i, :rg]])

    def step():
        for t in acc:
            t.zero_()
        win = R.Accum(acc, G=len(lens), version=1)
        for b in range(len(mbs)):
            mb_pass(b, win)
        R.rr_accum_check_complete(win)

    # parity gate on member 0 (sampled rows, one KV group) before any timing
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    mb_pass(0)
    torch.cuda.synchronize()
    mem_g1 = torch.cuda.max_memory_allocated()
    rows = synth.sample_rows(w.seed, int(lens[0]), a.cpu_rows, w.block) if a.cpu_rows > 0 else None
    got = None
    if rows is not None:
        grp = w.Hq // w.Hkv
        o0, _, dq0, dk0, dv0 = outs(len(mbs[0][0]), mbs[0][3].R_max)
        r0 = int(lens[0])
        got = {"o": o0[0, rows, :grp].double().cpu().numpy(), "dq": dq0[0, rows, :grp].double().cpu().numpy(),
               # response-key gradients of member 0's last TAIL keys, KV head 0 (only its last
               # TAIL positions reach them)
               "dk": dk0[0, r0 - TAIL:r0, 0].double().cpu().numpy(),
               "dv": dv0[0, r0 - TAIL:r0, 0].double().cpu().numpy()}

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    R.rr_profile_begin()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    prof = R.rr_profile_end()
    mem_g8 = torch.cuda.max_memory_allocated()
    ms_per_step = (t2 - t1) * 1e3 / a.steps

    flops_step = 0.0
    per_kernel_flops = {"fwd_partials": 0.0, "dq_partials": 0.0, "dkdv": 0.0}
    if full:
        per_kernel_flops["prompt_dkdv"] = 0.0
    for rg in lens:
        kf = kernel_flops(w, int(rg))
        flops_step += configs.flops_dense(w.Hq, w.d_qk, w.d_v, int(rg), w.P)["total"]
        if full:
            flops_step += kf["prompt_dkdv"]
        for k in per_kernel_flops:
            per_kernel_flops[k] += kf[k]
    tflops = flops_step / (ms_per_step * 1e-3) / 1e12
    tokens_s = float(lens.sum()) / (ms_per_step * 1e-3)

    # dominant kernel by device time
    dom = max(prof.items(), key=lambda kv_: kv_[1][1])
    dom_name, (dom_launches, dom_ms) = dom[0], dom[1]
    roof = None
    if dom_name in per_kernel_flops:
        launches_per_step = dom_launches / a.steps
        flops_per_launch = per_kernel_flops[dom_name] / launches_per_step
        avg_ms = dom_ms / dom_launches
        achieved = flops_per_launch / (avg_ms * 1e-3) / 1e12
        src = KERNEL_SOURCES[dom_name]
        roof = {"bound": "mfma", "kernel": dom_name, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_from_profiles(dom_name, w.name, source_sha(src)),
                "avg_launch_ms": round(avg_ms, 4), "flops_per_launch": flops_per_launch}
    kernels = {k: {"launches_per_step": v[0] / a.steps, "ms_per_step": round(v[1] / a.steps, 3)}
               for k, v in sorted(prof.items(), key=lambda kv_: -kv_[1][1])}
    for k in per_kernel_flops:
        if k in kernels:
            kernels[k]["tflops"] = round(per_kernel_flops[k] / (kernels[k]["ms_per_step"] * 1e-3) / 1e12, 2)
    # HBM-bound phases: algorithmic bytes per step / device time, against 8 TB/s
    n_rows = float(sum(int(rg) for rg in lens)) * w.Hq    # (row, head) pairs of the group
    hbm_bytes = {
        # read every part's partial (O and lse), write O and lse
        "lse_merge": n_rows * (w.n_chunks + 2) * (w.d_v + 1) * 4,
        # read O (fp32) and dO (bf16), write D
        "bwd_pre": n_rows * (w.d_v * 6 + 4),
        # read every part's dQ partial, write dQ
        "dq_reduce": n_rows * (w.n_chunks + 2) * w.d_qk * 4,
        # read the member's dQ, dK, dV and the accumulators, write the accumulators
        "grad_accum": 12.0 * sum(int(rg) * (w.Hq * w.d_qk + w.Hkv * (w.d_qk + w.d_v)) for rg in lens),
    }
    for k, nb in hbm_bytes.items():
        if k in kernels and kernels[k]["ms_per_step"] > 0:
            gbs = nb / (kernels[k]["ms_per_step"] * 1e-3) / 1e9
            kernels[k]["gbs"] = round(gbs, 1)
            kernels[k]["hbm_frac"] = round(gbs / PEAK_HBM_GBS, 3)

    # CPU baseline: the oracle on the machine's host cores, on bounded legs of the work (the
    # tiny fp32 configuration in full, sampled 2M rows, and the 2M response-key gradients of
    # member 0's last keys); the full step's oracle time is an extrapolation at the
    # measured oracle rate
    cpu = None
    parity = None
    if rows is not None:
        from oracle import dense
        try:
            from threadpoolctl import threadpool_info
            blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            blas_threads = None
        grp = w.Hq // w.Hkv
        f = lambda x: synth.as_f64(x, w.dtype)
        legs = []
        # leg 1: the tiny fp32 configuration, every row, forward and full response-only backward
        wt = configs.TINY_F32
        rt, mt = synth.resident(wt), synth.member(wt, 0)
        ft = lambda x: synth.as_f64(x, wt.dtype)
        tc = time.perf_counter()
        dense.attend(ft(mt["q"]), ft(rt["k_p"]), ft(rt["v_p"]), ft(mt["k_r"]), ft(mt["v_r"]), wt.tau)
        dense.attend_bwd(ft(mt["q"]), ft(rt["k_p"]), ft(rt["v_p"]), ft(mt["k_r"]), ft(mt["v_r"]), ft(mt["d_o"]),
                         wt.tau)
        legs.append({"leg": f"{wt.name}, all {wt.R} rows x {wt.Hq} heads, fwd + bwd (dQ, dK_r, dV_r)",
                     "flops": configs.flops_dense(wt.Hq, wt.d_qk, wt.d_v, wt.R, wt.P)["total"],
                     "s": time.perf_counter() - tc})
        # leg 2: sampled rows of member 0 over all P prompt keys (also the parity gate)
        kp64, vp64 = f(res["k_p"][:, :1]), f(res["v_p"][:, :1])
        qs, kr, vr, do = f(host_m0["q"][:, :grp]), f(host_m0["k_r"][:, :1]), f(host_m0["v_r"][:, :1]), \
            f(host_m0["d_o"][:, :grp])
        tc = time.perf_counter()
        ro, _ = dense.attend(qs, kp64, vp64, kr, vr, w.tau, rows=rows)
        rgr = dense.attend_bwd(qs, kp64, vp64, kr, vr, do, w.tau, rows=rows)
        legs.append({"leg": f"member 0 (R={int(lens[0])}): {len(rows)} sampled query rows "
                            f"{list(map(int, rows))} x KV head 0's {grp} query heads, fwd + dQ over all "
                            f"{w.P} prompt keys and the causal response keys",
                     "flops": sum(grp * 10.0 * w.d_qk * (w.P + int(r) + 1) for r in rows),
                     "s": time.perf_counter() - tc})
        # leg 3: the response-key gradients dK_r, dV_r of member 0's last TAIL keys (KV head
        # 0): every head of its last TAIL positions, forward and backward over all keys
        r0 = int(lens[0])
        tail_rows = np.repeat(np.arange(r0 - TAIL, r0), grp)
        tail_heads = np.tile(np.arange(grp), TAIL)
        tc = time.perf_counter()
        rt_ = dense.attend_rows(qs, kp64, vp64, kr, vr, do, w.tau, tail_rows, tail_heads)
        legs.append({"leg": f"member 0: dK_r, dV_r of its last {TAIL} keys (KV head 0) from every head "
                            f"of its last {TAIL} positions, fwd + bwd over all keys",
                     "flops": sum(grp * 10.0 * w.d_qk * (w.P + int(r) + 1) for r in range(r0 - TAIL, r0)),
                     "s": time.perf_counter() - tc})
        cpu_s = sum(l["s"] for l in legs)
        cpu_flops = sum(l["flops"] for l in legs)
        for l in legs:
            l["tflops"] = round(l["flops"] / l["s"] / 1e12, 6)
            l["s"] = round(l["s"], 2)
        cores = len(os.sched_getaffinity(0))
        cpu = {"value": round(cpu_flops / cpu_s / 1e12, 6), "unit": "TFLOP/s",
               "cores": blas_threads or cores, "kind": "oracle",
               "sample": "; ".join(l["leg"] for l in legs) + f" ({cpu_s:.1f} s in all)",
               "legs": legs, "host_cpus_affinity": cores, "host_cpu_count": os.cpu_count(),
               "extrapolated_full_step_s": round(flops_step / (cpu_flops / cpu_s), 1),
               "extrapolation": "the full G=8 group at the oracle's measured rate (not run)"}
        rel = lambda x, y: float(np.linalg.norm(x - y) / np.linalg.norm(y))
        parity = {"rows": len(rows), "o_rel_l2": rel(got["o"], ro), "dq_rel_l2": rel(got["dq"], rgr["dq"]),
                  "o_max_abs": float(np.abs(got["o"] - ro).max()),
                  "dq_max_abs": float(np.abs(got["dq"] - rgr["dq"]).max()),
                  "tail_keys": TAIL,
                  "dk_rel_l2": rel(got["dk"], rt_["dk_r"][r0 - TAIL:r0, 0]),
                  "dv_rel_l2": rel(got["dv"], rt_["dv_r"][r0 - TAIL:r0, 0]),
                  "dk_max_abs": float(np.abs(got["dk"] - rt_["dk_r"][r0 - TAIL:r0, 0]).max()),
                  "dv_max_abs": float(np.abs(got["dv"] - rt_["dv_r"][r0 - TAIL:r0, 0]).max())}
        parity["pass"] = bool(all(parity[k] <= 5e-3 for k in ("o_rel_l2", "dq_rel_l2", "dk_rel_l2", "dv_rel_l2"))
                              and all(parity[k] <= 2e-2 for k in ("o_max_abs", "dq_max_abs", "dk_max_abs",
                                                                   "dv_max_abs")))

    fs = None
    if full:   # norms of the group's response-side and prompt-side gradients after the last step
        nrm = lambda x: float(torch.linalg.vector_norm(x, dtype=torch.float64))
        n_resp = float(np.sqrt(sum(nrm(t) ** 2 for t in acc)))
        n_prompt = float(np.sqrt(nrm(dk_p) ** 2 + nrm(dv_p) ** 2))
        fs = {"prompt_flops_per_step": float(sum(kernel_flops(w, int(rg))["prompt_dkdv"] for rg in lens)),
              "norm_response_grads": n_resp, "norm_dk_p": nrm(dk_p), "norm_dv_p": nrm(dv_p),
              "cosine_response_only_vs_full": n_resp / float(np.hypot(n_resp, n_prompt)),
              "note": "gradient vector (dQ, dK_r, dV_r, dK_p, dV_p) of the group at the attention "
                      "boundary; the response-only vector has dK_p = dV_p = 0"}

    out = {
        "metric": "response-replay attention fwd+bwd TFLOP/s + % bf16 MFMA peak at P=2M"
                  + (", full-sequence differential mode" if full else ""),
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_per_step, 2), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "P": w.P, "G": len(lens), "R_g": [int(x) for x in lens],
                   "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d_qk, "chunk": w.chunk, "block": w.block,
                   "replay_microbatch": Kmb, "flops_per_step": flops_step,
                   "mode": "full_sequence" if full else "response_only"},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "tokens_per_s": round(tokens_s, 1),
        "roofline": roof, "cpu_baseline": cpu, "parity": parity, "kernels": kernels,
        "full_sequence": fs,
        "peak_mem_bytes": {"after_1_microbatch": int(mem_g1), "timed_G_groups": int(mem_g8)},
        "input_gen_s": round(gen_s, 1),
    }
    print(json.dumps(out), flush=True)
    return 0 if (parity is None or parity["pass"]) else 1


LATENT_SOURCES = {
    "topk_select": ["k_topk.hip", "k_common.h", "k_lds.h", "k_addr.h"],
    "sparse_fwd": ["k_sparse.hip", "k_lds.h", "k_addr.h", "k_common.h"],
    "sparse_dq": ["k_sparse.hip", "k_lds.h", "k_addr.h", "k_common.h"],
    "xty_dk": ["k_sparse.hip", "k_lds.h", "k_addr.h", "k_common.h"],
    "xty_dv": ["k_sparse.hip", "k_lds.h", "k_addr.h", "k_common.h"],
}


TAIL = 32   # response keys of member 0 whose dK_r / dV_r the bench's oracle leg checks


def latent_kernel_model(w, R: int) -> dict:
    """Algorithmic flops / HBM bytes of each launch kind for one response of length R of
    the latent-page variant.  Bytes count each selected latent row once per query row
    (the gather), every other operand once; response rows re-read by later query rows
    are not counted (they are a few MB and stay in cache)."""
    H, dk, dv, P, k, di = w.Hq, w.d_qk, w.d_v, w.P, w.topk, w.idx_dim
    n_p, n_r = R * k, R * (R + 1) // 2
    row = dk * 2
    q_b, do_b = R * H * dk * 2, R * H * dv * 2
    return {
        # the index contraction (2 di flops per score) runs as three bf16 products per
        # element on the matrix cores (hi/lo split), so its peak is a third of bf16's;
        # bytes: the index keys and queries once, the selection out
        "topk_select": {"flops": 2.0 * di * R * P, "peak": PEAK_BF16_TFLOPS / 3.0,
                        "bytes": P * di * 4 + R * di * 4 + R * k * 4},
        "sparse_fwd": {"flops": H * (2.0 * dk + 2.0 * dv) * (n_p + n_r), "peak": PEAK_BF16_TFLOPS,
                       "bytes": n_p * row + R * row + q_b + R * H * (dv + 1) * 4 + R * k * 4},
        "sparse_dq": {"flops": H * (4.0 * dk + 2.0 * dv) * (n_p + n_r), "peak": PEAK_BF16_TFLOPS,
                      "bytes": n_p * row + R * row + q_b + do_b + R * H * dk * 4 + 2 * H * n_r * 2},
        "xty_dk": {"flops": H * 2.0 * dk * n_r, "peak": PEAK_BF16_TFLOPS,
                   "bytes": H * n_r * 2 + q_b + R * dk * 4},
        "xty_dv": {"flops": H * 2.0 * dv * n_r, "peak": PEAK_BF16_TFLOPS,
                   "bytes": H * n_r * 2 + do_b + R * dv * 4},
    }


def roofline_entry(name, model, launches_per_step, avg_ms, traffic):
    """The bound with the longer ideal time decides: MFMA (flops / peak) or HBM (bytes /
    8 TB/s)."""
    t_f = model["flops"] / (model["peak"] * 1e12) if model["peak"] else 0.0
    t_b = model["bytes"] / (PEAK_HBM_GBS * 1e9)
    per = 1.0 / launches_per_step
    if t_f >= t_b:
        ach = model["flops"] * per / (avg_ms * 1e-3) / 1e12
        return {"bound": "mfma", "kernel": name, "achieved": round(ach, 2), "peak": model["peak"],
                "unit": "TFLOP/s", "frac": round(ach / model["peak"], 4), "traffic": traffic,
                "avg_launch_ms": round(avg_ms, 4), "flops_per_launch": model["flops"] * per,
                "algorithmic_bytes_per_launch": model["bytes"] * per}
    ach = model["bytes"] * per / (avg_ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": name, "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic,
            "avg_launch_ms": round(avg_ms, 4), "algorithmic_bytes_per_launch": model["bytes"] * per,
            "flops_per_launch": model["flops"] * per}


def run_lastkv(a, w) -> int:
    """One layer's current chunk of a LastKV recurrence (C = w.R positions after w.P of
    history): blend of the previous chunk (K, V), forward, response-only backward of the
    chunk, the blended chunk's gradient (rr_attn_prompt_grads over its key range) and the
    blend's backward (both K/V sources and the gate)."""
    import torch

    from resident_kv_response_amd import configs, rr_attn as R, synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    C, P = w.R, w.P
    t0 = time.time()
    x = synth.lastkv_chunk(w)

    def up(v):
        return torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).to(dev).view(torch.bfloat16)

    hist_k, hist_v = up(x["k_last"]), up(x["v_last"])           # the previous chunk's slot: [P-C, P)
    kL_prev, vL_prev = hist_k[P - C:].clone(), hist_v[P - C:].clone()
    kl_prev, vl_prev = up(x["k_prev_layer"]), up(x["v_prev_layer"])
    q, k_cur, v_cur, d_o = (up(x[n])[None] for n in ("q", "k_cur", "v_cur", "d_o"))
    alpha = torch.tensor(x["alpha"], device=dev)
    gen_s = time.time() - t0
    kv = R.resident(hist_k, hist_v, version=1)
    prob = R.Problem(P=P, R_max=C, Hq=w.Hq, Hkv=w.Hkv, d_qk=w.d_qk, d_v=w.d_v, chunk=w.chunk, block=w.block,
                     tau=w.tau, K=1)
    ws_f = R.workspace(prob, R.RR_OP_FWD, dev)
    ws_b = R.workspace(prob, R.RR_OP_BWD, dev)
    ws_pg = R.workspace(prob, R.RR_OP_PROMPT_GRADS, dev)
    f32 = dict(device=dev, dtype=torch.float32)
    o = torch.empty(1, C, w.Hq, w.d_v, **f32)
    lse = torch.empty(1, C, w.Hq, **f32)
    dq = torch.empty(1, C, w.Hq, w.d_qk, **f32)
    dk = torch.empty(1, C, w.Hkv, w.d_qk, **f32)
    dv = torch.empty(1, C, w.Hkv, w.d_v, **f32)
    dkb = torch.empty(C, w.Hkv, w.d_qk, **f32)
    dvb = torch.empty(C, w.Hkv, w.d_v, **f32)
    g_src = {n: torch.empty(C, w.Hkv, w.d_qk, **f32) for n in ("kl", "kL", "vl", "vL")}
    d_alpha = torch.empty(w.Hkv, **f32)

    def step():
        R.rr_lastkv_blend(alpha, kl_prev, kL_prev, hist_k[P - C:])
        R.rr_lastkv_blend(alpha, vl_prev, vL_prev, hist_v[P - C:])
        R.rr_attn_fwd(prob, kv, q, k_cur, v_cur, [C], o=o, lse=lse, ws=ws_f)
        R.rr_attn_bwd(prob, kv, q, k_cur, v_cur, [C], o, lse, d_o, dq, dk, dv, ws=ws_b)
        R.rr_attn_prompt_grads(prob, kv, q, [C], o, lse, d_o, dkb, dvb, key_range=(P - C, P), ws=ws_pg)
        R.rr_lastkv_blend_bwd(alpha, kl_prev, kL_prev, dkb, g_src["kl"], g_src["kL"], d_alpha)
        R.rr_lastkv_blend_bwd(alpha, vl_prev, vL_prev, dvb, g_src["vl"], g_src["vL"], d_alpha, accumulate=1)

    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()
    rows = synth.sample_rows(w.seed, C, a.cpu_rows, w.block) if a.cpu_rows > 0 else None
    grp = w.Hq // w.Hkv
    got = None
    if rows is not None:
        got = {"o": o[0, rows, :grp].double().cpu().numpy(), "dq": dq[0, rows, :grp].double().cpu().numpy()}
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    R.rr_profile_begin()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    prof = R.rr_profile_end()
    ms_per_step = (t2 - t1) * 1e3 / a.steps

    kf = kernel_flops(w, C)
    per_kernel_flops = {"fwd_partials": kf["fwd_partials"], "dq_partials": kf["dq_partials"], "dkdv": kf["dkdv"],
                        "prompt_dkdv": 8.0 * w.d_qk * w.Hq * C * C}
    flops_step = configs.flops_dense(w.Hq, w.d_qk, w.d_v, C, P)["total"] + per_kernel_flops["prompt_dkdv"]
    tflops = flops_step / (ms_per_step * 1e-3) / 1e12
    dom_name, (dom_launches, dom_ms) = max(prof.items(), key=lambda kv_: kv_[1][1])
    roof = None
    if dom_name in per_kernel_flops:
        avg_ms = dom_ms / dom_launches
        flops_per_launch = per_kernel_flops[dom_name] / (dom_launches / a.steps)
        achieved = flops_per_launch / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dom_name, "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_from_profiles(dom_name, w.name, source_sha(KERNEL_SOURCES[dom_name])),
                "avg_launch_ms": round(avg_ms, 4), "flops_per_launch": flops_per_launch}
    kernels = {k: {"launches_per_step": v[0] / a.steps, "ms_per_step": round(v[1] / a.steps, 3)}
               for k, v in sorted(prof.items(), key=lambda kv_: -kv_[1][1])}
    for k, fl in per_kernel_flops.items():
        if k in kernels:
            kernels[k]["tflops"] = round(fl / (kernels[k]["ms_per_step"] * 1e-3) / 1e12, 2)

    cpu = parity = None
    if rows is not None:
        from oracle import dense, lastkv
        f = lambda v: synth.as_f64(v, w.dtype)
        tc = time.perf_counter()
        # history of KV head 0: last-layer K/V of the older chunks, then the blended chunk
        al = np.asarray(x["alpha"][:1], dtype=np.float64)
        hk = np.concatenate([f(x["k_last"][:P - C, :1]),
                             lastkv.blend(f(x["k_prev_layer"][:, :1]), f(x["k_last"][P - C:, :1]), al)], 0)
        hv = np.concatenate([f(x["v_last"][:P - C, :1]),
                             lastkv.blend(f(x["v_prev_layer"][:, :1]), f(x["v_last"][P - C:, :1]), al)], 0)
        qs, kr, vr, do = f(x["q"][:, :grp]), f(x["k_cur"][:, :1]), f(x["v_cur"][:, :1]), f(x["d_o"][:, :grp])
        ro, _ = dense.attend(qs, hk, hv, kr, vr, w.tau, rows=rows)
        rgr = dense.attend_bwd(qs, hk, hv, kr, vr, do, w.tau, rows=rows)
        cpu_s = time.perf_counter() - tc
        cpu_flops = sum(grp * 10.0 * w.d_qk * (P + int(r) + 1) for r in rows)
        cores = len(os.sched_getaffinity(0))
        cpu = {"value": round(cpu_flops / cpu_s / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
               "sample": f"{len(rows)} rows of the chunk {list(map(int, rows))}, KV head 0 and its {grp} query "
                         f"heads, blend + fwd + dQ over {P} history keys and the causal chunk keys; {cpu_s:.1f} s"}
        rel = lambda u, y: float(np.linalg.norm(u - y) / np.linalg.norm(y))
        parity = {"rows": len(rows), "o_rel_l2": rel(got["o"], ro), "dq_rel_l2": rel(got["dq"], rgr["dq"]),
                  "o_max_abs": float(np.abs(got["o"] - ro).max()),
                  "dq_max_abs": float(np.abs(got["dq"] - rgr["dq"]).max())}
        parity["pass"] = bool(parity["o_rel_l2"] <= 5e-3 and parity["dq_rel_l2"] <= 5e-3
                              and parity["o_max_abs"] <= 2e-2 and parity["dq_max_abs"] <= 2e-2)

    out = {
        "metric": "LastKV chunk attention fwd+bwd TFLOP/s + % bf16 MFMA peak (blend, history of 2M positions)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 2), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "history_P": P, "chunk_C": C, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d_qk,
                   "chunk": w.chunk, "flops_per_step": flops_step},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": roof, "cpu_baseline": cpu, "parity": parity, "kernels": kernels,
        "input_gen_s": round(gen_s, 1),
    }
    print(json.dumps(out), flush=True)
    return 0 if (parity is None or parity["pass"]) else 1


def run_latent(a, w) -> int:
    import torch

    from resident_kv_response_amd import configs, rr_attn as R, synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    Rr = w.R
    t0 = time.time()
    res = synth.resident(w)
    m0 = synth.member(w, 0)

    def up(x, dt="bf16"):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)

    lat_p, k_idx = up(res["latent_p"]), up(res["k_idx"], "f32")
    q, lat_r, d_o = up(m0["q"])[None], up(m0["latent_r"])[None], up(m0["d_o"])[None]
    q_idx = up(m0["q_idx"], "f32")[None]
    gen_s = time.time() - t0
    kv = R.resident(lat_p, None, version=1, k_idx=k_idx)
    prob = R.Problem(P=w.P, R_max=Rr, Hq=w.Hq, Hkv=1, d_qk=w.d_qk, d_v=w.d_v, chunk=w.chunk,
                     block=w.block, tau=w.tau, dtype=R.RR_BF16, K=1, topk=w.topk, idx_dim=w.idx_dim,
                     latent=1)
    ws_f = R.workspace(prob, R.RR_OP_FWD, dev)
    ws_b = R.workspace(prob, R.RR_OP_BWD, dev)
    f32 = dict(device=dev, dtype=torch.float32)
    o = torch.empty(1, Rr, w.Hq, w.d_v, **f32)
    lse = torch.empty(1, Rr, w.Hq, **f32)
    idx = torch.empty(1, Rr, w.topk, device=dev, dtype=torch.int32)
    dq = torch.empty(1, Rr, w.Hq, w.d_qk, **f32)
    dk = torch.empty(1, Rr, w.d_qk, **f32)
    dv = torch.empty(1, Rr, w.d_v, **f32)

    def step():
        R.rr_attn_fwd(prob, kv, q, lat_r, None, [Rr], o=o, lse=lse, q_idx=q_idx, topk_idx=idx, ws=ws_f)
        R.rr_attn_bwd(prob, kv, q, lat_r, None, [Rr], o, lse, d_o, dq, dk, dv, topk_idx=idx, ws=ws_b)

    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    step()
    torch.cuda.synchronize()
    rows = synth.sample_rows(w.seed, Rr, a.cpu_rows, w.block) if a.cpu_rows > 0 else None
    got = None
    if rows is not None:
        got = {"o": o[0, rows].double().cpu().numpy(), "dq": dq[0, rows].double().cpu().numpy(),
               "idx": idx[0, rows].cpu().numpy()}
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    R.rr_profile_begin()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    prof = R.rr_profile_end()
    peak_mem = torch.cuda.max_memory_allocated()
    ms_per_step = (t2 - t1) * 1e3 / a.steps

    flops_step = configs.flops_dense(w.Hq, w.d_qk, w.d_v, Rr, w.topk)["total"]
    index_flops = 2.0 * w.idx_dim * Rr * w.P
    tflops = flops_step / (ms_per_step * 1e-3) / 1e12
    model = latent_kernel_model(w, Rr)
    dom_name, (dom_launches, dom_ms) = max(prof.items(), key=lambda kv_: kv_[1][1])
    roof = None
    if dom_name in model:
        roof = roofline_entry(dom_name, model[dom_name], dom_launches / a.steps, dom_ms / dom_launches,
                              traffic_from_profiles(dom_name, w.name, source_sha(LATENT_SOURCES[dom_name])))
    kernels = {}
    for k, v in sorted(prof.items(), key=lambda kv_: -kv_[1][1]):
        e = {"launches_per_step": v[0] / a.steps, "ms_per_step": round(v[1] / a.steps, 3)}
        if k in model:
            t = v[1] / a.steps * 1e-3
            if model[k]["flops"]:
                e["tflops"] = round(model[k]["flops"] / t / 1e12, 2)
            e["gbs"] = round(model[k]["bytes"] / t / 1e9, 1)
        kernels[k] = e

    cpu = parity = None
    if rows is not None:
        from oracle import sparse
        f = lambda x: synth.as_f64(x, "bf16")
        tc = time.perf_counter()
        sig = sparse.index_scores(m0["q_idx"][rows], res["k_idx"])
        sel = np.zeros((Rr, w.topk), dtype=np.int64)
        sel[rows] = sparse.topk_select(sig, w.topk)
        lp, qq, lr, do = f(res["latent_p"]), f(m0["q"]), f(m0["latent_r"]), f(m0["d_o"])
        ro, _ = sparse.sparse_attend(qq, lp, lr, sel, w.tau, w.d_v, rows=rows)
        rgr = sparse.sparse_attend_bwd(qq, lp, lr, sel, do, w.tau, w.d_v, rows=rows)
        cpu_s = time.perf_counter() - tc
        # the same attention flops per row as the GPU value counts (the index scoring's
        # time is included, its flops are not, on both sides)
        H, dqk, dvv = w.Hq, w.d_qk, w.d_v
        cpu_flops = sum(H * ((2.0 * dqk + 2.0 * dvv) * (w.topk + int(r) + 1) + (4.0 * dqk + 2.0 * dvv) * w.topk
                             + (6.0 * dqk + 4.0 * dvv) * (int(r) + 1)) for r in rows)
        cores = len(os.sched_getaffinity(0))
        try:
            from threadpoolctl import threadpool_info
            blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            blas_threads = None
        cpu = {"value": round(cpu_flops / cpu_s / 1e12, 6), "unit": "TFLOP/s",
               "cores": blas_threads or cores, "kind": "oracle",
               "sample": f"{len(rows)} query rows {list(map(int, rows))} of the R={Rr} response: index "
                         f"scores over all {w.P} positions, top-{w.topk}, sparse attention fwd + bwd "
                         f"(64 heads); {cpu_s:.1f} s incl. widening the inputs to fp64",
               "host_cpus_affinity": cores, "host_cpu_count": os.cpu_count(),
               "extrapolated_full_step_s": round(flops_step / (cpu_flops / cpu_s), 1)}
        same = [n for n, r in enumerate(rows) if np.array_equal(got["idx"][n], sel[r])]
        rel = lambda x, y: float(np.linalg.norm(x - y) / np.linalg.norm(y))
        parity = {"rows": len(rows), "rows_with_identical_selection": len(same)}
        if same:
            s_ = np.array(same)
            parity.update({"o_rel_l2": rel(got["o"][s_], ro[s_]), "dq_rel_l2": rel(got["dq"][s_], rgr["dq"][s_]),
                           "o_max_abs": float(np.abs(got["o"][s_] - ro[s_]).max()),
                           "dq_max_abs": float(np.abs(got["dq"][s_] - rgr["dq"][s_]).max())})
        # the selections are decided by fp32 scores summed in different orders on the two
        # sides; a near tie at the k-th place may rank differently, which the GPU tests bound
        # position by position; here at most one sampled row in fifty may differ
        parity["pass"] = bool(len(same) >= int(np.ceil(0.98 * len(rows))) and parity.get("o_rel_l2", 1) <= 5e-3
                              and parity.get("dq_rel_l2", 1) <= 5e-3 and parity.get("o_max_abs", 1) <= 2e-2
                              and parity.get("dq_max_abs", 1) <= 2e-2)

    out = {
        "metric": "response-replay attention fwd+bwd TFLOP/s + % bf16 MFMA peak (latent top-k variant)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_per_step, 2), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "P": w.P, "R": Rr, "Hq": w.Hq, "latent": [w.d_v, w.d_qk - w.d_v],
                   "topk": w.topk, "idx_dim": w.idx_dim, "block": w.block,
                   "attention_flops_per_step": flops_step, "index_flops_fp32_per_step": index_flops},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "tokens_per_s": round(Rr / (ms_per_step * 1e-3), 1),
        "roofline": roof, "cpu_baseline": cpu, "parity": parity, "kernels": kernels,
        "peak_mem_bytes": int(peak_mem), "input_gen_s": round(gen_s, 1),
    }
    print(json.dumps(out), flush=True)
    return 0 if (parity is None or parity["pass"]) else 1


if __name__ == "__main__":
    sys.exit(main())
