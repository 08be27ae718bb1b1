"""Benchmark of the MoonEP hot path on one MI355X.

One step = one forward pass of the whole path over one batch of synthetic
routing for the 8-rank, S=4096, K=8, E=256 (B=32), H=7168, H'=2048,
token_padding=128 workload: plan -> dispatch -> prefetch_weight ->
grouped SwiGLU FFN (all 8 ranks) -> combine.  The timed steps cycle through
the imbalance sweep maxvio in {0, 0.5, 1, 2, 4, all-on-experts-0..7 (31)};
inputs are resident in HBM before timing starts.

Prints ONE JSON line.  `value` is plan+dispatch+combine GB/s (algorithmic
bytes over the summed stage times, HIP events on the launch stream); the
grouped-GEMM TFLOP/s, the per-maxvio breakdown, the roofline of the dominant
kernel (the grouped FFN GEMM) and of dispatch/combine, and the CPU oracle
timed on a bounded sample are reported alongside.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                    [--workload NAME] [--targets T,...] [--train]

--workload pages_r8_s8192_k8_e384 times the shape of the pages' own benchmark
(S=8192, E=384, maxvio 0.2/1/10/20); each sweep entry then also carries the
pages' stacked "dispatch" (plan + prefetch + dispatch).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

REPO = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, REPO)

import moonep_synth as synth  # noqa: E402

WORKLOAD = "fwd_r8_s4096_k8_e256"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s


def alg_bytes(w):
    """Algorithmic bytes per call (padding and its zero-fill not counted)."""
    R, S, K, E, B, H = w.R, w.S, w.K, w.E, w.B, w.H
    ntok = R * S
    plan = 8 * ntok * K + 4 * R * (E + B)              # topk in, dest out, cu_seqlens
    dispatch = ntok * (2 * H + 2 * H * K + 12 * K)     # row once in, K rows out, rw + dest
    combine = ntok * (2 * H * K + 2 * H + 12 * K)      # K rows in, row out, dest + rw in/out
    return plan, dispatch, combine


def ffn_bytes(w, plan):
    """Algorithmic HBM bytes of one ffn_gateup and one ffn_down launch for a
    plan: every used (rank, weight row) pair's weights once, every row of the
    ranks' segments (padding included) read once and its output written once."""
    EB = w.E + w.B
    seg = plan.arrays["seg_tokens"].cpu().numpy().reshape(w.R, EB)
    cu = plan.arrays["cu_seqlens"].cpu().numpy().reshape(w.R, EB)
    pairs = int((seg > 0).sum())
    rows = int(cu[:, -1].sum())
    wrow = w.H * w.Hp * 2
    return {"gateup_bytes": pairs * 2 * wrow + rows * (w.H + w.Hp) * 2,
            "down_bytes": pairs * wrow + rows * (w.Hp + w.H) * 2}


def ffn_roofline(name, flops, nbytes, t):
    """The binding roofline of a GEMM launch: HBM when its arithmetic intensity
    is below the machine balance (bf16 peak over HBM peak), MFMA otherwise."""
    hbm = flops / nbytes < BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if hbm:
        ach = nbytes / t / 1e9
        r = {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
             "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = flops / t / 1e12
        r = {"kernel": name, "bound": "mfma", "achieved": round(ach, 1),
             "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4)}
    r["per_launch"] = {"flops": flops, "bytes": nbytes, "avg_s": t}
    return r


def ffn_flops(w):
    """Algorithmic flops of the grouped FFN over every real slot (padding rows
    not counted): gate and up 2*H*H' each, down 2*H*H' per slot."""
    return 6.0 * w.H * w.Hp * w.R * w.S * w.K


def gateup_flops(w):
    return 4.0 * w.H * w.Hp * w.R * w.S * w.K


def down_flops(w):
    return 2.0 * w.H * w.Hp * w.R * w.S * w.K


TRAFFIC_FILE = os.path.join(REPO, "profiles", "traffic_ffn_gateup_fwd_r8_s4096_k8_e256.txt")
_CSRC = os.path.join(REPO, "grouped_gemm_moonep_amd", "csrc")
# kernel -> (hash key, sources the counters are valid for, bytes key) in TRAFFIC_FILE
TRAFFIC_KEYS = {
    "ffn_gateup": ("source_sha256", ("gemm_core.h", "gemm.hip"), "hbm_bytes_per_launch"),
    "ffn_down": ("source_sha256", ("gemm_core.h", "gemm.hip"), "down_hbm_bytes_per_launch"),
    "dispatch": ("move_source_sha256", ("move.hip",), "dispatch_hbm_bytes_per_launch"),
    "combine": ("move_source_sha256", ("move.hip",), "combine_hbm_bytes_per_launch"),
}


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` (a TRAFFIC_KEYS name) from the
    committed counter summary of the headline workload, or None when the
    kernel's sources have changed since the counters were taken."""
    import hashlib
    hkey, sources, bkey = TRAFFIC_KEYS[kernel]
    try:
        fields = dict(line.split(":", 1) for line in open(TRAFFIC_FILE)
                      if ":" in line and not line.startswith(" "))
        h = hashlib.sha256()
        for f in sources:
            h.update(open(os.path.join(_CSRC, f), "rb").read())
        src = h.hexdigest()
    except OSError:
        return None
    if fields.get(hkey, "").strip() != src or bkey not in fields:
        return None
    return int(fields[bkey].strip())


def _blas_threads():
    """Threads of the BLAS numpy calls into (threadpoolctl's report)."""
    try:
        import threadpoolctl
        n = [i["num_threads"] for i in threadpoolctl.threadpool_info() if i["user_api"] == "blas"]
        return int(n[0]) if n else None
    except Exception:
        return None


def cpu_ffn_leg(w, p, x_dev, home_dev, budget_s=15.0, max_segments=16):
    """The oracle's per-token SwiGLU (oracle.ffn_token, float64 BLAS on every
    core the process may use) over a bounded sample of the FFN: the segments
    of rank 0 in row order, each with its real tokens and its expert's home
    weights copied from the GPU, until `max_segments` or `budget_s` seconds of
    oracle time.  Returns the oracle's TFLOP/s over the sample (6 H H' flop
    per token, as the GPU figure counts) and the whole job's time at that
    rate."""
    import oracle
    import torch
    cores = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl
        limit = threadpoolctl.threadpool_limits(limits=cores, user_api="blas")
    except Exception:
        limit = None
    rows = [row for row in range(w.E + w.B) if p.seg_tokens[0, row] > 0]
    t_ffn, flops, toks, nseg = 0.0, 0.0, 0, 0
    xf = x_dev.reshape(-1, w.H)
    for row in rows[:max_segments]:
        e = row if row < w.E else int(p.prefetch_src[0, row - w.E])
        n = int(p.seg_tokens[0, row])
        start = int(p.cu_seqlens[0, row] - p.seg_len[0, row])
        tok = p.src[0, start:start + n] // w.K
        xs = xf[torch.from_numpy(tok.astype(np.int64)).to(x_dev.device)].cpu().view(
            torch.int16).numpy().view(np.uint16)
        wts = [home_dev[i][e].cpu().view(torch.int16).numpy().view(np.uint16) for i in range(3)]
        t0 = time.perf_counter()
        oracle.ffn_token(xs, *wts)
        t_ffn += time.perf_counter() - t0
        flops += 6.0 * w.H * w.Hp * n
        toks += n
        nseg += 1
        if t_ffn > budget_s:
            break
    threads = _blas_threads()
    if limit is not None:
        limit.restore_original_limits()
    rate = flops / t_ffn
    return {"value": round(rate / 1e12, 5), "unit": "TFLOP/s", "cores": threads or cores,
            "kind": "oracle",
            "sample": f"oracle.ffn_token (float64 BLAS) over the first {nseg} segments of rank 0 "
                      f"({toks} real tokens) at the baseline's routing, weights and tokens "
                      f"copied from the GPU; the whole job ({w.R} ranks x S*K slots) would take "
                      f"{ffn_flops(w) / rate:.1f} s at this rate",
            "seconds": round(t_ffn, 3), "flops": flops}


def cpu_baseline(w, host_routing, main_target, x_dev, home_dev, chunk=1024):
    """The oracle on the host, on a bounded sample of the workload.

    Plan + dispatch + combine (the GB/s half of the metric, numpy fancy
    indexing on one thread): the full plan of every routing in the sweep,
    then dispatch and combine of the whole hidden state for the `main_target`
    routing, in `chunk`-column slices (so the oracle's working set stays near
    1 GB).  Grouped FFN (the TFLOP/s half): cpu_ffn_leg on the same routing.
    The host's core count and the process's usable cores are stated."""
    import oracle
    import torch
    x = x_dev.cpu().view(torch.int16).numpy().view(np.uint16)
    t_plan = 0.0
    plans = {}
    for t, (topk, rw) in host_routing.items():
        t0 = time.perf_counter()
        plans[t] = oracle.plan(topk, w.E, w.B, w.token_padding)
        t_plan += time.perf_counter() - t0
    p, rw = plans[main_target], host_routing[main_target][1]
    t_disp = t_comb = 0.0
    for c0 in range(0, w.H, chunk):
        xs = np.ascontiguousarray(x[..., c0:c0 + chunk])
        t0 = time.perf_counter()
        x_nvs, rw_nvs = oracle.dispatch(p, xs, rw)
        t1 = time.perf_counter()
        oracle.combine(p, x_nvs, rw_nvs)
        t_disp += t1 - t0
        t_comb += time.perf_counter() - t1
        del x_nvs, rw_nvs
    pb, db, cb = alg_bytes(w)
    total = t_plan + t_disp + t_comb
    gbs = (len(plans) * pb + db + cb) / total / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"plan of all {len(plans)} {w.name} routings of the sweep + dispatch and "
                      f"combine of the full hidden state at maxvio {main_target} ({chunk}-column "
                      f"slices); numpy fancy indexing and fp32 sums, single-threaded",
            "seconds": {"plan": round(t_plan, 3), "dispatch": round(t_disp, 3),
                        "combine": round(t_comb, 3), "total": round(total, 3)},
            "host_cores": os.cpu_count(), "usable_cores": len(os.sched_getaffinity(0)),
            "ffn": cpu_ffn_leg(w, p, x_dev, home_dev)}


def time_backward(w, buf, plan, batches, x_nvs, z_ws, home, pool, steps, warmup, flush):
    """Backward of the step, timed per stage with HIP events on the launch
    stream.  For each batch the forward inputs of the backward (plan, x_nvs,
    prefetched weights, Z) are recomputed untimed, then the cache is flushed;
    then: combine bwd (dispatch of dOut), FFN backward (dZ, dG/dU, dX),
    dispatch bwd (unweighted combine of dX), dW for gate, up and down, and
    reduce_grad.  Stage times are medians per maxvio target; the weight
    gradients are also set against both of their bounds (MFMA and HBM)."""
    import torch
    dev = x_nvs.device
    g = torch.Generator(device=dev).manual_seed(1)
    x = torch.randn((w.R, w.S, w.H), generator=g, device=dev).to(torch.bfloat16)
    dout = torch.randn((w.R, w.S, w.H), generator=g, device=dev).to(torch.bfloat16)
    dy_nvs = torch.empty_like(x_nvs)
    dx_nvs = torch.empty_like(x_nvs)
    dz, dg, du = (torch.empty_like(z_ws) for _ in range(3))
    dx = torch.empty_like(x)
    grads = [torch.zeros((w.E, w.H, w.Hp), dtype=torch.float32, device=dev) for _ in range(3)]
    rbuf = [torch.zeros((w.R, w.B, w.H, w.Hp), dtype=torch.float32, device=dev) for _ in range(3)]
    names = ["combine_bwd", "ffn_bwd", "dispatch_bwd", "wgrad_x3", "reduce_grad"]
    per = {n: [] for n in names}
    wgrad_bytes = []
    reduce_bytes = []
    used = []
    EB = w.E + w.B
    for i in range(warmup + steps):
        t, topk, _ = batches[i % len(batches)]
        buf.plan(topk, plan=plan)
        buf.dispatch(plan, x, x_nvs=x_nvs)
        buf.prefetch_weight(plan, home, pool)
        buf.expert_gateup(plan, x_nvs, home, pool, z_ws)
        flush()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        ev[0].record()
        buf.dispatch(plan, dout, x_nvs=dy_nvs)
        ev[1].record()
        buf.expert_ffn_bwd(plan, x_nvs, dy_nvs, home, pool, dz, dg, du, dx_nvs)
        ev[2].record()
        buf.combine(plan, dx_nvs, out=dx)
        ev[3].record()
        buf.expert_wgrad(plan, x_nvs, dg, grads[0], rbuf[0])
        buf.expert_wgrad(plan, x_nvs, du, grads[1], rbuf[1])
        buf.expert_wgrad(plan, dy_nvs, z_ws, grads[2], rbuf[2])
        ev[4].record()
        buf.reduce_grad(plan, grads, rbuf)
        ev[5].record()
        torch.cuda.synchronize()
        if i >= warmup:
            used.append(t)
            for j, n in enumerate(names):
                per[n].append(ev[j].elapsed_time(ev[j + 1]) * 1e-3)
            # each used (rank, weight row) pair's fp32 gradient rows are read and
            # written once per projection; each segment row of the two operands
            # of each product is read once
            seg = plan.arrays["seg_tokens"].cpu().numpy().reshape(w.R, EB)
            rows = int(plan.arrays["cu_seqlens"].cpu().numpy().reshape(w.R, EB)[:, -1].sum())
            wgrad_bytes.append(3 * int((seg > 0).sum()) * float(w.H) * w.Hp * 4 * 2
                               + 3 * rows * (w.H + w.Hp) * 2)
            # reduce_grad, per projection: each home row with copies read and written
            # once, each holder slot read once and zeroed (fp32 rows of H H')
            ps = plan.arrays["prefetch_src"].cpu().numpy()
            holders = int((ps >= 0).sum())
            homes = len(set(int(e) for e in ps[ps >= 0]))
            reduce_bytes.append(3 * float(w.H) * w.Hp * 4 * (2 * homes + 2 * holders))
    slots = w.R * w.S * w.K
    hh = float(w.H) * w.Hp
    mean = {n: float(np.mean(v)) for n, v in per.items()}
    out = {n + "_ms": round(t * 1e3, 3) for n, t in mean.items()}
    out["ffn_bwd_TFLOPs"] = round(10 * hh * slots / mean["ffn_bwd"] / 1e12, 1)
    out["wgrad_TFLOPs"] = round(6 * hh * slots / mean["wgrad_x3"] / 1e12, 1)
    out["wgrad_GBps"] = round(sum(wgrad_bytes) / sum(per["wgrad_x3"]) / 1e9, 1)
    # the three weight-gradient launches against both bounds: the MFMA time of
    # their flops and the HBM time of their algorithmic bytes at the published
    # peaks; the binding one is the larger
    wb = float(np.mean(wgrad_bytes))
    t_mfma = 6 * hh * slots / (BF16_PEAK_TFLOPS * 1e12)
    t_hbm = wb / (HBM_PEAK_GBS * 1e9)
    out["roofline_wgrad"] = {
        "kernel": "wgrad_kernel x3 (dWg, dWu, dWd; all ranks)",
        "bound": "hbm" if t_hbm > t_mfma else "mfma",
        "mfma_floor_ms": round(t_mfma * 1e3, 3), "hbm_floor_ms": round(t_hbm * 1e3, 3),
        "measured_ms": round(mean["wgrad_x3"] * 1e3, 3),
        "frac": round(max(t_mfma, t_hbm) / mean["wgrad_x3"], 4),
        "frac_of_bf16_peak": round(t_mfma / mean["wgrad_x3"], 4),
        "algorithmic_bytes": wb, "flops": 6 * hh * slots}
    # reduce_grad over the steps that have prefetch copies (balanced routing has none)
    rt = [t for t, b in zip(per["reduce_grad"], reduce_bytes) if b > 0]
    if rt:
        rgbs = sum(b for b in reduce_bytes if b > 0) / sum(rt) / 1e9
        out["reduce_grad_GBps"] = round(rgbs, 1)
        out["roofline_reduce_grad"] = {
            "kernel": "reduce_grad_kernel (three projections, all ranks)", "bound": "hbm",
            "achieved": round(rgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(rgbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_mean": float(np.mean([b for b in reduce_bytes if b > 0]))}
    pb, db, cb = alg_bytes(w)
    out["combine_bwd_GBps"] = round(db / mean["combine_bwd"] / 1e9, 1)
    out["dispatch_bwd_GBps"] = round((slots * 2 * w.H + w.R * w.S * 2 * w.H + 4 * slots)
                                     / mean["dispatch_bwd"] / 1e9, 1)
    out["backward_ms"] = round(sum(mean.values()) * 1e3, 3)
    out["per_target_median_ms"] = {
        str(t): {n: round(float(np.median([per[n][i] for i, u in enumerate(used) if u == t]))
                          * 1e3, 3) for n in names}
        for t in dict.fromkeys(used)}
    out["note"] = ("flops per real slot: FFN backward 10 H H' (dZ 2, recomputed gate/up 4, "
                   "dX 4), weight gradients 6 H H'; weight-gradient bytes: fp32 read-modify-"
                   "write of each used (rank, weight row) pair's gradient per projection plus "
                   "the bf16 operand rows once; steps cycle the same maxvio targets")
    return out


def time_overlap(w, batches, home, pool, steps, warmup, num_cus=32):
    """Two micro-batches per step: communication calls (plan, dispatch,
    prefetch, combine) on a second stream through a handle whose kernels are
    capped at `num_cus` CUs (the README's num_sms budget), the FFN on the
    compute stream; combine of A overlaps the FFN of B and dispatch of B the
    FFN of A.  Reported beside the same two micro-batches run back to back."""
    import torch
    from grouped_gemm_moonep_amd import Buffer
    dev = home[0].device
    kw = dict(R=w.R, S=w.S, K=w.K, E=w.E, B=w.B, H=w.H, Hp=w.Hp, token_padding=w.token_padding)
    comp = Buffer(**kw)
    comm = Buffer(**kw, num_cus=num_cus)
    g = torch.Generator(device=dev).manual_seed(2)
    xs = [torch.randn((w.R, w.S, w.H), generator=g, device=dev).to(torch.bfloat16) for _ in range(2)]
    plans = [comp.new_plan() for _ in range(2)]
    x_nvs = [torch.empty((w.R, comp.NvS, w.H), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    rw_nvs = [torch.empty((w.R, comp.NvS), dtype=torch.float32, device=dev) for _ in range(2)]
    z = torch.empty((w.R, comp.NvS, w.Hp), dtype=torch.bfloat16, device=dev)
    outs = [torch.empty_like(xs[0]) for _ in range(2)]
    pools = [pool, [torch.empty_like(t) for t in pool]]
    s_comp = torch.cuda.current_stream()
    s_comm = torch.cuda.Stream(device=dev)

    def front(b, i, h):
        _, topk, rw = batches[(2 * i + b) % len(batches)]
        h.plan(topk, plan=plans[b])
        h.dispatch(plans[b], xs[b], rw, x_nvs=x_nvs[b], rw_nvs=rw_nvs[b])
        h.prefetch_weight(plans[b], home, pools[b])

    def ffn(b):
        comp.expert_gateup(plans[b], x_nvs[b], home, pools[b], z)
        comp.expert_down(plans[b], z, home, pools[b], x_nvs[b])

    def back(b, h):
        h.combine(plans[b], x_nvs[b], rw_nvs[b], out=outs[b], gather_rw=False)

    def serial(i):
        for b in range(2):
            front(b, i, comp)
            ffn(b)
            back(b, comp)

    def overlapped(i):
        ev = {k: torch.cuda.Event() for k in ("fa", "fb", "ffa", "ffb", "start")}
        ev["start"].record(s_comp)
        with torch.cuda.stream(s_comm):
            s_comm.wait_event(ev["start"])
            front(0, i, comm)
            ev["fa"].record(s_comm)
            front(1, i, comm)                 # overlaps the FFN of A
            ev["fb"].record(s_comm)
        s_comp.wait_event(ev["fa"])
        ffn(0)
        ev["ffa"].record(s_comp)
        with torch.cuda.stream(s_comm):
            s_comm.wait_event(ev["ffa"])
            back(0, comm)                     # overlaps the FFN of B
        s_comp.wait_event(ev["fb"])
        ffn(1)
        ev["ffb"].record(s_comp)
        with torch.cuda.stream(s_comm):
            s_comm.wait_event(ev["ffb"])
            back(1, comm)
        s_comp.wait_stream(s_comm)

    res = {}
    for name, fn in (("serial", serial), ("overlapped", overlapped)):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        res[name] = (time.perf_counter() - t0) / steps
    comp.destroy()
    comm.destroy()
    return {"num_cus": num_cus, "micro_batches": 2,
            "serial_ms": round(res["serial"] * 1e3, 3),
            "overlapped_ms": round(res["overlapped"] * 1e3, 3),
            "speedup": round(res["serial"] / res["overlapped"], 3),
            "note": "ms per two micro-batches (plan, dispatch, prefetch, FFN, combine each); "
                    "wall clock over the timed steps"}


def time_views(w, buf, batches, home, pool, x, steps):
    """The FFN and prefetch over per-rank [E+B,H,H'] views on virtual memory
    (SymmetricBuffer: every rank's view maps the same home chunks) beside the
    same calls over ordinary home / pool tensors, on the same plans and
    inputs, alternating step by step."""
    import torch
    from grouped_gemm_moonep_amd import SymmetricBuffer
    sbs = [SymmetricBuffer(buf) for _ in range(3)]
    for i, sb in enumerate(sbs):
        sb.home.copy_(home[i])
    views = [sb.views for sb in sbs]
    dev = x.device
    plan = buf.new_plan()
    x_nvs = torch.empty((w.R, buf.NvS, w.H), dtype=torch.bfloat16, device=dev)
    y = torch.empty_like(x_nvs)
    z = torch.empty((w.R, buf.NvS, w.Hp), dtype=torch.bfloat16, device=dev)
    t = {"prefetch_views": [], "ffn_views": [], "prefetch_split": [], "ffn_split": []}
    for i in range(steps + 1):
        _, topk, rw = batches[i % len(batches)]
        buf.plan(topk, plan=plan)
        buf.dispatch(plan, x, rw, x_nvs=x_nvs)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        ev[0].record()
        buf.prefetch_weight_views(plan, views)
        ev[1].record()
        buf.expert_ffn_views(plan, x_nvs, views, z_ws=z, y_nvs=y)
        ev[2].record()
        ev[3].record()
        buf.prefetch_weight(plan, home, pool)
        ev[4].record()
        buf.expert_ffn(plan, x_nvs, home, pool, z_ws=z, y_nvs=y)
        ev[5].record()
        torch.cuda.synchronize()
        if i == 0:
            continue                          # first pass warms both paths
        t["prefetch_views"].append(ev[0].elapsed_time(ev[1]))
        t["ffn_views"].append(ev[1].elapsed_time(ev[2]))
        t["prefetch_split"].append(ev[3].elapsed_time(ev[4]))
        t["ffn_split"].append(ev[4].elapsed_time(ev[5]))
    m = {k: float(np.mean(v)) for k, v in t.items()}
    phys = sbs[0].physical_bytes
    gran = sbs[0].granularity
    del views
    for sb in sbs:
        sb.destroy()
    return {"ffn_ms_views": round(m["ffn_views"], 3), "ffn_ms_split": round(m["ffn_split"], 3),
            "ffn_views_over_split": round(m["ffn_views"] / m["ffn_split"], 4),
            "prefetch_us_views": round(m["prefetch_views"] * 1e3, 1),
            "prefetch_us_split": round(m["prefetch_split"] * 1e3, 1),
            "physical_bytes_per_projection": phys, "vmm_granularity": gran,
            "steps": steps,
            "note": "per-rank [E+B] views on hipMemMap'd chunks vs separate home/pool tensors"}


def time_graph(w, buf, batches, home, pool, x, steps):
    """The forward step (plan, dispatch, prefetch, FFN, combine) captured once
    as a HIP graph and replayed with each batch's routing copied into the
    captured input, beside the same step launched eagerly: the path has no
    host synchronisation and static shapes, so one graph serves every
    routing."""
    import torch
    dev = x.device
    plan = buf.new_plan()
    topk_in = torch.empty_like(batches[0][1])
    rw_in = torch.empty_like(batches[0][2])
    x_nvs = torch.empty((w.R, buf.NvS, w.H), dtype=torch.bfloat16, device=dev)
    rw_nvs = torch.empty((w.R, buf.NvS), dtype=torch.float32, device=dev)
    z = torch.empty((w.R, buf.NvS, w.Hp), dtype=torch.bfloat16, device=dev)
    out = torch.empty((w.R, w.S, w.H), dtype=torch.bfloat16, device=dev)
    rw_sk = torch.empty((w.R, w.S, w.K), dtype=torch.float32, device=dev)

    def step():
        buf.plan(topk_in, plan=plan)
        buf.dispatch(plan, x, rw_in, x_nvs=x_nvs, rw_nvs=rw_nvs)
        buf.prefetch_weight(plan, home, pool)
        buf.expert_ffn(plan, x_nvs, home, pool, z_ws=z, y_nvs=x_nvs)
        buf.combine(plan, x_nvs, rw_nvs, out=out, rw_sk=rw_sk)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    res = {}
    for mode in ("eager", "graph", "eager", "graph"):
        t_total = 0.0
        for i in range(steps):
            _, topk, rw = batches[i % len(batches)]
            topk_in.copy_(topk)
            rw_in.copy_(rw)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            if mode == "graph":
                g.replay()
            else:
                step()
            torch.cuda.synchronize()
            t_total += time.perf_counter() - t0
        res[mode] = t_total / steps           # the second pass of each mode is kept
    del g
    return {"eager_ms": round(res["eager"] * 1e3, 3), "graph_ms": round(res["graph"] * 1e3, 3),
            "graph_over_eager": round(res["graph"] / res["eager"], 4), "steps": steps,
            "note": "host wall clock per step (launch to completion), inputs copied in "
                    "before each timed step"}


def time_per_rank(w, buf, batches, home, pool, x, reps=3):
    """The grouped FFN of each virtual rank on its own (moonep_expert_ffn with
    rank = d) at the first and the last routing of the sweep: the slowest and
    the mean rank, per rank 6 S K H H' flop.  The balanced plan gives every
    rank exactly S K slots, so the ranks stay level however skewed the
    routing."""
    import torch
    dev = x.device
    plan = buf.new_plan()
    x_nvs = torch.empty((w.R, buf.NvS, w.H), dtype=torch.bfloat16, device=dev)
    y = torch.empty_like(x_nvs)
    z = torch.empty((w.R, buf.NvS, w.Hp), dtype=torch.bfloat16, device=dev)
    flops = 6.0 * w.S * w.K * w.H * w.Hp
    out = {}
    for t, topk, rw in (batches[0], batches[-1]):
        buf.plan(topk, plan=plan)
        buf.dispatch(plan, x, rw, x_nvs=x_nvs)
        buf.prefetch_weight(plan, home, pool)
        for d in range(w.R):                                               # warm every rank
            buf.expert_ffn(plan, x_nvs, home, pool, z_ws=z, y_nvs=y, rank=d)
        ms = []
        for d in range(w.R):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            for _ in range(reps):
                buf.expert_ffn(plan, x_nvs, home, pool, z_ws=z, y_nvs=y, rank=d)
            ev[1].record()
            torch.cuda.synchronize()
            ms.append(ev[0].elapsed_time(ev[1]) / reps)
        out[str(t)] = {"rank_ms": [round(v, 3) for v in ms], "slowest_ms": round(max(ms), 3),
                       "mean_ms": round(float(np.mean(ms)), 3),
                       "slowest_TFLOPs": round(flops / (max(ms) * 1e-3) / 1e12, 1),
                       "mean_TFLOPs": round(flops / (float(np.mean(ms)) * 1e-3) / 1e12, 1),
                       "slowest_over_mean": round(max(ms) / float(np.mean(ms)), 3)}
    out["note"] = ("each rank's FFN launched on its own (one rank's tiles fill the GPU less "
                   "than the all-rank launch timed above); slowest_over_mean is the balance")
    return out


def _smi_sample():
    """One amd-smi reading of the GPU: socket power (W) and the shader clock of
    each XCD (MHz), or None when amd-smi is not available."""
    import re
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "-g", "0"], capture_output=True,
                           text=True, timeout=30)
    except (OSError, subprocess.TimeoutExpired):
        return None
    p = re.findall(r"SOCKET_POWER: (\d+) W", r.stdout)
    c = re.findall(r"GFX_\d+:\s+CLK: (\d+) MHz", r.stdout)
    if not p or not c:
        return None
    return int(p[0]), [int(x) for x in c]


def power_probe(w, secs):
    """Board power and shader clocks while one kind of kernel runs back to
    back for `secs` seconds (after a warm-up), sampled with amd-smi from a
    second thread: the idle GPU, a plain 4 GiB copy (HBM traffic alone), and
    the headline's gate/up GEMM, down GEMM and one weight-gradient GEMM at
    balanced routing."""
    import threading
    import torch
    from grouped_gemm_moonep_amd import Buffer
    dev = "cuda"
    topk, _ = synth.routing(w, 0.0)
    home = [torch.empty((w.E, w.H, w.Hp), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    for i in range(3):
        synth.expert_weights_device(w, i, home[i])
    pool = [torch.zeros((w.R, w.B, w.H, w.Hp), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    buf = Buffer(R=w.R, S=w.S, K=w.K, E=w.E, B=w.B, H=w.H, Hp=w.Hp, token_padding=w.token_padding)
    plan = buf.plan(torch.from_numpy(topk).to(dev))
    g = torch.Generator(device=dev).manual_seed(0)
    x = torch.randn((w.R, w.S, w.H), generator=g, device=dev).to(torch.bfloat16)
    x_nvs, _ = buf.dispatch(plan, x)
    z = torch.empty((w.R, buf.NvS, w.Hp), dtype=torch.bfloat16, device=dev)
    y = torch.empty((w.R, buf.NvS, w.H), dtype=torch.bfloat16, device=dev)
    a = torch.ones(1 << 30, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    legs = {
        "idle": None,
        "copy_4GiB": lambda: b.copy_(a),
        "ffn_gateup": lambda: buf.expert_gateup(plan, x_nvs, home, pool, z),
        "ffn_down": lambda: buf.expert_down(plan, z, home, pool, y),
    }
    out = {}
    for name, f in list(legs.items()) + [("wgrad_kernel", "wgrad")]:
        if f == "wgrad":
            del legs, a, b
            home = pool = None
            torch.cuda.empty_cache()
            gh = torch.zeros((w.E, w.H, w.Hp), dtype=torch.float32, device=dev)
            rb = torch.zeros((w.R, w.B, w.H, w.Hp), dtype=torch.float32, device=dev)
            f = lambda: buf.expert_wgrad(plan, x_nvs, z, gh, rb)
        print(f"[bench] power: {name}", file=sys.stderr, flush=True)
        samples, stop = [], threading.Event()

        def sampler():
            time.sleep(2.0)                       # past the warm-up
            while not stop.is_set():
                s = _smi_sample()
                if s is None:
                    return
                samples.append(s)
                time.sleep(0.25)

        th = threading.Thread(target=sampler)
        n, t_ms = 0, 0.0
        if f is not None:
            f()
        torch.cuda.synchronize()
        th.start()
        t0 = time.time()
        while time.time() - t0 < secs:
            if f is None:
                time.sleep(0.1)
                continue
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                f()
            e1.record()
            torch.cuda.synchronize()
            n += 10
            t_ms += e0.elapsed_time(e1)
        stop.set()
        th.join()
        if not samples:
            out[name] = "amd-smi unavailable"
            continue
        pw = [p for p, _ in samples]
        clk = [c for _, cs in samples for c in cs]
        out[name] = {"samples": len(samples), "socket_power_W": [min(pw), max(pw)],
                     "shader_clock_MHz_mean": round(float(np.mean(clk)), 1),
                     "shader_clock_MHz_range": [min(clk), max(clk)],
                     "launches": n, "ms_per_launch": round(t_ms / n, 3) if n else None}
    buf.destroy()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=12)
    ap.add_argument("--warmup", type=int, default=6)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=WORKLOAD, choices=sorted(synth.WORKLOADS),
                    help="workload to time (default: the 8-rank S=4096 E=256 forward); "
                         "pages_r8_s8192_k8_e384 is the shape of the pages' own benchmark")
    ap.add_argument("--targets", default=None,
                    help="comma-separated maxvio targets (default: the workload's sweep)")
    ap.add_argument("--train", action="store_true",
                    help="also time a training step's backward (combine bwd, FFN backward, "
                         "dispatch bwd, three weight gradients, reduce_grad) and report it "
                         "under 'train'; needs ~90 GB more HBM for the fp32 gradient buffers")
    ap.add_argument("--overlap", action="store_true",
                    help="also time two pipelined micro-batches with dispatch/combine on a "
                         "second stream at a 32-CU budget against running them back to back")
    ap.add_argument("--no-per-rank", action="store_true",
                    help="skip the per-virtual-rank FFN leg (profiling runs: keeps the kernel "
                         "statistics to the timed steps' launches)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the forward step as one HIP graph replayed for every "
                         "routing beside the same step launched eagerly")
    ap.add_argument("--views", action="store_true",
                    help="also time prefetch and the FFN over per-rank [E+B] views on virtual "
                         "memory (SymmetricBuffer) beside ordinary home/pool tensors; needs "
                         "~45 GB more HBM at the headline shape")
    ap.add_argument("--flush-mb", type=int, default=1024, metavar="MIB",
                    help="before every timed step, write a scratch buffer of MIB MiB so "
                         "that the 256 MB last-level cache (MALL) holds nothing of the "
                         "step's inputs (0: no flush)")
    ap.add_argument("--sweep-reps", type=int, default=20,
                    help="per maxvio target: timed repetitions (after 3 warm-up ones) of "
                         "the step, each after a cache flush; the per-target table reports "
                         "their medians")
    ap.add_argument("--power", type=float, default=0.0, metavar="SECONDS",
                    help="only measure board power and shader clocks (amd-smi) while the idle "
                         "GPU, a 4 GiB copy, gate/up, down and one weight gradient each run "
                         "for SECONDS at the headline shape, and print them as one JSON line")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="before warmup, run torch.neg over a float32 buffer of MIB MiB "
                         "three times: a plain kernel of known traffic (reads and writes "
                         "MIB MiB) that calibrates FETCH_SIZE / WRITE_SIZE counter runs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the R EP ranks are emulated as R regions "
              f"of one GPU's HBM); --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    from grouped_gemm_moonep_amd import Buffer

    w = synth.WORKLOADS[args.workload]
    if args.power > 0:
        print(json.dumps({"power": power_probe(w, args.power), "workload": w.name,
                          "note": "amd-smi metric -p -c every ~0.3 s from a second thread while "
                                  "each leg's kernel runs back to back"}), flush=True)
        return
    dev = "cuda"
    if args.targets is None:
        targets = list(synth.SWEEPS[args.workload])
    else:
        targets = [t if t == "adv" else float(t) for t in args.targets.split(",")]
    print(f"[bench] {w.name}: generating routing for {targets}", file=sys.stderr, flush=True)
    batches = []
    host_routing = {}
    for t in targets:
        topk, rw = synth.routing(w, t)
        host_routing[t] = (topk, rw)
        batches.append((t, torch.from_numpy(topk).to(dev), torch.from_numpy(rw).to(dev)))

    print("[bench] drawing weights and hidden states on the GPU", file=sys.stderr, flush=True)
    home = [torch.empty((w.E, w.H, w.Hp), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    for i in range(3):
        synth.expert_weights_device(w, i, home[i])
    pool = [torch.zeros((w.R, w.B, w.H, w.Hp), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    g = torch.Generator(device=dev).manual_seed(0)
    x = torch.randn((w.R, w.S, w.H), generator=g, device=dev).to(torch.bfloat16)

    buf = Buffer(R=w.R, S=w.S, K=w.K, E=w.E, B=w.B, H=w.H, Hp=w.Hp,
                 token_padding=w.token_padding)
    plan = buf.new_plan()
    x_nvs = torch.empty((w.R, buf.NvS, w.H), dtype=torch.bfloat16, device=dev)
    rw_nvs = torch.empty((w.R, buf.NvS), dtype=torch.float32, device=dev)
    z_ws = torch.empty((w.R, buf.NvS, w.Hp), dtype=torch.bfloat16, device=dev)
    out = torch.empty((w.R, w.S, w.H), dtype=torch.bfloat16, device=dev)
    rw_sk = torch.empty((w.R, w.S, w.K), dtype=torch.float32, device=dev)

    def step(i, ev=None):
        t, topk, rw = batches[i % len(batches)]
        rec = (lambda j: ev[j].record()) if ev is not None else (lambda j: None)
        rec(0)
        buf.plan(topk, plan=plan)
        rec(1)
        buf.dispatch(plan, x, rw, x_nvs=x_nvs, rw_nvs=rw_nvs)
        rec(2)
        buf.prefetch_weight(plan, home, pool)
        rec(3)
        buf.expert_gateup(plan, x_nvs, home, pool, z_ws)
        rec(4)
        buf.expert_down(plan, z_ws, home, pool, x_nvs)      # in place (zero copy)
        rec(5)
        buf.combine(plan, x_nvs, rw_nvs, out=out, rw_sk=rw_sk)
        rec(6)
        return t

    if args.copy_probe > 0:
        n = args.copy_probe * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b
        print(f"[bench] copy probe: 3 x neg over {args.copy_probe} MiB", file=sys.stderr, flush=True)

    scratch_flush = (torch.empty(args.flush_mb << 20, dtype=torch.uint8, device=dev)
                     if args.flush_mb > 0 else None)

    def flush():
        if scratch_flush is not None:
            scratch_flush.fill_(1)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        flush()
        step(i)
    torch.cuda.synchronize()

    # per-maxvio stats (duplicates, realized imbalance) from the GPU plan
    stats = {}
    for t, topk, _ in batches:
        buf.plan(topk, plan=plan)
        st = buf.read_stats(plan)
        stats[t] = {"dups": int(st[1]), "maxvio": float(np.int32(st[5]).view(np.float32)),
                    "pad_rows": int(st[4])}
        stats[t].update(ffn_bytes(w, plan))

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    used = []
    for i in range(args.steps):
        flush()
        used.append(step(i, events[i]))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    names = ["plan", "dispatch", "prefetch", "gateup", "down", "combine"]
    per = {n: [] for n in names}
    for ev in events:
        for j, n in enumerate(names):
            per[n].append(ev[j].elapsed_time(ev[j + 1]) * 1e-3)     # seconds
    per["ffn"] = [a + b for a, b in zip(per["gateup"], per["down"])]
    pb, db, cb = alg_bytes(w)
    t_pdc = sum(per["plan"]) + sum(per["dispatch"]) + sum(per["combine"])
    gbs = args.steps * (pb + db + cb) / t_pdc / 1e9
    t_ffn = float(np.mean(per["ffn"]))
    tflops = ffn_flops(w) / t_ffn / 1e12
    t_gu = float(np.mean(per["gateup"]))
    t_dn = float(np.mean(per["down"]))
    t_disp = float(np.mean(per["dispatch"]))
    t_comb = float(np.mean(per["combine"]))
    t_plan = float(np.mean(per["plan"]))

    # per-target sweep: 3 warm-up and sweep_reps timed steps at each target,
    # each after a cache flush; stage medians
    print(f"[bench] sweep: {args.sweep_reps} steps per target", file=sys.stderr, flush=True)
    sw = {}
    for ti, t in enumerate(targets):
        for _ in range(3):
            flush()
            step(ti)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)]
               for _ in range(args.sweep_reps)]
        for r in range(args.sweep_reps):
            flush()
            step(ti, evs[r])
        torch.cuda.synchronize()
        sw[t] = {n: [ev[j].elapsed_time(ev[j + 1]) * 1e-3 for ev in evs]
                 for j, n in enumerate(names)}
        sw[t]["ffn"] = [a + b for a, b in zip(sw[t]["gateup"], sw[t]["down"])]
        # the plan alone, back to back after one cache flush (in the step it follows
        # the previous step's FFN, whose power state slows this latency-bound kernel chain)
        flush()
        pe = [torch.cuda.Event(enable_timing=True) for _ in range(args.sweep_reps + 4)]
        _, topk_t, _ = batches[ti]
        pe[0].record()
        for r in range(args.sweep_reps + 3):
            buf.plan(topk_t, plan=plan)
            pe[r + 1].record()
        torch.cuda.synchronize()
        sw[t]["plan_b2b"] = [pe[r].elapsed_time(pe[r + 1]) * 1e-3 for r in range(3, args.sweep_reps + 3)]

    sweep = {}
    for t in targets:
        if args.sweep_reps <= 0:
            continue
        m = lambda n: float(np.median(sw[t][n]))
        sweep[str(t)] = {
            "realized_maxvio": round(stats[t]["maxvio"], 4), "dups": stats[t]["dups"],
            "pad_rows": stats[t]["pad_rows"],
            "plan_us": round(m("plan") * 1e6, 2),
            "plan_back_to_back_us": round(m("plan_b2b") * 1e6, 2),
            "plan_GBps": round(pb / m("plan") / 1e9, 1),
            "dispatch_us": round(m("dispatch") * 1e6, 1),
            "prefetch_us": round(m("prefetch") * 1e6, 1), "ffn_ms": round(m("ffn") * 1e3, 3),
            "gateup_ms": round(m("gateup") * 1e3, 3), "down_ms": round(m("down") * 1e3, 3),
            "combine_us": round(m("combine") * 1e6, 1),
            "pdc_GBps": round((pb + db + cb) / (m("plan") + m("dispatch") + m("combine")) / 1e9, 1),
            "dispatch_stacked_us": round((m("plan") + m("prefetch") + m("dispatch")) * 1e6, 1),
            "gemm_TFLOPs": round(ffn_flops(w) / m("ffn") / 1e12, 1),
        }

    # flatness (MoonEP README "Performance": time nearly flat in maxvio): each
    # target's FFN and plan+dispatch+combine time over the lowest target's
    keys = list(sweep)
    if keys:
        t0 = keys[0]
        for k in keys:
            sweep[k]["ffn_over_first"] = round(sweep[k]["ffn_ms"] / sweep[t0]["ffn_ms"], 3)
            sweep[k]["pdc_over_first"] = round(sweep[t0]["pdc_GBps"] / sweep[k]["pdc_GBps"], 3)
            for st in ("plan_us", "dispatch_us", "combine_us"):
                sweep[k][st.split("_")[0] + "_over_first"] = round(sweep[k][st] / sweep[t0][st], 3)

    # algorithmic FFN bytes averaged over the timed steps (each step's plan)
    gu_bytes = float(np.mean([stats[u]["gateup_bytes"] for u in used]))
    dn_bytes = float(np.mean([stats[u]["down_bytes"] for u in used]))
    result = {
        "metric": "plan+dispatch+combine GB/s, grouped-GEMM TFLOP/s vs maxvio, 1 rank",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Zipf-biased top-K routing, N(0,1) hidden, N(0,0.02) weights)",
        "config": {"workload": w.name, "R": w.R, "S": w.S, "K": w.K, "E": w.E, "B": w.B,
                   "H": w.H, "Hp": w.Hp, "token_padding": w.token_padding,
                   "maxvio_targets": [str(t) for t in targets],
                   "step": f"plan, dispatch, prefetch_weight, expert_gateup + expert_down "
                           f"({w.R} ranks), combine"},
        "gemm_tflops": round(tflops, 1),
        "roofline": {**ffn_roofline(
            f"ffn_gateup (gate and up GEMMs + SwiGLU, all {w.R} ranks, one launch)",
            gateup_flops(w), gu_bytes, t_gu),
            "traffic": measured_traffic("ffn_gateup") if w.name == WORKLOAD else None},
        "roofline_down": {**ffn_roofline(f"ffn_down (down GEMM, all {w.R} ranks, one launch)",
                                         down_flops(w), dn_bytes, t_dn),
                          "traffic": measured_traffic("ffn_down") if w.name == WORKLOAD else None},
        "roofline_dispatch": {"bound": "hbm", "achieved": round(db / t_disp / 1e9, 1),
                              "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(db / t_disp / 1e9 / HBM_PEAK_GBS, 4),
                              "traffic": measured_traffic("dispatch") if w.name == WORKLOAD else None,
                              "per_launch": {"bytes": db, "avg_s": t_disp}},
        "roofline_plan": {"bound": "latency", "achieved": round(pb / t_plan / 1e9, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(pb / t_plan / 1e9 / HBM_PEAK_GBS, 5),
                          "note": "three dependent kernels over 2 MB: bound by latency, not bytes",
                          "per_launch": {"bytes": pb, "avg_s": t_plan}},
        "roofline_combine": {"bound": "hbm", "achieved": round(cb / t_comb / 1e9, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(cb / t_comb / 1e9 / HBM_PEAK_GBS, 4),
                             "traffic": measured_traffic("combine") if w.name == WORKLOAD else None,
                             "per_launch": {"bytes": cb, "avg_s": t_comb}},
        "sweep": sweep,
    }
    if not args.no_per_rank:
        result["per_rank_ffn"] = time_per_rank(w, buf, batches, home, pool, x)
    props = torch.cuda.get_device_properties(0)
    result["device"] = {"name": getattr(props, "name", None),
                        "arch": getattr(props, "gcnArchName", None),
                        "compute_units": getattr(props, "multi_processor_count", None)}

    # the copy that zero-copy avoids (README "API guide > zero_copy"): copy
    # mode adds one copy of the used slots to dispatch and one to combine
    t_last, topk_last, _ = batches[-1]
    buf.plan(topk_last, plan=plan)
    scratch = torch.empty_like(x_nvs)
    for _ in range(2):
        buf.copy_rows(plan, x_nvs, scratch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        buf.copy_rows(plan, x_nvs, scratch)
    e1.record()
    torch.cuda.synchronize()
    t_copy = e0.elapsed_time(e1) / 5 * 1e-3
    used = int(buf.read_stats(plan)[4]) + w.R * w.S * w.K          # padding + real rows
    result["copy_mode"] = {
        "copy_rows_us": round(t_copy * 1e6, 1),
        "copy_rows_GBps": round(2 * 2 * w.H * used / t_copy / 1e9, 1),
        "dispatch_us_copy_mode": round((t_disp + t_copy) * 1e6, 1),
        "combine_us_copy_mode": round((t_comb + t_copy) * 1e6, 1),
        "note": f"one copy of the used slots (real + padding rows) per call, timed at maxvio {t_last}"}
    del scratch

    if args.graph:
        result["graph"] = time_graph(w, buf, batches, home, pool, x, max(3, args.steps))

    if args.views:
        result["views"] = time_views(w, buf, batches, home, pool, x, max(2, args.steps // 2))

    if args.overlap:
        result["overlap"] = time_overlap(w, batches, home, pool, max(2, args.steps // 2),
                                         max(1, args.warmup // 2))

    if args.train:
        result["train"] = time_backward(w, buf, plan, batches, x_nvs, z_ws, home, pool,
                                        args.steps, args.warmup, flush)
    buf.destroy()
    scratch_flush = None
    result["timing"] = (f"stage times from HIP events on the launch stream; {args.flush_mb} MiB "
                        f"written before every timed step (outside the stage events, inside "
                        f"ms_per_step) so the last-level cache holds none of the step's inputs; "
                        f"value and roofline: mean over the {args.steps} timed steps; sweep: "
                        f"medians of {args.sweep_reps} steps per target (plan_back_to_back_us: "
                        f"medians of {args.sweep_reps} plans in a row after one flush, outside "
                        f"the steps)")
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        t1 = 1.0 if 1.0 in host_routing else targets[0]
        result["cpu_baseline"] = cpu_baseline(w, host_routing, t1, x, home)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
