#!/usr/bin/env python3
"""Benchmark of the per-rank state-sharding engine on one MI355X.

One step is one pass of the whole hot path over the 7B Llama-style model's
rank-0 FSDP2 shard (N = 8 logical ranks, grad_acc = 4), all inputs resident
in HBM before timing starts:

  1. fs_pack    x33 groups  all-gather copy-in of every group (all N shards)
  2. fs_unpack  x33 groups  all-gather copy-out into per-parameter tensors
  3. fs_reduce_shard        32 bf16 gradient slices -> fp32 shard (842,301,440)
  4. fs_adamw_step          fp32 master/m/v update + bf16 parameter copy

The layout plans are built and uploaded once, before timing (a plan is made
once per group).  Throughput is algorithmic bytes (what the method must read
and write) per second; per-kernel durations come from HIP events recorded on
the stream the kernels run on.

Where the buffers land in HBM moves the rates by several percent, and the
process's allocation order decides it.  So the step is set up and timed once
per allocation order (parameters first, shard state first, plan tables
first), each from a freshly emptied allocator; the headline figures are those
of the order with the median step time, and every order's figures (and the
worst) are in the line too.  The 32 gradient slices live in one buffer, and
theta, m, v and the fp32 gradient in another (the engine's shard state as
one allocation).

After the 7B buffers are freed, the 70B model's rank-0 shard (80 blocks,
grad_acc = 2) is measured: the per-group reduce over a reused slice pool,
the whole-shard AdamW, and the per-group fused reduce + AdamW.  The CPU
baseline is the plain C oracle on a bounded sample of the 7B workload,
single-threaded and on every host core.

Prints one JSON line.  `--gpus N` with N > 1 is refused: this engine runs all
logical ranks on one GPU.
"""
import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E peak, 8 TB/s
KERNEL_SRCS = [os.path.join(ROOT, "fsdp_sharded_state_amd", "csrc", f)
               for f in ("fs_kernels.hip", "fs_internal.h", "fs_plan_impl.h", "fs_plan.cpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_7b_shard_step.json")

WORKLOADS = {
    # name: (n_blocks, d, f, kv, vocab, world, grad_acc)
    "7b": (32, 4096, 11008, None, 32000, 8, 4),
    "70b": (80, 8192, 28672, 1024, 32000, 8, 2),
}
# llama_model_groups(n_blocks, d, f, vocab, kv) arguments per workload
_WL_SHAPES = {k: (v[0], v[1], v[2], v[4], v[3]) for k, v in WORKLOADS.items()}
ORDERS = ("params_first", "state_first", "plans_first")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the library's sources with comments and layout removed: it
    changes when the code of a kernel, its launch shape or the planner's
    tiling changes, not when a comment does."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        src = open(path).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def setup(workload: str = "7b", seed: int = 4, order: str = "params_first", pooled: bool = True):
    """Allocate and fill every input in HBM, in the given order of the three
    allocation families: parameters, gathered buffers and copy-out targets
    ("params"); the gradient-slice pool, the fp32 shard state pool and the
    bf16 parameter copy ("state"); the plans' device tables ("plans")."""
    import torch

    import fsdp_sharded_state_amd as fs
    import synth

    n_blocks, d, f, kv, vocab, world, grad_acc = WORKLOADS[workload]
    groups = synth.llama_model_groups(n_blocks, d, f, vocab=vocab, kv=kv)
    probe = [fs.fs_plan(g, "bf16", world, False, "fsdp2", grad_acc) for g in groups]   # host only
    S = sum(p.shard_numel for p in probe)
    P = sum(p.total_numel for p in probe)
    gathered_numels = [p.gathered_numel for p in probe]
    del probe
    log(f"workload {workload}, order {order}: {len(groups)} groups, P={P}, shard S={S}, N={world}, A={grad_acc}")

    t0 = time.time()
    W = dict(fs=fs, S=S, P=P, world=world, grad_acc=grad_acc, groups=len(groups), workload=workload, order=order)

    def alloc_state():
        T = world * grad_acc
        if pooled:
            pool = torch.empty(T * S, dtype=torch.bfloat16, device="cuda")
            bufs = [pool[t * S:(t + 1) * S] for t in range(T)]
            st = torch.empty(4 * S, dtype=torch.float32, device="cuda")
            master, exp_avg, exp_avg_sq, grad32 = (st[i * S:(i + 1) * S] for i in range(4))
        else:
            bufs = [torch.empty(S, dtype=torch.bfloat16, device="cuda") for _ in range(T)]
            master, exp_avg, exp_avg_sq, grad32 = (torch.empty(S, dtype=torch.float32, device="cuda")
                                                   for _ in range(4))
        slices = []
        for j in range(grad_acc):
            for k in range(world):
                t = j * world + k
                slices.append(synth.fill_normal(bufs[t], seed, synth.stream_grad(j, k, world), 1e-3))
        synth.fill_normal(master, seed, synth.STREAM_MASTER, 0.02)
        exp_avg.zero_()
        exp_avg_sq.zero_()
        W.update(slices=slices, master=master, exp_avg=exp_avg, exp_avg_sq=exp_avg_sq, grad32=grad32,
                 p16=torch.empty(S, dtype=torch.bfloat16, device="cuda"))
        log(f"gradient slices and shard state generated ({time.time() - t0:.1f}s)")

    def alloc_params():
        params, gathered, outs = [], [], []
        off = 0
        for g, gn in zip(groups, gathered_numels):
            ps = []
            for s in g:
                n = math.prod(s)
                ps.append(synth.normal_bf16(seed, synth.STREAM_PARAMS, n, 0.02, device="cuda", start=off).view(*s))
                off += n
            params.append(ps)
            gathered.append(torch.empty(gn, dtype=torch.bfloat16, device="cuda"))
            outs.append([torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in g])
        W.update(params=params, gathered=gathered, outs=outs)
        log(f"parameters generated ({time.time() - t0:.1f}s)")

    def alloc_plans():
        W["plans"] = [fs.fs_plan(g, "bf16", world, False, "fsdp2", grad_acc).upload() for g in groups]

    steps = {"state_first": (alloc_state, alloc_params, alloc_plans),
             "plans_first": (alloc_plans, alloc_params, alloc_state),
             "params_first": (alloc_params, alloc_state, alloc_plans)}[order]
    for fn in steps:
        fn()
    torch.cuda.synchronize()
    log(f"inputs generated on the GPU in {time.time() - t0:.1f}s; "
        f"{torch.cuda.memory_allocated() / 1e9:.1f} GB allocated")
    return W


def release(W):
    """Drop every buffer of a setup and return the memory to the device."""
    import gc

    import torch
    W.clear()
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def algorithmic_bytes(W) -> dict:
    """Bytes each kernel must move (pads written by pack count; pads are never read)."""
    P, S, N, A = W["P"], W["S"], W["world"], W["grad_acc"]
    gathered = sum(p.gathered_numel for p in W["plans"])
    return {
        "pack": 2 * P + 2 * gathered,      # read every parameter, write every gathered element
        "unpack": 2 * P + 2 * P,           # read every parameter element of the gathered buffers, write it out
        "reduce": (2 * N * A + 4) * S,     # read N*A bf16 slices, write fp32
        "adamw": 30 * S,                   # read g, theta, m, v (fp32); write theta, m, v (fp32) + bf16 param
    }


def run_step(W, step_t, ev=None):
    fs = W["fs"]
    if ev:
        ev[0].record()
    for p, ps, g in zip(W["plans"], W["params"], W["gathered"]):
        fs.fs_pack(p, ps, g)
    if ev:
        ev[1].record()
    for p, g, o in zip(W["plans"], W["gathered"], W["outs"]):
        fs.fs_unpack(p, g, o)
    if ev:
        ev[2].record()
    fs.fs_reduce_shard(W["slices"], W["grad32"], W["world"], W["grad_acc"])
    if ev:
        ev[3].record()
    fs.fs_adamw_step(W["master"], W["exp_avg"], W["exp_avg_sq"], W["grad32"], W["p16"],
                     lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=step_t)
    if ev:
        ev[4].record()


PHASES = ["pack", "unpack", "reduce", "adamw"]


def measure_order(W, steps: int, warmup: int) -> dict:
    """Warm-up steps, then exactly `steps` timed steps (wall time between two
    device synchronizations, per-phase HIP events on the launch stream), then
    the fused reduce + AdamW entry point on the same shard."""
    import torch
    fs = W["fs"]
    alg = algorithmic_bytes(W)
    t = 1
    for _ in range(warmup):
        run_step(W, t)
        t += 1
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        run_step(W, t, evs[k])
        t += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / steps
    ms = {ph: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / steps for i, ph in enumerate(PHASES)}
    med = {ph: sorted(e[i].elapsed_time(e[i + 1]) for e in evs)[steps // 2] for i, ph in enumerate(PHASES)}
    kern = {ph: {"ms": round(ms[ph], 4), "ms_median": round(med[ph], 4), "GB": round(alg[ph] / 1e9, 3),
                 "GBps": round(alg[ph] / (ms[ph] * 1e-3) / 1e9, 1),
                 "frac_hbm_peak": round(alg[ph] / (ms[ph] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
            for ph in PHASES}
    ra_ms = ms["reduce"] + ms["adamw"]
    ra_gbps = (alg["reduce"] + alg["adamw"]) / (ra_ms * 1e-3) / 1e9
    kern["reduce_adamw"] = {"ms": round(ra_ms, 4), "GBps": round(ra_gbps, 1),
                            "frac_hbm_peak": round(ra_gbps / HBM_PEAK_GBPS, 4)}
    fz = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for k in range(steps):
        fz[k][0].record()
        fs.fs_reduce_adamw_step(W["slices"], W["master"], W["exp_avg"], W["exp_avg_sq"], W["p16"], None,
                                world=W["world"], grad_acc=W["grad_acc"], lr=1e-3, beta1=0.9, beta2=0.999,
                                eps=1e-8, weight_decay=0.01, step=t)
        fz[k][1].record()
        t += 1
    torch.cuda.synchronize()
    fused_ms = sum(e[0].elapsed_time(e[1]) for e in fz) / steps
    fused_bytes = (2 * W["world"] * W["grad_acc"] + 26) * W["S"]
    kern["reduce_adamw_fused"] = {"ms": round(fused_ms, 4), "GB": round(fused_bytes / 1e9, 3),
                                  "GBps": round(fused_bytes / (fused_ms * 1e-3) / 1e9, 1),
                                  "frac_hbm_peak": round(fused_bytes / (fused_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                                  "step_ms_with_fused": round(ms["pack"] + ms["unpack"] + fused_ms, 4)}
    step_bytes = sum(alg.values())
    return {"order": W["order"], "ms_per_step": ms_step, "value": step_bytes / (ms_step * 1e-3) / 1e9,
            "step_bytes": step_bytes, "alg": alg, "ms": ms, "kernels": kern, "next_t": t}


def placement_summary(r: dict) -> dict:
    k = r["kernels"]
    own = {f"{n}_of_own_buffer_ceiling": round(k[n]["GBps"] / r["own"][n]["ceiling_GBps"], 4)
           for n in ("reduce", "adamw") if "own" in r}
    return {**own, "ms_per_step": round(r["ms_per_step"], 4), "value_GBps": round(r["value"], 1),
            "frac_hbm_peak": round(r["value"] / HBM_PEAK_GBPS, 4),
            "reduce_GBps": k["reduce"]["GBps"], "adamw_GBps": k["adamw"]["GBps"],
            "pack_GBps": k["pack"]["GBps"], "unpack_GBps": k["unpack"]["GBps"],
            "reduce_adamw_ms": k["reduce_adamw"]["ms"], "reduce_adamw_frac_hbm_peak": k["reduce_adamw"]["frac_hbm_peak"],
            "reduce_adamw_fused_ms": k["reduce_adamw_fused"]["ms"],
            "reduce_adamw_fused_frac_hbm_peak": k["reduce_adamw_fused"]["frac_hbm_peak"]}


def _timed(fn, reps):
    import torch
    fn()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for e in evs:
        e[0].record()
        fn()
        e[1].record()
    torch.cuda.synchronize()
    return sum(e[0].elapsed_time(e[1]) for e in evs) / reps


def _timed_graph(fn, reps, calls=8):
    """GPU time per call of fn for launches too short to hide the Python
    call: `calls` calls of fn are captured back to back into one HIP graph
    (as a sequence of groups would issue them), the graph is replayed reps
    times, and the time is divided by reps * calls."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        g.replay()
    e.record()
    e.synchronize()
    del g
    return s.elapsed_time(e) / (reps * calls)


def extra_measurements(W, reps, small: bool = True) -> dict:
    """The engine's other entry points on the same workload, outside the
    headline step: the bf16 reduce dtype over the same 32 slices, and the
    fp32 -> bf16 cast copy-in of every group from fp32 parameters."""
    import torch

    import synth
    fs, S, N, A = W["fs"], W["S"], W["world"], W["grad_acc"]
    out = {}
    ms = _timed(lambda: fs.fs_reduce_shard_ex(W["slices"], W["grad32"], N, A, reduce_dtype="bf16"), reps)
    b = (2 * N * A + 4) * S
    out["reduce_bf16_reduce_dtype"] = {"ms": round(ms, 4), "GB": round(b / 1e9, 3),
                                       "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                                       "frac_hbm_peak": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    p32, off = [], 0
    for ps in W["params"]:
        g = []
        for t in ps:
            g.append(synth.normal_f32(4, synth.STREAM_MASTER, t.numel(), 0.02, device="cuda", start=off))
            off += t.numel()
        p32.append(g)

    def cast_all():
        for p, g, gath in zip(W["plans"], p32, W["gathered"]):
            fs.fs_pack_cast(p, g, gath)
    ms = _timed(cast_all, reps)
    b = 4 * W["P"] + 2 * sum(p.gathered_numel for p in W["plans"])
    out["pack_cast_fp32_to_bf16"] = {"ms": round(ms, 4), "GB": round(b / 1e9, 3),
                                     "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                                     "frac_hbm_peak": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    del p32
    torch.cuda.empty_cache()
    # re-shard every group's gathered buffer from N to N/2 logical ranks
    import synth as _s
    groups = _s.llama_model_groups(*_WL_SHAPES[W["workload"]])
    half = [fs.fs_plan(g, "bf16", max(1, N // 2), False, "fsdp2", A).upload() for g in groups]
    rs = [fs.fs_reshard_plan(p, q).upload() for p, q in zip(W["plans"], half)]
    dst = [torch.empty(q.gathered_numel, dtype=torch.bfloat16, device="cuda") for q in half]

    def reshard_all():
        for r, g, d in zip(rs, W["gathered"], dst):
            fs.fs_reshard(r, g, d)
    ms = _timed(reshard_all, reps)
    b = 2 * W["P"] + 2 * sum(q.gathered_numel for q in half)
    out["reshard_n_to_half_n"] = {"ms": round(ms, 4), "GB": round(b / 1e9, 3),
                                  "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                                  "frac_hbm_peak": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    del dst, rs, half
    torch.cuda.empty_cache()
    # sharded state-dict import of rank 0 (fs_load_local): every group's local
    # pieces, held as separate tensors, written into that rank's shard buffer
    pieces, shards = [], []
    for p, gath in zip(W["plans"], W["gathered"]):
        views = p.local_views(gath[:p.shard_numel], 0)
        pieces.append([v.clone() for v in views])
        shards.append(torch.empty(p.shard_numel, dtype=torch.bfloat16, device="cuda"))

    def load_all():
        for p, pc, sh in zip(W["plans"], pieces, shards):
            p.load_local(sh, 0, pc)
    ms = _timed_graph(load_all, reps, calls=2)   # 33 launches of about 20 us each: replayed as a graph
    b = 2 * sum(v.numel() for pc in pieces for v in pc) + 2 * sum(sh.numel() for sh in shards)
    out["load_local_rank0"] = {"ms": round(ms, 4), "GB": round(b / 1e9, 3), "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                               "frac_hbm_peak": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    del pieces, shards
    torch.cuda.empty_cache()
    # the same groups under the FSDP1 FlatParameter layout (use_orig_params):
    # 16-byte-aligned parameter starts, flat chunked into N equal shards
    f1 = [fs.fs_plan(g, "bf16", N, True, "fsdp1", A).upload() for g in groups] if small else []
    if f1 and all(p.gathered_numel == g.numel() for p, g in zip(f1, W["gathered"])):
        ms_p = _timed(lambda: [fs.fs_pack(p, ps, g) for p, ps, g in zip(f1, W["params"], W["gathered"])], reps)
        ms_u = _timed(lambda: [fs.fs_unpack(p, g, o) for p, g, o in zip(f1, W["gathered"], W["outs"])], reps)
        bp = 2 * W["P"] + 2 * sum(p.gathered_numel for p in f1)
        bu = 4 * W["P"]
        out["fsdp1_flat_pack"] = {"ms": round(ms_p, 4), "GB": round(bp / 1e9, 3), "GBps": round(bp / (ms_p * 1e-3) / 1e9, 1)}
        out["fsdp1_flat_unpack"] = {"ms": round(ms_u, 4), "GB": round(bu / 1e9, 3), "GBps": round(bu / (ms_u * 1e-3) / 1e9, 1)}
    del f1
    if not small:
        return out
    # one transformer block's shard at a time, the granularity at which FSDP
    # reduces a group: 8 gradient buffers (grad_acc = 1) of 25,297,920 elements
    sb = 25_297_920
    sl1 = [t[:sb] for t in W["slices"][:N]]
    gb, th, m, v, pb = (W[k][:sb] for k in ("grad32", "master", "exp_avg", "exp_avg_sq", "p16"))
    ms_r = _timed_graph(lambda: fs.fs_reduce_shard(sl1, gb, N, 1), 4 * reps)
    ms_a = _timed_graph(lambda: fs.fs_adamw_step(th, m, v, gb, pb, lr=1e-3, step=2), 4 * reps)
    ms_f = _timed_graph(lambda: fs.fs_reduce_adamw_step(sl1, th, m, v, pb, None, world=N, grad_acc=1, step=3),
                        4 * reps)
    br, ba, bfz = (2 * N + 4) * sb, 30 * sb, (2 * N + 26) * sb
    # one block group's copy-in (all N shards) and copy-out, 202,383,360 parameters
    bpl, bps, bg, bo = W["plans"][0], W["params"][0], W["gathered"][0], W["outs"][0]
    ms_bp = _timed_graph(lambda: fs.fs_pack(bpl, bps, bg), 4 * reps)
    ms_bu = _timed_graph(lambda: fs.fs_unpack(bpl, bg, bo), 4 * reps)
    bbp, bbu = 2 * bpl.total_numel + 2 * bpl.gathered_numel, 4 * bpl.total_numel
    # the padding-stress parameter list (97 parameters, 21,444,378 elements, FSDP1
    # with use_orig_params, N = 8): alignment and world pads, short segments
    st = [(n,) for n in synth.padding_stress_numels()]
    pst = fs.fs_plan(st, "bf16", N, True, "fsdp1", 1).upload()
    prm = [synth.normal_bf16(3, synth.STREAM_PARAMS, n[0], 0.02, device="cuda") for n in st]
    gst = torch.empty(pst.gathered_numel, dtype=torch.bfloat16, device="cuda")
    ost = [torch.empty_like(t) for t in prm]
    ms_p = _timed_graph(lambda: fs.fs_pack(pst, prm, gst), 4 * reps)
    ms_u = _timed_graph(lambda: fs.fs_unpack(pst, gst, ost), 4 * reps)
    bp, bu = 2 * pst.total_numel + 2 * pst.gathered_numel, 4 * pst.total_numel
    out["padding_stress_fsdp1"] = {
        "params": len(st), "numel": pst.total_numel, "gathered_numel": pst.gathered_numel,
        "pack": {"us": round(ms_p * 1e3, 1), "GBps": round(bp / (ms_p * 1e-3) / 1e9, 1)},
        "unpack": {"us": round(ms_u * 1e3, 1), "GBps": round(bu / (ms_u * 1e-3) / 1e9, 1)}}
    del prm, gst, ost
    out["block_shard_grad_acc_1"] = {
        "shard_numel": sb,
        "reduce": {"us": round(ms_r * 1e3, 1), "GB": round(br / 1e9, 3), "GBps": round(br / (ms_r * 1e-3) / 1e9, 1)},
        "adamw": {"us": round(ms_a * 1e3, 1), "GB": round(ba / 1e9, 3), "GBps": round(ba / (ms_a * 1e-3) / 1e9, 1)},
        "reduce_adamw_fused": {"us": round(ms_f * 1e3, 1), "GB": round(bfz / 1e9, 3),
                               "GBps": round(bfz / (ms_f * 1e-3) / 1e9, 1)},
        "pack": {"params": bpl.total_numel, "us": round(ms_bp * 1e3, 1), "GB": round(bbp / 1e9, 3),
                 "GBps": round(bbp / (ms_bp * 1e-3) / 1e9, 1)},
        "unpack": {"params": bpl.total_numel, "us": round(ms_bu * 1e3, 1), "GB": round(bbu / 1e9, 3),
                   "GBps": round(bbu / (ms_bu * 1e-3) / 1e9, 1)}}
    return out


def tiny_step_latency(fs, reps=200) -> dict:
    """The launch-bound tiny case (2-layer MLP, FSDP1 with use_orig_params,
    N = 4): pack of all ranks, unpack, reduce and AdamW, timed per step
    eagerly and as one replayed HIP graph of the same four launches."""
    import torch

    import synth
    shapes = synth.mlp_tiny_shapes()
    N = 4
    plan = fs.fs_plan(shapes, "bf16", N, True, "fsdp1", 1).upload()
    S = plan.shard_numel
    params, off = [], 0
    for s in shapes:
        n = math.prod(s)
        params.append(synth.normal_bf16(1, synth.STREAM_PARAMS, n, 0.02, device="cuda", start=off).view(*s))
        off += n
    outs = [torch.empty_like(p) for p in params]
    gathered = torch.empty(plan.gathered_numel, dtype=torch.bfloat16, device="cuda")
    slices = [synth.normal_bf16(1, synth.stream_grad(0, k, N), S, 1e-3, device="cuda") for k in range(N)]
    master = synth.normal_f32(1, synth.STREAM_MASTER, S, 0.02, device="cuda")
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    g32, p16 = torch.empty_like(master), torch.empty(S, dtype=torch.bfloat16, device="cuda")

    def step():
        fs.fs_pack(plan, params, gathered)
        fs.fs_unpack(plan, gathered, outs)
        fs.fs_reduce_shard(slices, g32, N, 1)
        fs.fs_adamw_step(master, m, v, g32, p16, lr=1e-3, step=1)

    for _ in range(10):
        step()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        step()
    e.record()
    e.synchronize()
    eager_us = s.elapsed_time(e) * 1e3 / reps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(10):
        g.replay()
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        g.replay()
    e.record()
    e.synchronize()
    graph_us = s.elapsed_time(e) * 1e3 / reps
    del g
    return {"eager_us_per_step": round(eager_us, 2), "graph_us_per_step": round(graph_us, 2),
            "launches_per_step": 4, "shard_numel": S}


def stream_ceilings(fs, nbytes=8 << 30, reps=5) -> dict:
    """Achieved GB/s of a plain read-only stream and a plain write-only
    stream of nbytes (median of reps), the two ends between which every
    kernel's read/write mix falls."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.uint8, device="cuda")
    fs.fs_stream_fill(a, 0x01010101)
    out = {}
    for name, fn in (("read", lambda: fs.fs_stream_read(a, sink)), ("write", lambda: fs.fs_stream_fill(a, 0x01010101))):
        fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(reps):
            s.record()
            fn()
            e.record()
            e.synchronize()
            times.append(s.elapsed_time(e))
        out[name] = nbytes / (sorted(times)[len(times) // 2] * 1e-3) / 1e9
    del a, sink
    torch.cuda.empty_cache()
    return out


def own_buffer_ceilings(W, reps=3) -> dict:
    """The reduce's and AdamW's bytes streamed over their own buffers, reads
    and writes apart: read-only passes over every input buffer and write-only
    passes over every output buffer, timed with events around each pass (median
    of reps).  Same buffers, so the same physical placement as the kernels.
    Overwrites the shard state: run it last."""
    import torch
    fs = W["fs"]
    sink = torch.zeros(4, dtype=torch.uint8, device="cuda")

    def med(fn):
        fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(reps):
            s.record()
            fn()
            e.record()
            e.synchronize()
            ts.append(s.elapsed_time(e))
        return sorted(ts)[len(ts) // 2]

    out = {}
    for name, reads, writes in (("reduce", W["slices"], [W["grad32"]]),
                                ("adamw", [W["grad32"], W["master"], W["exp_avg"], W["exp_avg_sq"]],
                                 [W["master"], W["exp_avg"], W["exp_avg_sq"], W["p16"]])):
        t_r = sum(med(lambda t=t: fs.fs_stream_read(t, sink)) for t in reads)
        t_w = sum(med(lambda t=t: fs.fs_stream_fill(t, 0)) for t in writes)
        rb = sum(t.numel() * t.element_size() for t in reads)
        wb = sum(t.numel() * t.element_size() for t in writes)
        out[name] = {"read_GBps": round(rb / (t_r * 1e-3) / 1e9, 1), "write_GBps": round(wb / (t_w * 1e-3) / 1e9, 1),
                     "ceiling_GBps": round((rb + wb) / ((t_r + t_w) * 1e-3) / 1e9, 1)}
    return out


def mix_ceiling(read_bytes: float, write_bytes: float, ceil: dict) -> float:
    """GB/s a kernel moving these bytes would reach if its reads ran at the
    read-only stream rate and its writes at the write-only rate, one after
    the other."""
    t = read_bytes / ceil["read"] + write_bytes / ceil["write"]
    return (read_bytes + write_bytes) / t


def copy_ceiling(fs, nbytes=1 << 32, reps=5):
    """Achieved GB/s of a plain dwordx4 copy (read + write) of nbytes."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    fs.fs_copy_bytes(b, a)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(reps):
        s.record()
        fs.fs_copy_bytes(b, a)
        e.record()
        e.synchronize()
        times.append(s.elapsed_time(e))
    del a, b
    torch.cuda.empty_cache()
    t = sorted(times)[len(times) // 2]
    return 2 * nbytes / (t * 1e-3) / 1e9



def measure_70b(reps: int = 3, seed: int = 5) -> dict:
    """The 70B Llama-style model's rank-0 FSDP2 shard (80 blocks with grouped
    k/v, N = 8, grad_acc = 2): 8,622,080,000 elements of fp32 theta, m, v and
    gradient plus the bf16 copy, resident at once (155 GB).  The reduce runs
    group by group, as FSDP reduces a group at a time, over a slice pool that
    holds one block group's 16 slices and is reused by every group (each
    launch still streams its slices from HBM: 3.4 GB against a 256 MB cache);
    AdamW runs once over the whole shard; the fused reduce + AdamW runs group
    by group.  Median of `reps` passes each."""
    import torch

    import fsdp_sharded_state_amd as fs
    import synth

    n_blocks, d, f, kv, vocab, N, A = WORKLOADS["70b"]
    blk = fs.fs_plan(synth.llama_block_shapes(d, f, kv), "bf16", N, False, "fsdp2", A)
    root = fs.fs_plan([(vocab, d), (vocab, d)], "bf16", N, False, "fsdp2", A)
    sizes = [blk.shard_numel] * n_blocks + [root.shard_numel]
    S, T, Sb = sum(sizes), N * A, max(sizes)
    t0 = time.time()
    st = torch.empty(4 * S, dtype=torch.float32, device="cuda")
    master, m, v, g32 = (st[i * S:(i + 1) * S] for i in range(4))
    synth.fill_normal(master, seed, synth.STREAM_MASTER, 0.02)
    m.zero_()
    v.zero_()
    p16 = torch.empty(S, dtype=torch.bfloat16, device="cuda")
    pool = torch.empty(T * Sb, dtype=torch.bfloat16, device="cuda")
    for j in range(A):
        for k in range(N):
            t = j * N + k
            synth.fill_normal(pool[t * Sb:(t + 1) * Sb], seed, synth.stream_grad(j, k, N), 1e-3)
    torch.cuda.synchronize()
    log(f"70B shard state ({S} elements) and slice pool generated in {time.time() - t0:.1f}s; "
        f"{torch.cuda.memory_allocated() / 1e9:.1f} GB allocated")
    offs = [0]
    for n in sizes:
        offs.append(offs[-1] + n)
    sl = [[pool[t * Sb:t * Sb + n] for t in range(T)] for n in sizes[-2:]]   # block and root views
    views = [sl[0] if i < n_blocks else sl[1] for i in range(len(sizes))]

    def reduce_all():
        for i, n in enumerate(sizes):
            fs.fs_reduce_shard(views[i], g32[offs[i]:offs[i + 1]], N, A)

    def fused_all(step):
        for i, n in enumerate(sizes):
            a, b = offs[i], offs[i + 1]
            fs.fs_reduce_adamw_step(views[i], master[a:b], m[a:b], v[a:b], p16[a:b], None, world=N, grad_acc=A,
                                    step=step)

    def med(fn):
        fn(1)
        torch.cuda.synchronize()
        ts = []
        for r in range(reps):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn(r + 2)
            e.record()
            e.synchronize()
            ts.append(s.elapsed_time(e))
        return sorted(ts)[len(ts) // 2]

    ms_r = med(lambda step: reduce_all())
    ms_a = med(lambda step: fs.fs_adamw_step(master, m, v, g32, p16, step=step))
    ms_f = med(fused_all)
    br, ba, bf = (2 * N * A + 4) * S, 30 * S, (2 * N * A + 26) * S

    def ent(ms, b, target_ms=None):
        e = {"ms": round(ms, 3), "GB": round(b / 1e9, 2), "GBps": round(b / (ms * 1e-3) / 1e9, 1),
             "frac_hbm_peak": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        if target_ms:
            e["target_ms_at_80pct"] = target_ms
        return e
    out = {"workload": "70B Llama-style model (80 blocks, d 8192, f 28672, k/v 8192x1024, vocab 32000), "
                       "rank 0's FSDP2 1/8 shard, grad_acc 2",
           "shard_numel": S, "groups": len(sizes),
           "launches_per_reduce": sum(launches_per_call("reduce", c, N * A, N) for c in sizes),
           "launches_per_adamw": launches_per_call("adamw", S),
           "reduce": ent(ms_r, br, round(br / (0.8 * HBM_PEAK_GBPS) / 1e6, 1)),
           "adamw": ent(ms_a, ba, round(ba / (0.8 * HBM_PEAK_GBPS) / 1e6, 1)),
           "reduce_adamw": ent(ms_r + ms_a, br + ba),
           "reduce_adamw_fused": ent(ms_f, bf)}
    del st, master, m, v, g32, p16, pool, sl, views
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def cpu_baseline(workload: str = "7b", seed: int = 4, reps: int = 5) -> dict:
    """The oracle, as it stands, on a bounded sample of the same workload:
    reduce (32 bf16 slices) + AdamW over the first n_s shard elements, and
    pack + unpack of one transformer block group.  Timed single-threaded (the
    build every check uses) and with its OpenMP build on every host core the
    process may use: one warm-up pass, then `reps` passes, median."""
    import numpy as np

    import oracle
    import synth

    n_blocks, d, f, kv, vocab, world, grad_acc = WORKLOADS[workload]
    n_s = 1 << 22
    # same generator and streams as the GPU run, evaluated on the GPU for speed
    sl = [synth.to_numpy_bits(synth.normal_bf16(seed, synth.stream_grad(j, k, world), n_s, 1e-3, device="cuda"))
          for j in range(grad_acc) for k in range(world)]
    th = synth.normal_f32(seed, synth.STREAM_MASTER, n_s, 0.02, device="cuda").cpu().numpy()
    z = np.zeros(n_s, np.float32)
    block = synth.llama_block_shapes(d, f, kv)
    L = oracle.fsdp2_layout(block, 2, world)
    nb = int(L.numel.sum())
    prm = [np.frombuffer(np.random.default_rng(k).bytes(2 * int(n)), np.uint16) for k, n in enumerate(L.numel)]
    hp = oracle.AdamWHparams(step=1)
    sample_bytes = ((2 * world * grad_acc + 4) * n_s + 30 * n_s + (2 * nb + 2 * L.gathered_numel) + 4 * nb)

    def one_pass(par):
        t0 = time.perf_counter()
        g = oracle.reduce_shard(sl, world, grad_acc, parallel=par)
        oracle.adamw_step(th, z, z, g, hp, parallel=par)
        gath = oracle.pack(L, prm, parallel=par)
        oracle.unpack(L, gath, parallel=par)
        return time.perf_counter() - t0

    res = {}
    for par in (False, True):
        one_pass(par)
        ts = sorted(one_pass(par) for _ in range(reps))
        res[par] = (sample_bytes / ts[len(ts) // 2] / 1e9, ts[len(ts) // 2])
    threads = oracle.threads(True)
    return {
        "value": res[True][0], "unit": "GB/s", "cores": threads, "kind": "oracle",
        "value_1t": res[False][0], "value_all_cores": res[True][0],
        "host_cpu_count": os.cpu_count(),
        "sample": (f"reduce ({world * grad_acc} bf16 slices) + AdamW over {n_s} of the rank-0 shard's elements, "
                   f"pack + unpack of one block group ({nb} params): {sample_bytes / 1e9:.2f} GB of algorithmic "
                   f"traffic per pass; median of {reps} passes after one warm-up: "
                   f"{res[False][1]:.2f} s single-threaded, {res[True][1]:.3f} s on {threads} threads "
                   f"(OpenMP build of the same source)"),
    }


def traffic_for(kernel: str, launch_bytes_alg: float):
    """HBM bytes per launch from the committed PMC summary, or None when the
    kernel source changed since the counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


# the reduce's kernel for passes of more than 16 terms (its template argument
# is the number of 4-element groups per lane)
REDUCE_KERNEL = "reduce_chunk_kernel<16>"

# The library runs a call over n elements as consecutive launches over
# sub-ranges of at most this many elements (per pass of up to 32 terms); the
# values mirror kSpan, kRsSpan and kAdamSpan in fs_kernels.hip (a CPU test
# checks that they agree).
LAUNCH_SPAN = {"reduce": 32 << 20, "reduce_bf16_reduce_dtype": 16 << 20, "reduce_adamw_fused": 32 << 20,
               "adamw": 64 << 20}


def launches_per_call(phase: str, n: int, terms: int = 32, world: int = 8) -> int:
    """Kernel launches of one call of `phase` over n elements."""
    spans = -(-n // LAUNCH_SPAN[phase])
    if phase == "reduce":
        passes = -(-terms // 32)
    elif phase == "reduce_bf16_reduce_dtype":
        passes = -(-(terms // world) // (32 // world))
    else:
        passes = 1            # AdamW; the fused step's passes before the last are reduce launches
    return spans * passes

KERNELS = {  # rocprofv3 kernel-name fragment -> bench phase
    REDUCE_KERNEL: "reduce",
    "scatter_kernel<2, (anonymous namespace)::UnpackSrc": "reshard",
    "reduce_rs_chunk_kernel": "reduce_bf16_reduce_dtype",
    "pack_cast_kernel": "pack_cast",
    "reduce_adamw_chunk_kernel": "reduce_adamw_fused",
    "adamw_kernel": "adamw",
    "scatter_kernel<2, (anonymous namespace)::PackSrc": "pack",
    "unpack_kernel": "unpack",
    "copy_kernel": "copy",
}


def summarize_rocprof(kt_dir: str, fetch_dir: str, write_dir: str, commands: list, bench_line: str = "",
                      out_dir: str = os.path.join(ROOT, "profiles")):
    """Turn rocprofv3 CSV output (kernel trace + stats, and one --pmc pass each
    for FETCH_SIZE and WRITE_SIZE) into profiles/kernels_7b_shard_step.md and
    profiles/traffic_7b_shard_step.json.  HBM bytes per launch are the counter
    values (KiB) scaled by what the same counter reads for the plain copy
    kernel (bench's copy-ceiling launches: 4 GiB read and 4 GiB written)."""
    import csv
    import glob

    def one(d, pat):
        f = glob.glob(os.path.join(d, "**", pat), recursive=True)
        if not f:
            raise SystemExit(f"no {pat} under {d}")
        return f[0]

    def kname(n):
        for frag in KERNELS:
            i = n.find("(anonymous namespace)::" + frag)
            if i >= 0 and n[i + len("(anonymous namespace)::" + frag):][:1] in ("(", "<", ">"):
                return frag
        return None

    stats = {}
    for r in csv.DictReader(open(one(kt_dir, "*kernel_stats.csv"))):
        k = kname(r["Name"])
        if k:
            stats[k] = {"calls": int(r["Calls"]), "avg_ns": float(r["AverageNs"]),
                        "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"])}
    counters = {}
    for d, pat in ((fetch_dir, "*counter_collection.csv"), (write_dir, "*counter_collection.csv")):
        for r in csv.DictReader(open(one(d, pat))):
            k = kname(r["Kernel_Name"])
            if k:
                counters.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    avg = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in counters.items()}
    copy_bytes = float(1 << 32)
    f_fetch = copy_bytes / (avg["copy_kernel"]["FETCH_SIZE"] * 1024)
    f_write = copy_bytes / (avg["copy_kernel"]["WRITE_SIZE"] * 1024)
    # algorithmic bytes per call of the 7B shard step, and the launches of one call
    S, N, A = 842301440, 8, 4
    alg = {REDUCE_KERNEL: (2 * N * A + 4) * S, "adamw_kernel": 30 * S,
           "reduce_adamw_chunk_kernel": (2 * N * A + 26) * S,
           "reduce_rs_chunk_kernel": (2 * N * A + 4) * S,
           "copy_kernel": 2 * copy_bytes}
    nl = {REDUCE_KERNEL: launches_per_call("reduce", S, N * A, N),
          "adamw_kernel": launches_per_call("adamw", S),
          "reduce_adamw_chunk_kernel": launches_per_call("reduce_adamw_fused", S),
          "reduce_rs_chunk_kernel": launches_per_call("reduce_bf16_reduce_dtype", S, N * A, N),
          "copy_kernel": 1}
    for k in KERNELS:
        alg.setdefault(k, None)   # pack / unpack / reshard: per group, reported as means below
        nl.setdefault(k, 1)
    rec = {"kernel_source_sha256_16": kernel_source_hash(), "fetch_scale": f_fetch, "write_scale": f_write,
           "kernels": {}}
    rows = []
    for k in KERNELS:
        if k not in avg or k not in stats:
            continue
        fe = avg[k].get("FETCH_SIZE", 0.0) * 1024 * f_fetch
        wr = avg[k].get("WRITE_SIZE", 0.0) * 1024 * f_write
        hbm = fe + wr
        a = alg.get(k) / nl[k] if alg.get(k) else None      # mean algorithmic bytes per launch
        ent = {"avg_ns": stats[k]["avg_ns"], "calls": stats[k]["calls"], "launches_per_call": nl[k],
               "fetch_bytes_per_launch": fe, "write_bytes_per_launch": wr, "hbm_bytes_per_launch": hbm}
        if a:
            ent["alg_bytes_per_launch"] = a
            ent["hbm_over_alg"] = hbm / a
            ent["alg_GBps_from_trace"] = a / stats[k]["avg_ns"]
        rec["kernels"][KERNELS[k]] = ent
        rows.append((k, stats[k], fe, wr, a, nl[k]))
    os.makedirs(out_dir, exist_ok=True)
    json.dump(rec, open(os.path.join(out_dir, os.path.basename(TRAFFIC_FILE)), "w"), indent=1)
    md = ["# Kernel profile: 7B rank-0 FSDP2 shard step (N=8, grad_acc=4)", "",
          "Produced by these commands (from the repository root, on one MI355X):", ""]
    md += ["    " + c for c in commands]
    md += ["", "then `python bench.py --rocprof-summary <trace dir> <FETCH_SIZE dir> <WRITE_SIZE dir>`.", "",
           f"Counter scale (bytes per counted byte, from the 4 GiB copy kernel): FETCH_SIZE x{f_fetch:.4f}, "
           f"WRITE_SIZE x{f_write:.4f}.", "",
           "Kernel rates move by up to about 10% between allocations running the same code, with the",
           "physical placement of the buffers; compare the trace with the bench line of the same run",
           "(at the end, one allocation order), not with another run's.", "",
           "Long calls run as several launches over sub-ranges of the shard (launches per call below);",
           "per-launch figures are means over those launches: the call's algorithmic bytes divided by",
           "its launches, against the mean launch duration and the mean counter values.", "",
           "| kernel | launches | per call | avg duration | HBM read / launch | HBM write / launch | algorithmic / launch | HBM / alg | alg GB/s (trace) |",
           "|---|---|---|---|---|---|---|---|---|"]
    for k, st, fe, wr, a, L in rows:
        md.append(f"| {k} | {st['calls']} | {L} | {st['avg_ns'] / 1e3:.1f} us | {fe / 1e9:.3f} GB | {wr / 1e9:.3f} GB | "
                  + (f"{a / 1e9:.3f} GB | {(fe + wr) / a:.3f} | {a / st['avg_ns']:.0f} |" if a else "per group (see below) | - | - |"))
    pk = "scatter_kernel<2, (anonymous namespace)::PackSrc"
    if pk in stats:
        P = 6738411520
        for k in (pk, "unpack_kernel"):
            tot_alg = (2 * P + 2 * P) / 33
            md.append("")
            md.append(f"{k}: mean over the 33 group launches of one step: {stats[k]['avg_ns'] / 1e3:.1f} us, "
                      f"mean algorithmic bytes per launch {tot_alg / 1e9:.3f} GB "
                      f"({tot_alg / stats[k]['avg_ns']:.0f} GB/s).")
    if bench_line:
        md += ["", "Bench line of the traced run:", "", "    " + bench_line.strip()]
    open(os.path.join(out_dir, "kernels_7b_shard_step.md"), "w").write("\n".join(md) + "\n")
    print("\n".join(md))


def main():
    if len(sys.argv) >= 2 and sys.argv[1] == "--rocprof-summary":
        # --rocprof-summary TRACE_DIR FETCH_DIR WRITE_DIR [COMMANDS_FILE [BENCH_JSON [OUT_DIR]]]
        kt, fe, wr = sys.argv[2:5]
        cmds = open(sys.argv[5]).read().strip().splitlines() if len(sys.argv) > 5 else []
        line = open(sys.argv[6]).read() if len(sys.argv) > 6 else ""
        out_dir = sys.argv[7] if len(sys.argv) > 7 else os.path.join(ROOT, "profiles")
        summarize_rocprof(kt, fe, wr, cmds, line, out_dir)
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--orders", default=",".join(ORDERS),
                    help="comma-separated allocation orders to set up and time, each from an emptied allocator "
                         f"(default: all of {', '.join(ORDERS)})")
    ap.add_argument("--separate", action="store_true",
                    help="allocate every gradient slice and every shard-state array on its own instead of "
                         "one buffer for the slices and one for theta, m, v and the gradient")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-70b", action="store_true", help="skip the 70B shard measurement")
    ap.add_argument("--no-small", action="store_true",
                    help="skip the tiny launch-bound step, the one-block, padding-stress and FSDP1 "
                         "measurements (their launches would mix into a per-kernel profile of the 7B step)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this engine runs all N logical ranks on one GPU; "
                                   "--gpus above 1 is not supported", "n_gpus": args.gpus}))
        sys.exit(2)
    orders = [o for o in args.orders.split(",") if o]
    for o in orders:
        if o not in ORDERS:
            sys.exit(f"unknown allocation order {o!r}; choose from {', '.join(ORDERS)}")

    import torch
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    import fsdp_sharded_state_amd as fs

    runs, extra, mixes = [], None, None
    for i, order in enumerate(orders):
        W = setup("7b", order=order, pooled=not args.separate)
        r = measure_order(W, args.steps, args.warmup)
        log(f"order {order}: {r['ms_per_step']:.3f} ms per step, {r['value']:.0f} GB/s; reduce "
            f"{r['kernels']['reduce']['GBps']:.0f}, adamw {r['kernels']['adamw']['GBps']:.0f}, fused "
            f"{r['kernels']['reduce_adamw_fused']['ms']:.3f} ms")
        if i == 0:
            # the engine's other entry points, on the first order's placement
            extra = extra_measurements(W, args.steps, small=not args.no_small)
        # the streaming ceilings of the reduce's and AdamW's own buffers on this
        # placement; last on this setup: it overwrites the shard state
        r["own"] = own_buffer_ceilings(W)
        if i == 0:
            P, S, N, A = W["P"], W["S"], W["world"], W["grad_acc"]
            gath = sum(p.gathered_numel for p in W["plans"])
            mixes = {"pack": (2 * P, 2 * gath), "unpack": (2 * P, 2 * P), "reduce": (2 * N * A * S, 4 * S),
                     "adamw": (16 * S, 14 * S), "reduce_adamw_fused": ((2 * N * A + 12) * S, 14 * S),
                     "reduce_bf16_reduce_dtype": (2 * N * A * S, 4 * S),
                     "pack_cast_fp32_to_bf16": (4 * P, 2 * gath),
                     "load_local_rank0": (2 * S, 2 * S),
                     "reshard_n_to_half_n": (2 * P, extra["reshard_n_to_half_n"]["GB"] * 1e9 - 2 * P)}
            cfg = {"params": W["P"], "shard_numel": W["S"], "world": W["world"], "grad_acc": W["grad_acc"],
                   "groups": W["groups"]}
        runs.append(r)
        release(W)
        del W
    ceiling = copy_ceiling(fs)
    streams = stream_ceilings(fs)
    tiny = None if args.no_small else tiny_step_latency(fs)
    big = None if args.no_70b else measure_70b()

    # headline: the allocation order with the median step time
    ranked = sorted(runs, key=lambda r: r["ms_per_step"])
    head = ranked[len(ranked) // 2]
    worst = ranked[-1]
    kern = dict(head["kernels"])
    kern.update(extra)
    for k, (rb, wb) in mixes.items():
        c = mix_ceiling(rb, wb, streams)
        if k in kern:
            kern[k]["frac_of_copy_ceiling"] = round(kern[k]["GBps"] / ceiling, 4)
            kern[k]["mix_ceiling_GBps"] = round(c, 1)
            kern[k]["frac_of_mix_ceiling"] = round(kern[k]["GBps"] / c, 4)
    for k, v in head["own"].items():
        kern[k]["own_buffers"] = dict(v, frac=round(kern[k]["GBps"] / v["ceiling_GBps"], 4))
    if big is not None:
        kern["config5_70b"] = big
    alg = head["alg"]
    red_gbps = alg["reduce"] / (head["ms"]["reduce"] * 1e-3) / 1e9
    red_launches = launches_per_call("reduce", cfg["shard_numel"], cfg["world"] * cfg["grad_acc"], cfg["world"])
    traffic = traffic_for("reduce", alg["reduce"] / red_launches)
    ra = [r["kernels"]["reduce_adamw"]["frac_hbm_peak"] for r in runs]
    out = {
        "metric": "sharded AdamW+reduce step GB/s and % HBM peak; pack/unpack GB/s (7B, N=8)",
        "value": round(head["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "dtype_detail": {"pack/unpack": "bf16 bit copy", "reduce": "fp32 accumulate",
                         "adamw": "f64 math on fp32 state, bf16 copy"},
        "data": "synthetic",
        "config": dict({"workload": ("7B Llama-style model, rank 0's FSDP2 1/8 shard: pack + unpack of all 33 "
                                     "groups, reduce of 4x8 bf16 gradient slices, AdamW"),
                        "allocation_order": head["order"], "orders_timed": orders,
                        "state_buffers": "per array" if args.separate else "pooled",
                        "headline": "the allocation order with the median step time",
                        "step_bytes": head["step_bytes"]}, **cfg),
        "kernels": kern,
        "placements": {r["order"]: placement_summary(r) for r in runs},
        "value_worst_order": round(worst["value"], 1),
        "reduce_adamw_GBps": kern["reduce_adamw"]["GBps"],
        "reduce_adamw_frac_hbm_peak": kern["reduce_adamw"]["frac_hbm_peak"],
        "reduce_adamw_frac_hbm_peak_worst": min(ra),
        "reduce_adamw_frac_hbm_peak_median": statistics.median(ra),
        "copy_ceiling_GBps": round(ceiling, 1),
        "stream_ceilings_GBps": {k: round(v, 1) for k, v in streams.items()},
        "tiny_mlp_step": tiny,
        "roofline": {"bound": "hbm", "kernel": REDUCE_KERNEL, "achieved": round(red_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(red_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "alg_bytes_per_launch": round(alg["reduce"] / red_launches),
                     "launches_per_call": red_launches,
                     "note": ("per-launch bytes are means over the call's launches; achieved = the call's "
                              "algorithmic bytes over its time on HIP events")},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
