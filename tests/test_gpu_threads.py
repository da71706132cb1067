"""Calls from several host threads at once, each thread with its own stream,
plan and buffers.  The library's host side keeps no shared mutable state
besides per-device caches (atomics, or a lock for the no-allocation scratch
address) and a thread-local error message, so every thread's results must
equal a single-threaded run bit for bit, and an error in one thread must not
show up in another.  ctypes releases the GIL during each foreign call, so the
threads' calls do overlap on the host."""
import threading

import numpy as np
import pytest
import torch

import synth
from gpu_util import bits, say

pytestmark = pytest.mark.gpu
fs = pytest.importorskip("fsdp_sharded_state_amd")

SHAPES = [(1000, 37), (513,), (3, 333), (4097,), (64, 257)]
N, A = 4, 3          # 12 terms: one reduce pass
NT = 4               # threads
ITERS = 12


def _case(seed):
    """One thread's parameters (bf16, counter-based values from `seed`)."""
    numel = [int(np.prod(s)) for s in SHAPES]
    params = [synth.normal_bf16(seed, synth.STREAM_PARAMS, n, 0.02, device="cuda", start=o)
              for n, o in zip(numel, np.cumsum([0] + numel[:-1]).tolist())]
    return params


def _run(seed, stream, out, err_probe=0):
    """One thread's work: plan, pack, unpack, reduce, AdamW and the
    no-allocation fused step, ITERS times from the same inputs; the last
    iteration's outputs go to `out`.  With err_probe 1 or 2, every iteration
    also makes an invalid call of its own kind (a reduce with world 0, a pack
    to a rank out of range) and checks that its own message comes back."""
    with torch.cuda.stream(stream):
        plan = fs.fs_plan(SHAPES, "bf16", N, True, "fsdp1").upload(stream=stream)
        params = _case(seed)
        S = plan.shard_numel
        slices = [synth.normal_bf16(seed, synth.stream_grad(j, k, N), S, 1e-3, device="cuda")
                  for j in range(A) for k in range(N)]
        th0 = synth.normal_f32(seed, synth.STREAM_MASTER, S, 0.02, device="cuda")
        m0 = synth.normal_f32(seed, synth.STREAM_EXP_AVG, S, 1e-3, device="cuda")
        v0 = synth.normal_f32(seed, synth.STREAM_EXP_AVG_SQ, S, 1e-3, device="cuda") ** 2
        gathered = torch.empty(plan.gathered_numel, dtype=torch.bfloat16, device="cuda")
        outs = [torch.empty_like(p) for p in params]
        g = torch.empty(S, device="cuda")
        for it in range(ITERS):
            th, m, v = th0.clone(), m0.clone(), v0.clone()
            thf, mf, vf = th0.clone(), m0.clone(), v0.clone()
            p16, pf = (torch.empty(S, dtype=torch.bfloat16, device="cuda") for _ in range(2))
            fs.fs_pack(plan, params, gathered)
            fs.fs_unpack(plan, gathered, outs)
            fs.fs_reduce_shard(slices, g, N, A)
            fs.fs_adamw_step(th, m, v, g, p16, step=it + 1)
            fs.fs_reduce_adamw_step_noalloc(slices, thf, mf, vf, pf, world=N, grad_acc=A, step=it + 1)
            if err_probe == 1:
                with pytest.raises(fs.FsError, match=r"^FS_E_INVAL: fs_reduce_shard: world and grad_acc"):
                    fs.fs_reduce_shard([], g, 0, A)
            elif err_probe == 2:
                with pytest.raises(fs.FsError, match=rf"^FS_E_INVAL: fs_pack: rank {N + 3} out of range"):
                    fs.fs_pack(plan, params, gathered[:S], rank=N + 3)
        stream.synchronize()
    out.update({"gathered": bits(gathered), "outs": [bits(o) for o in outs], "g": bits(g),
                "state": [bits(x) for x in (th, m, v, p16)], "fused": [bits(x) for x in (thf, mf, vf, pf)]})


def test_threads_match_a_single_threaded_run():
    seeds = [71 + t for t in range(NT)]
    say("threads: single-threaded reference")
    ref = []
    for s in seeds:
        r = {}
        _run(s, torch.cuda.Stream(), r)
        ref.append(r)
    say("threads:", NT, "at once")
    got = [dict() for _ in seeds]
    failures = []

    def body(i):
        try:
            _run(seeds[i], torch.cuda.Stream(), got[i], err_probe=i % 3)
        except BaseException as e:   # reported below, in the main thread
            failures.append((i, repr(e)))

    threads = [threading.Thread(target=body, args=(i,)) for i in range(NT)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=100)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    torch.cuda.synchronize()
    assert not failures, failures
    for r, g in zip(ref, got):
        np.testing.assert_array_equal(r["gathered"], g["gathered"])
        for a, b in zip(r["outs"], g["outs"]):
            np.testing.assert_array_equal(a, b)
        np.testing.assert_array_equal(r["g"], g["g"])
        for a, b in zip(r["state"] + r["fused"], g["state"] + g["fused"]):
            np.testing.assert_array_equal(a, b)
    # the unpack round trip and the fused step's agreement with the two kernels
    for s, g in zip(seeds, got):
        for p, o in zip(_case(s), g["outs"]):
            np.testing.assert_array_equal(bits(p), o)
        for a, b in zip(g["state"], g["fused"]):
            np.testing.assert_array_equal(a, b)
