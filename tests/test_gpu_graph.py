"""Every launching entry point captured into one HIP graph (torch.cuda.graph)
and replayed: each replay must reproduce the eager run bit for bit.

The library allocates nothing, copies nothing and never synchronizes inside
a launching call, so a whole shard step can be captured once and replayed
(the launch-bound small groups gain most).  Pointer tables and plan
workspaces are uploaded by a warm-up call before capture.  Between replays
the test does its own eager work (restoring the state, scribbling over the
outputs, a full eager step on other buffers) and synchronizes; every replay
is compared with the eager result.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import bits, say

pytestmark = pytest.mark.gpu

fs = pytest.importorskip("fsdp_sharded_state_amd")

CASES = [
    # name, mode, shapes, world, use_orig_params, grad_acc
    ("mlp_tiny_fsdp1", "fsdp1", synth.mlp_tiny_shapes(), 4, True, 1),
    ("llama_block_d512_fsdp2", "fsdp2", synth.llama_block_shapes(512, 1376), 8, False, 4),
]

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fs.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


class Step:
    """Buffers of one shard step and the calls that make it."""

    def __init__(self, mode, shapes, N, uo, A, seed):
        self.N, self.A = N, A
        self.plan = fs.fs_plan(shapes, "bf16", N, uo, mode, A).upload()
        half = max(1, N // 2)
        self.plan_half = fs.fs_plan(shapes, "bf16", half, uo, mode, A).upload()
        self.resh = fs.fs_reshard_plan(self.plan, self.plan_half).upload()
        S = self.plan.shard_numel
        off, self.params, self.params32 = 0, [], []
        for s in shapes:
            n = int(np.prod(s)) if len(s) else 1
            self.params.append(synth.normal_bf16(seed, synth.STREAM_PARAMS, n, 0.02, device="cuda", start=off))
            self.params32.append(synth.normal_f32(seed, synth.STREAM_MASTER, n, 0.02, device="cuda", start=off))
            off += n
        self.slices = [synth.normal_bf16(seed, synth.stream_grad(j, k, N), S, 1e-3, device="cuda")
                       for j in range(A) for k in range(N)]
        self.init = [synth.normal_f32(seed, synth.STREAM_MASTER, S, 0.02, device="cuda"),
                     synth.normal_f32(seed, synth.STREAM_EXP_AVG, S, 1e-3, device="cuda"),
                     synth.normal_f32(seed, synth.STREAM_EXP_AVG_SQ, S, 1e-3, device="cuda").square()]
        self.state = [t.clone() for t in self.init]        # two-kernel path
        self.state_f = [t.clone() for t in self.init]      # fused path
        bf, f32 = torch.bfloat16, torch.float32
        self.outs = {
            "gathered": torch.empty(self.plan.gathered_numel, dtype=bf, device="cuda"),
            "shard0": torch.empty(S, dtype=bf, device="cuda"),
            "cast": torch.empty(self.plan.gathered_numel, dtype=bf, device="cuda"),
            "resharded": torch.empty(self.plan_half.gathered_numel, dtype=bf, device="cuda"),
            "grad32": torch.empty(S, dtype=f32, device="cuda"),
            "grad_rs": torch.empty(S, dtype=f32, device="cuda"),
            "p16": torch.empty(S, dtype=bf, device="cuda"),
            "p16_f": torch.empty(S, dtype=bf, device="cuda"),
            "grad_f": torch.empty(S, dtype=f32, device="cuda"),
        }
        self.unpacked = [torch.empty_like(p) for p in self.params]

    def reset(self):
        """Eager: restore the optimizer state, scribble over every output."""
        for dst, src in zip(self.state + self.state_f, self.init + self.init):
            dst.copy_(src)
        for t in list(self.outs.values()) + self.unpacked:
            t.view(torch.int16 if t.element_size() == 2 else torch.int32).fill_(0x5A5A)

    def run(self, t):
        o, p = self.outs, self.plan
        fs.fs_pack(p, self.params, o["gathered"])
        fs.fs_pack(p, self.params, o["shard0"], rank=0)
        fs.fs_pack_cast(p, self.params32, o["cast"])
        fs.fs_unpack(p, o["gathered"], self.unpacked)
        fs.fs_reshard(self.resh, o["gathered"], o["resharded"])
        fs.fs_reduce_shard_ex(self.slices, o["grad_rs"], self.N, self.A, reduce_dtype="bf16")
        fs.fs_reduce_shard(self.slices, o["grad32"], self.N, self.A)
        fs.fs_adamw_step(*self.state, o["grad32"], o["p16"], step=t, **HP)
        fs.fs_reduce_adamw_step(self.slices, *self.state_f, o["p16_f"], o["grad_f"], world=self.N,
                                grad_acc=self.A, step=t, **HP)

    def snapshot(self):
        ts = list(self.outs.values()) + self.unpacked + self.state + self.state_f
        return [bits(x) for x in ts]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_graph_replay_matches_eager(case):
    name, mode, shapes, N, uo, A = case
    t = 7
    say("graph eager reference", name)
    st = Step(mode, shapes, N, uo, A, seed=11)
    st.reset()
    st.run(t)
    torch.cuda.synchronize()
    ref = st.snapshot()

    say("graph warm-up on a side stream", name)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.reset()
        st.run(t)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    say("graph capture", name)
    st.reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run(t)
    torch.cuda.synchronize()

    other = Step(mode, shapes, N, uo, A, seed=12)
    for rep in range(3):
        say("graph replay", name, rep)
        st.reset()
        g.replay()
        torch.cuda.synchronize()
        got = st.snapshot()
        for k, (a, b) in enumerate(zip(got, ref)):
            np.testing.assert_array_equal(a, b, err_msg=f"{name}: replay {rep}, buffer {k}")
        # eager work between replays: a whole step on other buffers
        other.reset()
        other.run(t + rep)
        torch.cuda.synchronize()
    del g


def test_captured_pointer_table_outlives_later_pointer_sets(monkeypatch):
    """A captured graph holds the device address of the plan's pointer table
    for its parameters.  Ten other pointer sets going through the same plan
    afterwards (more than the cache keeps) must not release that table: the
    replay still packs the right parameters and the table keeps its address.
    A pointer set first seen during capture is refused (its upload would be
    a captured copy from host memory)."""
    say("graph: pinned pointer table")
    shapes, N = synth.llama_block_shapes(256, 688), 8
    plan = fs.fs_plan(shapes, "bf16", N, False, "fsdp2").upload()
    params, off = [], 0
    for s in shapes:
        n = int(np.prod(s))
        params.append(synth.normal_bf16(3, synth.STREAM_PARAMS, n, 0.02, device="cuda", start=off))
        off += n
    out = torch.empty(plan.gathered_numel, dtype=torch.bfloat16, device="cuda")
    fs.fs_pack(plan, params, out)            # eager call: makes the table
    torch.cuda.synchronize()
    ref = out.clone()
    addr = plan.ptr_table(params, "params").data_ptr()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fs.fs_pack(plan, params, out)
    scratch = torch.empty_like(out)
    for k in range(10):
        others = [p.clone() for p in params]
        fs.fs_pack(plan, others, scratch)
        del others
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    assert plan.ptr_table(params, "params").data_ptr() == addr
    del g
    fresh = [p.clone() for p in params]
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: True)
    with pytest.raises(RuntimeError, match="capture"):
        plan.ptr_table(fresh, "params")
