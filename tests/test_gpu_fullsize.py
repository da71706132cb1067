"""GPU parity at full size: the 7B model's rank-0 FSDP2 shard (N = 8,
grad_acc = 4, S = 842,301,440), in the launch configuration the benchmark
times (one fs_reduce_shard over 32 separate bf16 slices, one fs_adamw_step
with an fp32 gradient and a bf16 copy, fs_pack with rank -1 and fs_unpack
per group), plus the bf16 reduce dtype and the fused reduce + AdamW over the
same slices, and per group the re-shard, the cast pack and the state-dict
import; at these sizes the reduce, AdamW, unpack, re-shard and cast pack
launches cap their resident workgroups.

The oracle cannot run the whole shard here, so it computes sampled outputs
one by one from inputs it regenerates itself (synth is counter-based: element
i of every buffer is a function of (seed, stream, i)), and the sampled GPU
outputs must match: bit-exact for the reduce, pack and unpack, within
tolerance for AdamW.  Samples: random indices, both ends, and every 2^k
boundary.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import bits, say

pytestmark = pytest.mark.gpu
fs = pytest.importorskip("fsdp_sharded_state_amd")

SEED = 4
N, A = 8, 4


@pytest.fixture(scope="module")
def plans():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    groups = synth.llama_model_groups(32, 4096, 11008)
    ps = [fs.fs_plan(g, "bf16", N, False, "fsdp2", A).upload() for g in groups]
    yield groups, ps
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _sample(n, k, rng):
    idx = set(rng.integers(0, n, size=k).tolist())
    idx.update(range(0, min(n, 64)))
    idx.update(range(max(0, n - 64), n))
    p = 1
    while p < n:
        idx.update(x for x in (p - 1, p) if x < n)
        p *= 2
    return np.array(sorted(idx), np.int64)


def test_fullsize_reduce_and_adamw(plans):
    groups, ps = plans
    S = sum(p.shard_numel for p in ps)
    assert S == 842_301_440
    say("full-size reduce: generating 32 slices of", S)
    slices = [synth.normal_bf16(SEED, synth.stream_grad(j, k, N), S, 1e-3, device="cuda")
              for j in range(A) for k in range(N)]
    g32 = torch.empty(S, dtype=torch.float32, device="cuda")
    say("full-size reduce: launch")
    fs.fs_reduce_shard(slices, g32, N, A)
    # the bf16 reduce dtype over the same slices (its launches cap residency at this size)
    g_rs = torch.empty(S, dtype=torch.float32, device="cuda")
    say("full-size bf16 reduce dtype: launch")
    fs.fs_reduce_shard_ex(slices, g_rs, N, A, reduce_dtype="bf16")
    master = synth.normal_f32(SEED, synth.STREAM_MASTER, S, 0.02, device="cuda")
    m = torch.zeros(S, device="cuda")
    v = torch.zeros(S, device="cuda")
    p16 = torch.empty(S, dtype=torch.bfloat16, device="cuda")
    # the fused step from the same state: bit-identical to the two kernels below
    fmaster, fm, fv = master.clone(), torch.zeros(S, device="cuda"), torch.zeros(S, device="cuda")
    fp16 = torch.empty(S, dtype=torch.bfloat16, device="cuda")
    say("full-size fused reduce + AdamW: launch")
    fs.fs_reduce_adamw_step(slices, fmaster, fm, fv, fp16, None, world=N, grad_acc=A, lr=1e-3, beta1=0.9,
                            beta2=0.999, eps=1e-8, weight_decay=0.01, step=1)
    del slices
    say("full-size AdamW: launch")
    fs.fs_adamw_step(master, m, v, g32, p16, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                     weight_decay=0.01, step=1)
    torch.cuda.synchronize()

    rng = np.random.default_rng(11)
    idx = _sample(S, 300_000, rng)
    it = torch.from_numpy(idx)
    sl_host = [synth.to_numpy_bits(synth.normal_bf16_at(SEED, synth.stream_grad(j, k, N), it, 1e-3))
               for j in range(A) for k in range(N)]
    ref_g = oracle.reduce_shard(sl_host, N, A)
    it_dev = it.cuda()
    got_g = g32[it_dev].cpu().numpy()
    np.testing.assert_array_equal(got_g.view(np.uint32), ref_g.view(np.uint32))
    ref_rs = oracle.reduce_shard_bf16rs(sl_host, N, A)
    np.testing.assert_array_equal(g_rs[it_dev].cpu().numpy().view(np.uint32), ref_rs.view(np.uint32))
    del g_rs

    th0 = synth.normal_f32_at(SEED, synth.STREAM_MASTER, it, 0.02).numpy()
    z = np.zeros(idx.size, np.float32)
    rt, rm, rv, rp = oracle.adamw_step(th0, z, z, ref_g, oracle.AdamWHparams(step=1))
    gt = master[it_dev].cpu().numpy()
    gm = m[it_dev].cpu().numpy()
    gv = v[it_dev].cpu().numpy()
    gp = bits(p16[it_dev]).astype(np.int32)
    assert np.all(np.abs(gt - rt) <= 1e-6 * np.maximum(np.abs(rt), np.abs(th0)))
    assert np.all(np.abs(gm - rm) <= 1e-6 * np.abs(rm))
    assert np.all(np.abs(gv - rv) <= 1e-6 * np.abs(rv))
    assert np.all(np.abs(gp - rp.astype(np.int32)) <= 1)
    inexact = np.mean((gt.view(np.uint32) != rt.view(np.uint32)) | (gm.view(np.uint32) != rm.view(np.uint32)) |
                      (gv.view(np.uint32) != rv.view(np.uint32)))
    assert inexact <= 1e-6, inexact
    for a, b in ((fmaster, master), (fm, m), (fv, v)):
        np.testing.assert_array_equal(a[it_dev].cpu().numpy().view(np.uint32), b[it_dev].cpu().numpy().view(np.uint32))
    np.testing.assert_array_equal(bits(fp16[it_dev]), bits(p16[it_dev]))


@pytest.mark.parametrize("which", ["block0", "block31", "root"])
def test_fullsize_pack_unpack_groups(plans, which):
    """Pack (all ranks), unpack and re-shard (N -> N/2) of a full-size group;
    sampled elements of the gathered buffers and of the unpacked parameters
    against the oracle's layouts, and every pad element zero.  Also the
    fp32 -> bf16 cast pack of fp32 parameters (sampled, against the oracle's
    rounding of the regenerated values) and the state-dict import of ranks 0
    and N-1 from their local pieces of the parameters (whole shard, equal to
    that rank's shard of the packed buffer)."""
    groups, ps = plans
    gi = {"block0": 0, "block31": 31, "root": 32}[which]
    shapes, plan = groups[gi], ps[gi]
    off = sum(math.prod(s) for g in groups[:gi] for s in g)   # element offset of the group's parameters
    say("full-size pack/unpack", which)
    params, starts = [], []
    o = off
    for s in shapes:
        n = math.prod(s)
        params.append(synth.bits16(SEED, synth.STREAM_PARAMS, n, device="cuda", start=o).view(torch.bfloat16))
        starts.append(o)
        o += n
    gathered = torch.empty(plan.gathered_numel, dtype=torch.bfloat16, device="cuda")
    fs.fs_pack(plan, params, gathered)
    outs = [torch.empty_like(p) for p in params]
    fs.fs_unpack(plan, gathered, outs)
    # re-shard the gathered buffer from N to N/2 logical ranks
    half = fs.fs_plan(shapes, "bf16", N // 2, False, "fsdp2", A).upload()
    rs = fs.fs_reshard_plan(plan, half).upload()
    regathered = torch.empty(half.gathered_numel, dtype=torch.bfloat16, device="cuda")
    fs.fs_reshard(rs, gathered, regathered)
    # cast pack of fp32 parameters, all ranks
    p32 = [synth.normal_f32(SEED, synth.STREAM_MASTER, math.prod(s), 0.02, device="cuda", start=st)
           for s, st in zip(shapes, starts)]
    gcast = torch.empty(plan.gathered_numel, dtype=torch.bfloat16, device="cuda")
    fs.fs_pack_cast(plan, p32, gcast)
    # state-dict import: each rank's local pieces of the parameters into a fresh shard
    imported = {}
    for r in (0, N - 1):
        pieces = [params[i].view(-1)[pc[1]:pc[1] + pc[2]] if pc else params[i].view(-1)[:0]
                  for i, pc in enumerate(plan.local_pieces(r))]
        imported[r] = torch.full((plan.shard_numel,), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        plan.load_local(imported[r], r, pieces)
    torch.cuda.synchronize()
    for r, sh in imported.items():
        c = plan.shard_numel
        assert torch.equal(sh.view(torch.int16), gathered.view(torch.int16)[r * c:(r + 1) * c])
    del p32, imported

    L = oracle.fsdp2_layout(shapes, 2, N)
    Lh = oracle.fsdp2_layout(shapes, 2, N // 2)
    rng = np.random.default_rng(gi)
    for i, (s, st) in enumerate(zip(shapes, starts)):
        n = math.prod(s)
        e = _sample(n, 20_000, rng)
        x = L.index_at(np.full(e.size, i, np.int32), e)
        expect = synth.to_numpy_bits(synth.bits16_at(SEED, synth.STREAM_PARAMS, torch.from_numpy(e + st)))
        got = bits(gathered.view(torch.int16)[torch.from_numpy(x).cuda()])
        np.testing.assert_array_equal(got, expect)
        xh = Lh.index_at(np.full(e.size, i, np.int32), e)
        np.testing.assert_array_equal(bits(regathered.view(torch.int16)[torch.from_numpy(xh).cuda()]), expect)
        x32 = synth.normal_f32_at(SEED, synth.STREAM_MASTER, torch.from_numpy(e + st), 0.02).numpy()
        np.testing.assert_array_equal(bits(gcast.view(torch.int16)[torch.from_numpy(x).cuda()]), oracle.bf16_round(x32))
        got_u = bits(outs[i].view(-1).view(torch.int16)[torch.from_numpy(e).cuda()])
        np.testing.assert_array_equal(got_u, expect)
        assert torch.equal(outs[i].view(torch.int16), params[i].view(torch.int16))
    # every dim 0 of this model is divisible by 8: no pads, the gathered
    # buffer is all data, and the round trip above covers every element
    assert plan.tail_pad == 0


# ---------------------------------------------------------------- 70B --
#
# The 70B Llama-style model (80 blocks, d 8192, f 28672, k/v 8192x1024, vocab
# 32000): rank 0's FSDP2 shard holds S = 8,622,080,000 elements, so its fp32
# master, moments and gradient plus the bf16 copy take 155 GB of HBM.  AdamW
# runs over the whole shard; the reduce (grad_acc = 2) and pack/unpack run
# per group, as FSDP issues one reduce-scatter and one all-gather per group,
# on the first block, the last block and the root group.

N70, A70 = 8, 2


@pytest.fixture(scope="module")
def plans70():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.empty_cache()
    groups = synth.llama_model_groups(80, 8192, 28672, kv=1024)
    ps = [fs.fs_plan(g, "bf16", N70, False, "fsdp2", A70).upload() for g in groups]
    yield groups, ps
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_fullsize_70b_adamw_over_whole_shard(plans70):
    groups, ps = plans70
    S = sum(p.shard_numel for p in ps)
    assert S == 8_622_080_000
    say("70B AdamW: generating state for", S)
    master = synth.normal_f32(SEED, synth.STREAM_MASTER, S, 0.02, device="cuda")
    m = synth.normal_f32(SEED, synth.STREAM_EXP_AVG, S, 1e-3, device="cuda")
    v = torch.zeros(S, dtype=torch.float32, device="cuda")
    g32 = synth.normal_f32(SEED, 100, S, 1e-3, device="cuda")
    p16 = torch.empty(S, dtype=torch.bfloat16, device="cuda")
    say("70B AdamW: launch")
    fs.fs_adamw_step(master, m, v, g32, p16, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                     weight_decay=0.01, step=7)
    torch.cuda.synchronize()
    idx = _sample(S, 300_000, np.random.default_rng(70))
    it = torch.from_numpy(idx)
    th0 = synth.normal_f32_at(SEED, synth.STREAM_MASTER, it, 0.02).numpy()
    m0 = synth.normal_f32_at(SEED, synth.STREAM_EXP_AVG, it, 1e-3).numpy()
    g0 = synth.normal_f32_at(SEED, 100, it, 1e-3).numpy()
    rt, rm, rv, rp = oracle.adamw_step(th0, m0, np.zeros_like(m0), g0, oracle.AdamWHparams(step=7))
    itd = it.cuda()
    gt, gm, gv = (x[itd].cpu().numpy() for x in (master, m, v))
    assert np.all(np.abs(gt - rt) <= 1e-6 * np.maximum(np.abs(rt), np.abs(th0)))
    assert np.all(np.abs(gm - rm) <= 1e-6 * np.abs(rm))
    assert np.all(np.abs(gv - rv) <= 1e-6 * np.abs(rv))
    assert np.all(np.abs(bits(p16[itd]).astype(np.int32) - rp.astype(np.int32)) <= 1)
    del master, m, v, g32, p16
    torch.cuda.empty_cache()


@pytest.mark.parametrize("which", ["block0", "block79", "root"])
def test_fullsize_70b_group_reduce_pack_unpack(plans70, which):
    groups, ps = plans70
    gi = {"block0": 0, "block79": 79, "root": 80}[which]
    shapes, plan = groups[gi], ps[gi]
    shard_off = sum(p.shard_numel for p in ps[:gi])
    n = plan.shard_numel
    say("70B group reduce", which, n)
    slices = [synth.normal_bf16(SEED, synth.stream_grad(j, k, N70), n, 1e-3, device="cuda", start=shard_off)
              for j in range(A70) for k in range(N70)]
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    fs.fs_reduce_shard(slices, out, N70, A70)
    out_rs = torch.empty(n, dtype=torch.float32, device="cuda")
    fs.fs_reduce_shard_ex(slices, out_rs, N70, A70, reduce_dtype="bf16")
    torch.cuda.synchronize()
    del slices
    idx = _sample(n, 100_000, np.random.default_rng(gi))
    it = torch.from_numpy(idx)
    sl_host = [synth.to_numpy_bits(synth.normal_bf16_at(SEED, synth.stream_grad(j, k, N70), it + shard_off, 1e-3))
               for j in range(A70) for k in range(N70)]
    ref = oracle.reduce_shard(sl_host, N70, A70)
    np.testing.assert_array_equal(out[it.cuda()].cpu().numpy().view(np.uint32), ref.view(np.uint32))
    ref_rs = oracle.reduce_shard_bf16rs(sl_host, N70, A70)
    np.testing.assert_array_equal(out_rs[it.cuda()].cpu().numpy().view(np.uint32), ref_rs.view(np.uint32))
    del out, out_rs

    say("70B group pack/unpack", which)
    off = sum(math.prod(s) for g in groups[:gi] for s in g)
    params, starts, o = [], [], off
    for s in shapes:
        k = math.prod(s)
        params.append(synth.bits16(SEED, synth.STREAM_PARAMS, k, device="cuda", start=o).view(torch.bfloat16))
        starts.append(o)
        o += k
    gathered = torch.empty(plan.gathered_numel, dtype=torch.bfloat16, device="cuda")
    fs.fs_pack(plan, params, gathered)
    outs = [torch.empty_like(p) for p in params]
    fs.fs_unpack(plan, gathered, outs)
    torch.cuda.synchronize()
    L = oracle.fsdp2_layout(shapes, 2, N70)
    rng = np.random.default_rng(gi + 1)
    for i, (s, st) in enumerate(zip(shapes, starts)):
        e = _sample(math.prod(s), 20_000, rng)
        x = L.index_at(np.full(e.size, i, np.int32), e)
        expect = synth.to_numpy_bits(synth.bits16_at(SEED, synth.STREAM_PARAMS, torch.from_numpy(e + st)))
        np.testing.assert_array_equal(bits(gathered.view(torch.int16)[torch.from_numpy(x).cuda()]), expect)
        assert torch.equal(outs[i].view(torch.int16), params[i].view(torch.int16))
    del params, outs, gathered
    torch.cuda.empty_cache()
