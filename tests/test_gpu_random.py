"""Randomized GPU parity: seeded random parameter lists (scalars, empty
tensors, 1- to 3-D shapes of awkward sizes), random N, dtype, mode and
use_orig_params, random 0..7-element misalignment of every buffer.  Pack
(all ranks and one rank), unpack and re-shard to another random plan must
equal the oracle bit for bit.  The reduce family (fp32 and bf16 reduce
dtype, fused reduce + AdamW) runs on random sizes, N, grad_acc and
per-slice misalignment: reduces bit-exact, fused bit-identical to the two
kernels, AdamW within its tolerance of the oracle.  Every buffer sits in a
canary guard band.  fp32 state at random bf16 plans' element positions (the
plans' fp32 twins) packs, unpacks and re-shards bit for bit as well, and the
cast pack and the state-dict import match the oracle on the same lists.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, bits, from_bits, say

pytestmark = pytest.mark.gpu

fs = pytest.importorskip("fsdp_sharded_state_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fs.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(1, 40))
    shapes = []
    for _ in range(n):
        kind = rng.integers(0, 10)
        if kind == 0:
            shapes.append(())
        elif kind == 1:
            shapes.append((0, int(rng.integers(1, 5))))
        elif kind < 5:
            shapes.append((int(rng.integers(1, 70000)),))
        elif kind < 8:
            shapes.append((int(rng.integers(1, 600)), int(rng.integers(1, 300))))
        else:
            shapes.append((int(rng.integers(1, 40)), int(rng.integers(1, 30)), int(rng.integers(1, 9))))
    dt = "bf16" if rng.random() < 0.6 else "fp32"
    mode = "fsdp1" if rng.random() < 0.5 else "fsdp2"
    N = int(rng.integers(1, 17))
    uo = bool(rng.random() < 0.5) and mode == "fsdp1"
    mode2 = "fsdp1" if rng.random() < 0.5 else "fsdp2"
    N2 = int(rng.integers(1, 17))
    uo2 = bool(rng.random() < 0.5) and mode2 == "fsdp1"
    shifts = [int(x) for x in rng.integers(0, 8, size=n + 3)]
    return shapes, dt, mode, N, uo, mode2, N2, uo2, shifts


def _olayout(mode, shapes, dt, N, uo):
    eb = 2 if dt == "bf16" else 4
    return oracle.fsdp1_layout(shapes, eb, N, uo) if mode == "fsdp1" else oracle.fsdp2_layout(shapes, eb, N)


@pytest.mark.parametrize("seed", range(16))
def test_random_layout_pack_unpack_reshard(seed):
    shapes, dt, mode, N, uo, mode2, N2, uo2, shifts = _random_case(seed)
    say("random layout", seed, mode, dt, N, uo, "->", mode2, N2, uo2, len(shapes), "params")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    plan = fs.fs_plan(shapes, dt, N, uo, mode).upload()
    L = _olayout(mode, shapes, dt, N, uo)
    params, off = [], 0
    gen = synth.bits16 if dt == "bf16" else synth.bits32
    for s, sh in zip(shapes, shifts):
        n = int(np.prod(s)) if len(s) else 1
        params.append(Guarded(n, tdt, shift=sh, fill=gen(seed, synth.STREAM_PARAMS, n, device="cuda",
                                                           start=off).view(tdt)))
        off += n
    host = [bits(p.t) for p in params]
    ref = oracle.pack(L, host)

    G = Guarded(plan.gathered_numel, tdt, shift=shifts[-1])
    fs.fs_pack(plan, [p.t for p in params], G.t)
    torch.cuda.synchronize()
    G.check()
    np.testing.assert_array_equal(bits(G.t), ref)

    r = int(seed % N)
    Sh = Guarded(plan.shard_numel, tdt, shift=shifts[-2])
    fs.fs_pack(plan, [p.t for p in params], Sh.t, rank=r)
    torch.cuda.synchronize()
    Sh.check()
    np.testing.assert_array_equal(bits(Sh.t), ref[r * plan.shard_numel:(r + 1) * plan.shard_numel])

    # unpack from a gathered buffer whose pads hold garbage
    junk = ref.copy()
    mask = np.ones(junk.size, bool)
    mask[L.index_map()] = False
    junk[mask] = 0x7FFF if dt == "bf16" else 0x7FFFFFFF
    src = Guarded(plan.gathered_numel, tdt, shift=shifts[-3], fill=from_bits(junk, tdt))
    outs = [Guarded(p.n, tdt, shift=sh) for p, sh in zip(params, reversed(shifts))]
    fs.fs_unpack(plan, src.t, [o.t for o in outs])
    torch.cuda.synchronize()
    for o, h in zip(outs, host):
        o.check()
        np.testing.assert_array_equal(bits(o.t), h)

    plan2 = fs.fs_plan(shapes, dt, N2, uo2, mode2).upload()
    L2 = _olayout(mode2, shapes, dt, N2, uo2)
    D = Guarded(plan2.gathered_numel, tdt, shift=shifts[0])
    rs = fs.fs_reshard_plan(plan, plan2).upload()
    fs.fs_reshard(rs, src.t, D.t)
    torch.cuda.synchronize()
    D.check()
    src.check()
    np.testing.assert_array_equal(bits(D.t), oracle.reshard(L, L2, junk))


@pytest.mark.parametrize("seed", range(12))
def test_random_cast_pack_and_import(seed):
    """On the same random parameter lists (bf16 plans): the fp32 -> bf16 cast
    pack of misaligned fp32 parameters, all ranks and one rank, and the
    state-dict import of one rank from its local pieces held as separate
    misaligned tensors, against the oracle bit for bit."""
    shapes, _, mode, N, uo, _, _, _, shifts = _random_case(seed)
    say("random cast pack / import", seed, mode, N, uo, len(shapes), "params")
    plan = fs.fs_plan(shapes, "bf16", N, uo, mode).upload()
    L = _olayout(mode, shapes, "bf16", N, uo)
    p32, p16, off = [], [], 0
    for s, sh in zip(shapes, shifts):
        n = int(np.prod(s)) if len(s) else 1
        vals = synth.normal_f32(seed, synth.STREAM_MASTER, n, 0.02, device="cuda", start=off)
        if n >= 4:   # a NaN, an infinity, a bf16 tie and a denormal among the values
            vals[:4] = torch.tensor([float("nan"), -float("inf"), 1.0 + 2.0 ** -8, 1e-40], device="cuda")
        p32.append(Guarded(n, torch.float32, shift=sh, fill=vals))
        p16.append(Guarded(n, torch.bfloat16, shift=7 - sh,
                           fill=synth.bits16(seed, synth.STREAM_PARAMS, n, device="cuda", start=off).view(torch.bfloat16)))
        off += n
    ref_cast = oracle.pack_cast(L, [p.t.cpu().numpy() for p in p32])
    G = Guarded(plan.gathered_numel, torch.bfloat16, shift=shifts[-1])
    fs.fs_pack_cast(plan, [p.t for p in p32], G.t)
    r = int(seed % N)
    c = plan.shard_numel
    S = Guarded(c, torch.bfloat16, shift=shifts[-2])
    fs.fs_pack_cast(plan, [p.t for p in p32], S.t, rank=r)
    # import rank r's pieces of the bf16 parameters, each a separate misaligned tensor
    host16 = [bits(p.t) for p in p16]
    ref = oracle.pack(L, host16, rank=r)
    pieces = []
    for k, (pc, h) in enumerate(zip(plan.local_pieces(r), host16)):
        lo, cnt = (pc[1], pc[2]) if pc else (0, 0)
        pieces.append(Guarded(cnt, torch.bfloat16, shift=shifts[k % len(shifts)],
                              fill=from_bits(h[lo:lo + cnt], torch.bfloat16) if cnt else None))
    I = Guarded(c, torch.bfloat16, shift=shifts[-3], fill=torch.full((c,), -1, dtype=torch.int16).view(torch.bfloat16))
    plan.load_local(I.t, r, [q.t for q in pieces])
    torch.cuda.synchronize()
    for g in [G, S, I] + p32 + p16 + pieces:
        g.check()
    np.testing.assert_array_equal(bits(G.t), ref_cast)
    np.testing.assert_array_equal(bits(S.t), ref_cast[r * c:(r + 1) * c])
    np.testing.assert_array_equal(bits(I.t), ref)


@pytest.mark.parametrize("seed", range(8))
def test_random_twin_state(seed):
    """fp32 state at a bf16 plan's element positions (fs_plan_twin): pack,
    unpack and re-shard to another random plan's twin, against the oracle's
    bf16 layouts carrying 4-byte elements, with random misalignment."""
    shapes, _, mode, N, uo, mode2, N2, uo2, shifts = _random_case(100 + seed)
    if mode == "fsdp1":
        uo = True        # the case the twin is for: alignment by the bf16 parameter dtype
    say("random twin", seed, mode, N, uo, "->", mode2, N2, uo2, len(shapes), "params")
    T = fs.fs_plan(shapes, "bf16", N, uo, mode).twin("fp32").upload()
    T2 = fs.fs_plan(shapes, "bf16", N2, uo2, mode2).twin("fp32").upload()
    L = _olayout(mode, shapes, "bf16", N, uo).with_elem_bytes(4)
    L2 = _olayout(mode2, shapes, "bf16", N2, uo2).with_elem_bytes(4)
    params, off = [], 0
    for s, sh in zip(shapes, shifts):
        n = int(np.prod(s)) if len(s) else 1
        params.append(Guarded(n, torch.float32, shift=sh,
                              fill=synth.bits32(seed, synth.STREAM_MASTER, n, device="cuda", start=off).view(torch.float32)))
        off += n
    host = [bits(p.t) for p in params]
    ref = oracle.pack(L, host)
    G = Guarded(T.gathered_numel, torch.float32, shift=shifts[-1])
    fs.fs_pack(T, [p.t for p in params], G.t)
    torch.cuda.synchronize()
    G.check()
    np.testing.assert_array_equal(bits(G.t), ref)
    junk = ref.copy()
    mask = np.ones(junk.size, bool)
    mask[L.index_map()] = False
    junk[mask] = 0x7FFFFFFF
    src = Guarded(T.gathered_numel, torch.float32, shift=shifts[-3], fill=from_bits(junk, torch.float32))
    outs = [Guarded(p.n, torch.float32, shift=sh) for p, sh in zip(params, reversed(shifts))]
    fs.fs_unpack(T, src.t, [o.t for o in outs])
    D = Guarded(T2.gathered_numel, torch.float32, shift=shifts[0])
    fs.fs_reshard(fs.fs_reshard_plan(T, T2).upload(), src.t, D.t)
    torch.cuda.synchronize()
    for o, h in zip(outs, host):
        o.check()
        np.testing.assert_array_equal(bits(o.t), h)
    D.check()
    np.testing.assert_array_equal(bits(D.t), oracle.reshard(L, L2, junk))


def _random_reduce_case(seed):
    rng = np.random.default_rng(2000 + seed)
    n = int(rng.integers(1, 200000))
    N = int(rng.integers(1, 17))
    A = int(rng.integers(1, 6))
    if rng.random() < 0.5:
        shifts = [0] * (N * A)
        osh = 0
    else:
        shifts = [int(x) for x in rng.integers(0, 8, size=N * A)]
        osh = int(rng.integers(0, 4))
    return n, N, A, shifts, osh


@pytest.mark.parametrize("seed", range(12))
def test_random_reduce_family(seed):
    """fs_reduce_shard, the bf16 reduce dtype and the fused reduce + AdamW on
    random sizes, world sizes, micro-step counts (up to 80 terms: several
    passes) and per-slice misalignment."""
    n, N, A, shifts, osh = _random_reduce_case(seed)
    say("random reduce family", seed, n, N, A, shifts[:4], osh)
    sl = [Guarded(n, torch.bfloat16, shift=sh,
                  fill=synth.normal_bf16(seed, synth.stream_grad(t // N, t % N, N), n, 1e-3, device="cuda"))
          for t, sh in enumerate(shifts)]
    host = [bits(s.t) for s in sl]
    out = Guarded(n, torch.float32, shift=osh)
    fs.fs_reduce_shard([s.t for s in sl], out.t, N, A)
    rs = Guarded(n, torch.float32, shift=osh)
    fs.fs_reduce_shard_ex([s.t for s in sl], rs.t, N, A, reduce_dtype="bf16")
    th = synth.normal_f32(seed, synth.STREAM_MASTER, n, 0.02, device="cuda")
    m = synth.normal_f32(seed, synth.STREAM_EXP_AVG, n, 1e-3, device="cuda")
    v = synth.normal_f32(seed, synth.STREAM_EXP_AVG_SQ, n, 1e-3, device="cuda") ** 2
    two = [Guarded(n, torch.float32, shift=osh, fill=x) for x in (th, m, v)]
    fused = [Guarded(n, torch.float32, shift=osh, fill=x) for x in (th, m, v)]
    p_two, p_fused = Guarded(n, torch.bfloat16, shift=osh), Guarded(n, torch.bfloat16, shift=osh)
    g_fused = Guarded(n, torch.float32, shift=osh)
    fs.fs_adamw_step(*[x.t for x in two], out.t, p_two.t, step=seed + 1)
    fs.fs_reduce_adamw_step([s.t for s in sl], *[x.t for x in fused], p_fused.t, g_fused.t, world=N,
                            grad_acc=A, step=seed + 1)
    torch.cuda.synchronize()
    for g in [out, rs, p_two, p_fused, g_fused] + two + fused + sl:
        g.check()
    ref = oracle.reduce_shard(host, N, A)
    np.testing.assert_array_equal(bits(out.t), ref.view(np.uint32))
    np.testing.assert_array_equal(bits(g_fused.t), ref.view(np.uint32))
    np.testing.assert_array_equal(bits(rs.t), oracle.reduce_shard_bf16rs(host, N, A).view(np.uint32))
    for a, b in zip(two + [p_two], fused + [p_fused]):
        np.testing.assert_array_equal(bits(a.t), bits(b.t))
    rt, rm, rv, rp = oracle.adamw_step(th.cpu().numpy(), m.cpu().numpy(), v.cpu().numpy(), ref,
                                       oracle.AdamWHparams(step=seed + 1))
    gt, gm, gv = (x.t.cpu().numpy() for x in two)
    assert np.all(np.abs(gt - rt) <= 1e-6 * np.maximum(np.abs(rt), np.abs(th.cpu().numpy())))
    assert np.all(np.abs(gm - rm) <= 1e-6 * np.abs(rm))
    assert np.all(np.abs(gv - rv) <= 1e-6 * np.abs(rv))
    assert np.all(np.abs(bits(p_two.t).astype(np.int32) - rp.astype(np.int32)) <= 1)


@pytest.mark.parametrize("mode,dt,uo", [("fsdp1", "bf16", True), ("fsdp1", "fp32", False), ("fsdp2", "bf16", False)])
def test_many_tiny_parameters(mode, dt, uo):
    """20,000 parameters of 1-40 elements (tens of segments per 16-byte block
    range, so tiles are cut at the LDS segment cap): pack, unpack and re-shard
    to N = 3 bit-exact."""
    rng = np.random.default_rng(77)
    shapes = [(int(x),) for x in rng.integers(1, 41, size=20000)]
    if mode == "fsdp2":
        shapes = [(int(x), 2) for x in rng.integers(1, 21, size=20000)]
    N = 8
    say("many tiny parameters", mode, dt, uo)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    plan = fs.fs_plan(shapes, dt, N, uo, mode).upload()
    L = _olayout(mode, shapes, dt, N, uo)
    gen = synth.bits16 if dt == "bf16" else synth.bits32
    total = int(L.numel.sum())
    flat = gen(5, synth.STREAM_PARAMS, total, device="cuda").view(tdt)
    offs = np.concatenate([[0], np.cumsum(L.numel)]).astype(np.int64)
    params = [flat[offs[i]:offs[i + 1]] for i in range(len(shapes))]
    host_flat = bits(flat)
    host = [host_flat[offs[i]:offs[i + 1]] for i in range(len(shapes))]
    ref = oracle.pack(L, host)
    G = Guarded(plan.gathered_numel, tdt)
    fs.fs_pack(plan, params, G.t)
    torch.cuda.synchronize()
    G.check()
    np.testing.assert_array_equal(bits(G.t), ref)
    out_flat = torch.empty(total, dtype=tdt, device="cuda")
    outs = [out_flat[offs[i]:offs[i + 1]] for i in range(len(shapes))]
    fs.fs_unpack(plan, G.t, outs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out_flat), host_flat)
    plan3 = fs.fs_plan(shapes, dt, 3, uo, mode).upload()
    D = Guarded(plan3.gathered_numel, tdt)
    fs.fs_reshard(fs.fs_reshard_plan(plan, plan3).upload(), G.t, D.t)
    torch.cuda.synchronize()
    D.check()
    np.testing.assert_array_equal(bits(D.t), oracle.reshard(L, _olayout(mode, shapes, dt, 3, uo), ref))
