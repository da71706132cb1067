"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: bit-exact for pack, unpack and the reduce (fixed summation order);
AdamW within 1e-6 relative on fp32 theta/m/v (|d| <= 1e-6 * max(|ref|, |in|)
for theta, whose value can cross zero) and 1 bf16 ulp on the parameter copy.
Every output sits in a canary guard band.  Inputs come from the seeded
counter-based generator (synth.py), never from the HIP path.
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


def test_synth_same_bits_on_gpu_and_cpu():
    idx = torch.tensor([0, 1, 2, 3, 1000, 2 ** 31 + 5, 2 ** 33 + 7, 6_738_411_519], dtype=torch.int64)
    for fn in (lambda i: synth.bits16_at(5, 1, i), lambda i: synth.bits32_at(5, 2, i),
               lambda i: synth.normal_f32_at(4, 101, i, 1e-3), lambda i: synth.normal_bf16_at(4, 1, i, 0.02)):
        a = fn(idx)
        b = fn(idx.cuda()).cpu()
        assert torch.equal(a.view(torch.int16) if a.element_size() == 2 else a.view(torch.int32),
                           b.view(torch.int16) if b.element_size() == 2 else b.view(torch.int32))


# ------------------------------------------------------------ pack/unpack --

def _layout_cases():
    cases = [
        ("mlp_tiny", "fsdp1", synth.mlp_tiny_shapes(), "bf16", 4, True),
        ("mlp_tiny_fsdp2", "fsdp2", synth.mlp_tiny_shapes(), "bf16", 4, False),
        ("worked_example_f1T", "fsdp1", [(3,), (5,)], "bf16", 4, True),
        ("worked_example_f1F", "fsdp1", [(3,), (5,)], "bf16", 4, False),
        ("worked_example_f2", "fsdp2", [(3,), (5,)], "bf16", 4, False),
        ("tiny_mixed_f2_fp32", "fsdp2", [(6, 3), (), (0, 2), (9,), (1, 1), (13, 5)], "fp32", 4, False),
        ("tiny_mixed_f1F_fp32", "fsdp1", [(1,), (7,), (0,), (3, 3), (2,), (17,)], "fp32", 3, False),
        ("tiny_mixed_f1T", "fsdp1", [(1,), (7,), (0,), (3, 3), (2,), (17,)], "bf16", 5, True),
        ("single_N1", "fsdp1", [(100003,)], "bf16", 1, True),
        ("many_tiles_ragged", "fsdp2", [(1000, 37), (999,), (31, 3)], "bf16", 7, False),
        ("many_segments_per_tile", "fsdp1", [(k % 5 + 1,) for k in range(700)], "bf16", 8, False),
        ("many_segments_fsdp2", "fsdp2", [(k % 9 + 1, 2) for k in range(400)], "fp32", 8, False),
    ]
    st = [(n,) for n in synth.padding_stress_numels()]
    for dt in ("bf16", "fp32"):
        for uo in (True, False):
            cases.append((f"padding_stress_{dt}_{'T' if uo else 'F'}", "fsdp1", st, dt, 8, uo))
    cases.append(("llama_block_fsdp2", "fsdp2", synth.llama_block_shapes(), "bf16", 8, False))
    return cases


def _olayout(mode, shapes, dt, N, uo):
    eb = 2 if dt == "bf16" else 4
    return oracle.fsdp1_layout(shapes, eb, N, uo) if mode == "fsdp1" else oracle.fsdp2_layout(shapes, eb, N)


def _params(shapes, dt, seed, shift=0):
    """Uniform random bit patterns (NaN payloads included) per parameter."""
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out = []
    off = 0
    for s in shapes:
        n = int(np.prod(s)) if len(s) else 1
        g = synth.bits16 if dt == "bf16" else synth.bits32
        vals = g(seed, synth.STREAM_PARAMS, n, device="cuda", start=off).view(tdt)
        out.append(Guarded(n, tdt, shift=shift, fill=vals))
        off += n
    return out


@pytest.mark.parametrize("case", _layout_cases(), ids=lambda c: c[0])
def test_pack_unpack_bitexact(case):
    name, mode, shapes, dt, N, uo = case
    say("pack/unpack", name)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    plan = fs.fs_plan(shapes, dt, N, uo, mode).upload()
    L = _olayout(mode, shapes, dt, N, uo)
    params = _params(shapes, dt, seed=17)
    host = [bits(p.t) for p in params]
    ref = oracle.pack(L, host)

    G = Guarded(plan.gathered_numel, tdt)
    fs.fs_pack(plan, [p.t for p in params], G.t)
    torch.cuda.synchronize()
    G.check()
    np.testing.assert_array_equal(bits(G.t), ref)

    for r in sorted({0, N // 2, N - 1}):
        say("pack rank", name, r)
        S = Guarded(plan.shard_numel, tdt)
        fs.fs_pack(plan, [p.t for p in params], S.t, rank=r)
        torch.cuda.synchronize()
        S.check()
        np.testing.assert_array_equal(bits(S.t), ref[r * plan.shard_numel:(r + 1) * plan.shard_numel])

    # unpack from a gathered buffer whose pads hold garbage: pads are never read
    junk = ref.copy()
    idx = L.index_map()
    mask = np.ones(junk.size, bool)
    mask[idx] = False
    junk[mask] = 0x7FFF if dt == "bf16" else 0x7FFFFFFF
    say("unpack", name)
    src = from_bits(junk, tdt)
    outs = [Guarded(p.n, tdt) for p in params]
    fs.fs_unpack(plan, src, [o.t for o in outs])
    torch.cuda.synchronize()
    for o, h in zip(outs, host):
        o.check()
        np.testing.assert_array_equal(bits(o.t), h)


@pytest.mark.parametrize("case", [c for c in _layout_cases() if c[0] in (
    "mlp_tiny", "worked_example_f1F", "tiny_mixed_f2_fp32", "tiny_mixed_f1T", "many_tiles_ragged",
    "padding_stress_bf16_F", "many_segments_per_tile")], ids=lambda c: c[0])
@pytest.mark.parametrize("shift", [1, 3])
def test_pack_unpack_misaligned_buffers(case, shift):
    """Parameters and outputs that start off their 16-byte boundary take the
    realigning (funnel shift / shuffle) and per-element paths."""
    name, mode, shapes, dt, N, uo = case
    say("misaligned pack/unpack", name, shift)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    plan = fs.fs_plan(shapes, dt, N, uo, mode).upload()
    L = _olayout(mode, shapes, dt, N, uo)
    params = _params(shapes, dt, seed=29, shift=shift)
    host = [bits(p.t) for p in params]
    ref = oracle.pack(L, host)
    G = Guarded(plan.gathered_numel, tdt)
    fs.fs_pack(plan, [p.t for p in params], G.t)
    r = N - 1
    S = Guarded(plan.shard_numel, tdt, shift=shift)
    fs.fs_pack(plan, [p.t for p in params], S.t, rank=r)
    src = Guarded(plan.gathered_numel, tdt, shift=shift, fill=from_bits(ref, tdt))
    outs = [Guarded(p.n, tdt, shift=(shift + i) % 5) for i, p in enumerate(params)]
    fs.fs_unpack(plan, src.t, [o.t for o in outs])
    torch.cuda.synchronize()
    for g in (G, S, *outs):
        g.check()
    np.testing.assert_array_equal(bits(G.t), ref)
    np.testing.assert_array_equal(bits(S.t), ref[r * plan.shard_numel:(r + 1) * plan.shard_numel])
    for o, h in zip(outs, host):
        np.testing.assert_array_equal(bits(o.t), h)


@pytest.mark.parametrize("case", [c for c in _layout_cases() if c[0] in (
    "many_tiles_ragged", "padding_stress_bf16_F", "padding_stress_fp32_T", "llama_block_fsdp2")],
    ids=lambda c: c[0])
def test_unpack_aligned_source_misaligned_outputs(case):
    """A 16-byte-aligned gathered buffer with outputs off their 16-byte
    boundary: single-run tiles issue their aligned loads, find the
    destination misaligned, and finish on the segment path."""
    name, mode, shapes, dt, N, uo = case
    say("unpack: aligned source, misaligned outputs", name)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    plan = fs.fs_plan(shapes, dt, N, uo, mode).upload()
    L = _olayout(mode, shapes, dt, N, uo)
    params = _params(shapes, dt, seed=43)
    host = [bits(p.t) for p in params]
    src = Guarded(plan.gathered_numel, tdt, fill=from_bits(oracle.pack(L, host), tdt))
    outs = [Guarded(p.n, tdt, shift=1 + i % 3) for i, p in enumerate(params)]
    fs.fs_unpack(plan, src.t, [o.t for o in outs])
    torch.cuda.synchronize()
    for o, h in zip(outs, host):
        o.check()
        np.testing.assert_array_equal(bits(o.t), h)


def test_pack_empty_and_degenerate():
    say("pack empty/degenerate")
    p = fs.fs_plan([(0,), (0, 4)], "bf16", 4, False, "fsdp2").upload()
    e = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    fs.fs_pack(p, [torch.empty(0, dtype=torch.bfloat16, device="cuda")] * 2, e)
    fs.fs_unpack(p, e, [torch.empty(0, dtype=torch.bfloat16, device="cuda")] * 2)
    # all ranks past the data are pure pads
    p = fs.fs_plan([(3,)], "bf16", 8, False, "fsdp1").upload()
    x = Guarded(3, torch.bfloat16, fill=torch.tensor([1.0, 2.0, 3.0], dtype=torch.bfloat16, device="cuda"))
    for r in range(8):
        S = Guarded(1, torch.bfloat16)
        fs.fs_pack(p, [x.t], S.t, rank=r)
        torch.cuda.synchronize()
        S.check()
        assert S.t.item() == (float(r + 1) if r < 3 else 0.0)


# ----------------------------------------------------------------- reduce --

def _slices(n, terms, seed, shift=0, sigma=1e-3, specials=False):
    out = []
    for t in range(terms):
        vals = synth.normal_bf16(seed, 100 + t, n, sigma, device="cuda")
        if specials and n >= 16:
            sp = torch.tensor([float("nan"), float("inf"), -float("inf"), -0.0, 0.0, 1e-40, -1e-39,
                               3e38, -3e38, 2.0 ** 24, 1.0, -1.0], dtype=torch.bfloat16, device="cuda")
            vals[(t * 5) % 4: (t * 5) % 4 + sp.numel()] = sp.roll(t)
        out.append(Guarded(n, torch.bfloat16, shift=shift, fill=vals))
    return out


RED_CHUNK = 16384     # elements per workgroup of the reduce's passes of more than 16 terms
RED_SUB = 4096        # the partial last chunk is walked in sub-chunks of this many elements
REDUCE_CASES = [
    # (n, world, grad_acc, slice shift, out shift)
    (1, 1, 1, 0, 0), (7, 2, 1, 0, 0), (8, 8, 1, 0, 0), (9, 3, 1, 0, 0),
    (1000, 8, 4, 0, 0), (65536 + 3, 8, 4, 0, 0), (4099, 3, 5, 0, 0),
    (5003, 8, 5, 0, 0),          # 40 terms: two passes
    (3001, 2, 33, 0, 0),         # 66 terms: three passes
    (40000, 8, 5, 0, 0),         # 40 terms: a 32-term pass over whole chunks + remainder, then 8 terms
    (20000 + 7, 2, 33, 0, 0),    # 66 terms, chunks + ragged remainder
    (16384 * 7 + 1, 8, 4, 0, 0), # whole chunks and one element
    (RED_CHUNK * 3, 8, 4, 0, 0), # whole chunks only
    (RED_CHUNK * 2 + RED_SUB * 3 + 5, 8, 4, 0, 0),   # last chunk: four sub-chunks, 5 elements in the fourth
    (RED_CHUNK + RED_SUB - 1, 4, 8, 0, 0),           # last chunk: one sub-chunk, a straddling group of 3
    (RED_CHUNK - 1, 8, 4, 0, 0), (RED_CHUNK + 1, 8, 4, 0, 0),
    (4097, 8, 4, 1, 0), (4097, 8, 4, 3, 1), (4096, 4, 2, 0, 2),   # misaligned slices / out
    (70001, 8, 4, 1, 0),         # misaligned, large
    (30011, 5, 7, 0, 0),         # 35 terms: a 32-term pass (long chunks), then 3 terms (short chunks)
    (16384 * 5 + 4096 * 2 + 4093, 8, 4, 0, 0),   # last chunk: three sub-chunks, a straddling group of 1
    (16384 * 2 - 4096 + 3, 4, 8, 0, 0),          # last chunk: four sub-chunks, 3 elements in the fourth
    (4096 * 5 + 1027, 8, 1, 0, 0),   # few terms: last chunk of 1027 elements
    (1025, 8, 1, 0, 0), (4095, 16, 1, 0, 0), (4097, 17, 1, 0, 0),   # 16 / 17 terms: the chunk switch
    (25_297_920, 8, 1, 0, 0),    # one Llama-7B block shard, 8-buffer average
]


@pytest.mark.parametrize("case", REDUCE_CASES, ids=lambda c: "n%d_N%d_A%d_s%d_o%d" % c)
def test_reduce_bitexact(case):
    n, N, A, sh, osh = case
    say("reduce", case)
    sl = _slices(n, N * A, seed=n % 97, shift=sh, specials=True)
    out = Guarded(n, torch.float32, shift=osh)
    fs.fs_reduce_shard([s.t for s in sl], out.t, N, A)
    torch.cuda.synchronize()
    out.check()
    for s in sl:
        s.check()
    ref = oracle.reduce_shard([bits(s.t) for s in sl], N, A)
    got = bits(out.t)
    refb = ref.view(np.uint32)
    nan_ref = np.isnan(ref)
    np.testing.assert_array_equal(got[~nan_ref], refb[~nan_ref])
    assert np.isnan(got.view(np.float32)[nan_ref]).all()


def test_reduce_linear_model_identity_on_gpu():
    """The data-parallel identity on the GPU path: dyadic per-rank gradients
    of a tiny linear model, averaged by the kernel, equal the full-batch
    gradient; packed through the FSDP1 layout (the oracle carries the same
    identity as a pin)."""
    say("reduce linear-model identity")
    rng = np.random.default_rng(4)
    N, A, m, D, K = 8, 4, 4, 4, 3
    B = N * A * m
    X = rng.integers(-1, 2, size=(B, D))
    W = rng.integers(-3, 4, size=(D, K))
    T = rng.integers(-4, 5, size=(B, K))
    shapes = [(D, K)]
    plan = fs.fs_plan(shapes, "bf16", N, True, "fsdp1").upload()
    grads = []
    for j in range(A):
        for k in range(N):
            rows = slice((j * N + k) * m, (j * N + k + 1) * m)
            g = (X[rows].T @ (X[rows] @ W - T[rows])) / (m * A)
            gt = torch.tensor(g.reshape(-1), dtype=torch.float32).to(torch.bfloat16).cuda()
            full = torch.empty(plan.gathered_numel, dtype=torch.bfloat16, device="cuda")
            fs.fs_pack(plan, [gt], full)
            grads.append(full)
    full_grad = (X.T @ (X @ W - T)) / B
    for r in range(N):
        c = plan.shard_numel
        out = torch.empty(c, dtype=torch.float32, device="cuda")
        fs.fs_reduce_shard([g[r * c:(r + 1) * c] for g in grads], out, N, A)
        torch.cuda.synchronize()
        exp = np.zeros(c, np.float32)
        lo, hi = r * c, min((r + 1) * c, D * K)
        if hi > lo:
            exp[:hi - lo] = full_grad.reshape(-1)[lo:hi].astype(np.float32)
        np.testing.assert_array_equal(out.cpu().numpy(), exp)


# ------------------------------------------------------------------ AdamW --

def _adam_inputs(n, seed, step, grad_bf16, shift=0):
    th = synth.normal_f32(seed, synth.STREAM_MASTER, n, 0.02, device="cuda")
    if step == 1:
        m = torch.zeros(n, device="cuda")
        v = torch.zeros(n, device="cuda")
    else:
        m = synth.normal_f32(seed, synth.STREAM_EXP_AVG, n, 1e-3, device="cuda")
        v = synth.normal_f32(seed, synth.STREAM_EXP_AVG_SQ, n, 1e-3, device="cuda") ** 2
    g = synth.normal_f32(seed, 100, n, 1e-3, device="cuda")
    if n > 20:
        th[:4] = 0.0        # pad-like elements
        m[:4] = 0.0
        v[:4] = 0.0
        g[:4] = 0.0
    if grad_bf16:
        g = g.to(torch.bfloat16)
    G = [Guarded(n, torch.float32, shift=shift, fill=x) for x in (th, m, v)]
    Gg = Guarded(n, g.dtype, shift=shift, fill=g)
    P = Guarded(n, torch.bfloat16, shift=shift)
    return G, Gg, P


ADAM_WG = 256   # elements per workgroup of the aligned AdamW kernel (one wave, 4 per lane)
ADAM_CASES = [
    # (n, step, grad_bf16, with p16, shift); the aligned kernel's last
    # workgroup is cut by n
    (1, 1, False, True, 0), (7, 1, False, True, 0), (8, 2, True, True, 0), (1003, 1000, False, True, 0),
    (ADAM_WG - 1, 3, False, False, 0), (ADAM_WG, 1, False, False, 0), (ADAM_WG + 1, 2, True, False, 0),
    (4 * ADAM_WG - 1, 3, False, False, 0), (4 * ADAM_WG, 1, False, False, 0), (4 * ADAM_WG + 1, 2, True, False, 0),
    (1 << 20, 1, False, True, 0), (1 << 20, 1000, True, False, 0), (4101, 7, False, True, 1),
    # every <bf16 grad, bf16 copy> build over whole workgroups plus a ragged last one
    (ADAM_WG * 53 + 3, 3, True, True, 0), (ADAM_WG * 29 + 2, 5, False, False, 0),
    (ADAM_WG * 37 + 1, 4, True, False, 0), (ADAM_WG * 45 + 3, 6, False, True, 0),
    (50003, 9, True, True, 2),
    # long enough for the launch's resident-workgroup cap (at least 16 rounds)
    (25_297_920, 1000, False, True, 0), (ADAM_WG * 60_001 + 2, 11, True, True, 0),
]


@pytest.mark.parametrize("case", ADAM_CASES, ids=lambda c: "n%d_t%d_bf16g%d_p%d_s%d" % c)
def test_adamw_parity(case):
    n, step, gbf, with_p16, sh = case
    say("adamw", case)
    (T, M, V), Gg, P = _adam_inputs(n, seed=n % 89 + step, step=step, grad_bf16=gbf, shift=sh)
    th0, m0, v0 = (x.t.cpu().numpy().copy() for x in (T, M, V))
    g0 = bits(Gg.t) if gbf else Gg.t.cpu().numpy().copy()
    hp = oracle.AdamWHparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=step)
    fs.fs_adamw_step(T.t, M.t, V.t, Gg.t, P.t if with_p16 else None, lr=hp.lr, beta1=hp.beta1,
                     beta2=hp.beta2, eps=hp.eps, weight_decay=hp.weight_decay, step=step)
    torch.cuda.synchronize()
    for g in (T, M, V, Gg, P):
        g.check()
    rt, rm, rv, rp = oracle.adamw_step(th0, m0, v0, g0, hp)
    gt, gm, gv = (x.t.cpu().numpy() for x in (T, M, V))
    assert np.all(np.abs(gt - rt) <= 1e-6 * np.maximum(np.abs(rt), np.abs(th0)))
    assert np.all(np.abs(gm - rm) <= 1e-6 * np.abs(rm))
    assert np.all(np.abs(gv - rv) <= 1e-6 * np.abs(rv))
    if with_p16:
        gp = bits(P.t).astype(np.int32)
        assert np.all(np.abs(gp - rp.astype(np.int32)) <= 1)
    if n > 20:
        assert (bits(T.t)[:4] == 0).all() and (bits(M.t)[:4] == 0).all() and (bits(V.t)[:4] == 0).all()
    # beyond the tolerance: fp64 division and square root are correctly rounded
    # on gfx950, so the kernel reproduces the oracle's fp64 evaluation bit for
    # bit; allow one element in a million to differ in the last fp32 bit
    inexact = np.mean((bits(T.t) != rt.view(np.uint32)) | (bits(M.t) != rm.view(np.uint32)) |
                      (bits(V.t) != rv.view(np.uint32)))
    assert inexact <= 1e-6, inexact


# ------------------------------------------------------ fused reduce+AdamW --

FUSED_CASES = [
    # (n, world, grad_acc, slice shift, with p16, with grad_out, step)
    (1, 1, 1, 0, True, True, 1),
    (16384 * 3 + 5, 8, 4, 0, True, True, 1),
    (65536, 8, 4, 0, True, False, 3),
    (4097, 3, 2, 1, True, True, 2),
    (40000, 8, 5, 0, True, True, 5),      # 40 terms: partial sums pass through grad_out
    (20007, 2, 33, 0, False, True, 2),    # 66 terms
    (30011, 5, 7, 0, True, True, 3),      # 35 terms: one reduce pass, then a fused pass of 3 terms
    (16384 * 2 + 4096 * 3 + 5, 8, 4, 0, True, True, 2),   # last chunk in four sub-chunks, 5 elements in the fourth
    (4096 * 6 + 1029, 8, 1, 0, True, False, 1),           # few terms: a last chunk of 1029 elements
    (16384 + 4095, 4, 8, 0, False, True, 4),              # straddling group of 3 elements, no bf16 copy
    # the 4-group kernel's two shapes: four slices in flight up to 8 terms, one from 9 to 16
    (70001, 8, 2, 0, True, True, 3),                      # 16 terms, ragged last chunk
    (4096 * 7 + 13, 3, 4, 0, True, False, 2),             # 12 terms
    (50000, 6, 8, 0, True, True, 6),                      # 48 terms: a 32-term reduce pass, then 16 fused
    (9001, 3, 3, 1, True, True, 2),                       # 9 terms, misaligned: the general kernel
    (25_297_920, 8, 1, 0, True, False, 1000),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "n%d_N%d_A%d_s%d_p%d_g%d_t%d" % c)
def test_reduce_adamw_fused(case):
    """Fused path against the oracle (reduce, then AdamW on its fp32 output),
    and bit-identical to the two-kernel path on the same inputs."""
    n, N, A, sh, wp, wg, step = case
    say("fused reduce+adamw", case)
    sl = _slices(n, N * A, seed=n % 53 + 1, shift=sh)
    (T, M, V), _, P = _adam_inputs(n, seed=n % 31 + step, step=step, grad_bf16=False)
    th0, m0, v0 = (x.t.cpu().numpy().copy() for x in (T, M, V))
    # two-kernel path on copies of the same state
    T2, M2, V2 = (Guarded(n, torch.float32, fill=x.t.clone()) for x in (T, M, V))
    P2 = Guarded(n, torch.bfloat16)
    G2 = Guarded(n, torch.float32)
    fs.fs_reduce_shard([s.t for s in sl], G2.t, N, A)
    fs.fs_adamw_step(T2.t, M2.t, V2.t, G2.t, P2.t, step=step)
    Gout = Guarded(n, torch.float32) if wg else None
    fs.fs_reduce_adamw_step([s.t for s in sl], T.t, M.t, V.t, P.t if wp else None,
                            Gout.t if wg else None, world=N, grad_acc=A, step=step)
    torch.cuda.synchronize()
    for g in (T, M, V, P, T2, M2, V2, P2, G2) + ((Gout,) if wg else ()):
        g.check()
    ref_g = oracle.reduce_shard([bits(s.t) for s in sl], N, A)
    rt, rm, rv, rp = oracle.adamw_step(th0, m0, v0, ref_g, oracle.AdamWHparams(step=step))
    gt, gm, gv = (x.t.cpu().numpy() for x in (T, M, V))
    assert np.all(np.abs(gt - rt) <= 1e-6 * np.maximum(np.abs(rt), np.abs(th0)))
    assert np.all(np.abs(gm - rm) <= 1e-6 * np.abs(rm))
    assert np.all(np.abs(gv - rv) <= 1e-6 * np.abs(rv))
    if wp:
        assert np.all(np.abs(bits(P.t).astype(np.int32) - rp.astype(np.int32)) <= 1)
        np.testing.assert_array_equal(bits(P.t), bits(P2.t))
    if wg:
        np.testing.assert_array_equal(bits(Gout.t), ref_g.view(np.uint32))
    for a, b in ((T, T2), (M, M2), (V, V2)):
        np.testing.assert_array_equal(bits(a.t), bits(b.t))
    inexact = np.mean((bits(T.t) != rt.view(np.uint32)) | (bits(M.t) != rm.view(np.uint32)) |
                      (bits(V.t) != rv.view(np.uint32)))
    assert inexact <= 1e-6, inexact


def test_reduce_adamw_fused_needs_grad_out_beyond_32_terms():
    sl = [torch.zeros(64, dtype=torch.bfloat16, device="cuda") for _ in range(40)]
    st = [torch.zeros(64, device="cuda") for _ in range(3)]
    with pytest.raises(fs.FsError, match="grad_out"):
        fs.fs_reduce_adamw_step(sl, *st, world=8, grad_acc=5)


# ------------------------------------------------------ bf16 reduce dtype --

RS_CASES = [
    # (n, world, grad_acc, slice shift, out shift)
    (1, 1, 1, 0, 0), (7, 2, 2, 0, 0), (8192 * 2 + 5, 8, 4, 0, 0), (16384, 8, 4, 0, 0),
    (5000, 8, 5, 0, 0),       # 40 terms: passes of 4 micro-steps
    (20007, 2, 33, 0, 0),     # 66 terms: passes of 16 micro-steps
    (4097, 8, 4, 1, 0), (9000, 3, 3, 3, 1),
    (100003, 32, 1, 0, 0),    # N = 32
    (30011, 5, 7, 0, 0),      # 35 terms: a pass of 6 micro-steps (30 terms), then one of 1 (5 terms)
    (12345, 17, 3, 0, 0),     # one micro-step (17 terms) per pass
    (8192 * 3 + 4096 + 7, 8, 4, 0, 0),   # last chunk in two sub-chunks
    (4096 * 3 + 2051, 8, 2, 0, 0),       # few terms: last chunk of 2051 elements
    (25_297_920, 8, 4, 0, 0),
]


@pytest.mark.parametrize("case", RS_CASES, ids=lambda c: "n%d_N%d_A%d_s%d_o%d" % c)
def test_reduce_bf16_reduce_dtype_bitexact(case):
    n, N, A, sh, osh = case
    say("reduce bf16 reduce dtype", case)
    sl = _slices(n, N * A, seed=n % 71 + 5, shift=sh, specials=True)
    out = Guarded(n, torch.float32, shift=osh)
    fs.fs_reduce_shard_ex([s.t for s in sl], out.t, N, A, reduce_dtype="bf16")
    torch.cuda.synchronize()
    out.check()
    ref = oracle.reduce_shard_bf16rs([bits(s.t) for s in sl], N, A)
    got = bits(out.t)
    nan = np.isnan(ref)
    np.testing.assert_array_equal(got[~nan], ref.view(np.uint32)[~nan])
    assert np.isnan(got.view(np.float32)[nan]).all()
    # reduce dtype fp32 through the same entry point is fs_reduce_shard
    out2 = Guarded(n, torch.float32)
    fs.fs_reduce_shard_ex([s.t for s in sl], out2.t, N, A, reduce_dtype="fp32")
    torch.cuda.synchronize()
    ref2 = oracle.reduce_shard([bits(s.t) for s in sl], N, A)
    nan2 = np.isnan(ref2)
    np.testing.assert_array_equal(bits(out2.t)[~nan2], ref2.view(np.uint32)[~nan2])


# ------------------------------------------------------------ cast pack --

def _params_f32(shapes, seed, shift=0):
    out, off = [], 0
    for s in shapes:
        n = int(np.prod(s)) if len(s) else 1
        vals = synth.normal_f32(seed, synth.STREAM_MASTER, n, 0.02, device="cuda", start=off)
        if n >= 12:   # specials: NaN, infinities, a bf16 tie, denormals, -0
            vals[:8] = torch.tensor([float("nan"), float("inf"), -float("inf"), 1.0 + 2.0 ** -8,
                                     1e-40, -0.0, 3.4e38, -2.0 ** -133], device="cuda")
        out.append(Guarded(n, torch.float32, shift=shift, fill=vals))
        off += n
    return out


@pytest.mark.parametrize("case", [c for c in _layout_cases() if c[3] == "bf16"], ids=lambda c: c[0])
@pytest.mark.parametrize("shift", [0, 1])
def test_pack_cast_bitexact(case, shift):
    name, mode, shapes, dt, N, uo = case
    say("pack cast", name, shift)
    plan = fs.fs_plan(shapes, "bf16", N, uo, mode).upload()
    L = _olayout(mode, shapes, "bf16", N, uo)
    params = _params_f32(shapes, seed=41, shift=shift)
    ref = oracle.pack_cast(L, [p.t.cpu().numpy() for p in params])
    G = Guarded(plan.gathered_numel, torch.bfloat16)
    fs.fs_pack_cast(plan, [p.t for p in params], G.t)
    r = N - 1
    S = Guarded(plan.shard_numel, torch.bfloat16, shift=shift)
    fs.fs_pack_cast(plan, [p.t for p in params], S.t, rank=r)
    torch.cuda.synchronize()
    G.check()
    S.check()
    np.testing.assert_array_equal(bits(G.t), ref)
    np.testing.assert_array_equal(bits(S.t), ref[r * plan.shard_numel:(r + 1) * plan.shard_numel])


# ---------------------------------------------------------------- reshard --

def _lay(kind, shapes, dt, N, uo):
    return (kind, shapes, dt, N, uo)


st97 = [(n,) for n in synth.padding_stress_numels()]
RESHARD_CASES = [
    ("block_f2_8to4", ("fsdp2", synth.llama_block_shapes(), "bf16", 8, False), ("fsdp2", None, None, 4, False)),
    ("mixed_f2_8to3", ("fsdp2", [(6, 3), (1,), (0, 2), (9,), (), (17, 5)], "bf16", 8, False), ("fsdp2", None, None, 3, False)),
    ("mlp_f1T4_to_f2_8", ("fsdp1", synth.mlp_tiny_shapes(), "bf16", 4, True), ("fsdp2", None, None, 8, False)),
    ("stress_f1F8_to_f1T5", ("fsdp1", st97, "bf16", 8, False), ("fsdp1", None, None, 5, True)),
    ("stress_fp32_f1T8_to_f2_16", ("fsdp1", st97, "fp32", 8, True), ("fsdp2", None, None, 16, False)),
    ("segments_f1F8_to_f1F7", ("fsdp1", [(k % 5 + 1,) for k in range(700)], "bf16", 8, False), ("fsdp1", None, None, 7, False)),
    ("state_fp32_f2_8to16", ("fsdp2", synth.llama_block_shapes(1024, 2816), "fp32", 8, False), ("fsdp2", None, None, 16, False)),
]


@pytest.mark.parametrize("case", RESHARD_CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("shift", [0, 1])
def test_reshard_bitexact(case, shift):
    name, (ks, shapes, dt, Ns, uos), (kd, _, _, Nd, uod) = case
    say("reshard", name, shift)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    ps = fs.fs_plan(shapes, dt, Ns, uos, ks).upload()
    pd = fs.fs_plan(shapes, dt, Nd, uod, kd).upload()
    Ls, Ld = _olayout(ks, shapes, dt, Ns, uos), _olayout(kd, shapes, dt, Nd, uod)
    params = _params(shapes, dt, seed=53)
    src_bits = oracle.pack(Ls, [bits(p.t) for p in params])
    # the source's pads hold garbage: they must not be read
    mask = np.ones(src_bits.size, bool)
    mask[Ls.index_map()] = False
    src_bits[mask] = 0x7FFF if dt == "bf16" else 0x7FFFFFFF
    ref = oracle.reshard(Ls, Ld, src_bits)
    src = Guarded(ps.gathered_numel, tdt, shift=shift, fill=from_bits(src_bits, tdt))
    dst = Guarded(pd.gathered_numel, tdt, shift=shift)
    r = fs.fs_reshard_plan(ps, pd).upload()
    fs.fs_reshard(r, src.t, dst.t)
    torch.cuda.synchronize()
    dst.check()
    src.check()
    np.testing.assert_array_equal(bits(dst.t), ref)


def test_upload_rejects_host_workspace():
    """A plan's tables must live in device memory of the current device:
    pinned or pageable host memory is refused before anything is copied."""
    plan = fs.fs_plan(synth.mlp_tiny_shapes(), "bf16", 4, True, "fsdp1")
    nb = plan.workspace_bytes
    for host in (torch.empty(nb, dtype=torch.uint8, pin_memory=True), torch.empty(nb, dtype=torch.uint8)):
        rc = fs.lib().fs_plan_upload(plan._h, host.data_ptr(), host.numel(), None)
        assert rc == fs.FS_E_INVAL and b"device memory" in fs.lib().fs_last_error()
    r = fs.fs_reshard_plan(plan, fs.fs_plan(synth.mlp_tiny_shapes(), "bf16", 2, True, "fsdp1"))
    host = torch.empty(max(16, r.workspace_bytes), dtype=torch.uint8)
    rc = fs.lib().fs_reshard_upload(r._h, host.data_ptr(), host.numel(), None)
    assert rc == fs.FS_E_INVAL and b"device memory" in fs.lib().fs_last_error()
    plan.upload()                        # a device workspace still works afterwards
    out = torch.empty(plan.gathered_numel, dtype=torch.bfloat16, device="cuda")
    fs.fs_pack(plan, [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in synth.mlp_tiny_shapes()], out)
    torch.cuda.synchronize()
    assert (out.view(torch.int16) == 0).all()


@pytest.mark.parametrize("n,shift,gbf", [(4096 * 2 + 37, 0, False), (4096 * 2 + 37, 0, True), (2999, 1, False)])
def test_adamw_special_values(n, shift, gbf):
    """Non-finite, signed-zero, subnormal and extreme inputs (gradient, theta,
    moments): wherever the oracle's result is NaN the kernel's is NaN, every
    other stored value is bit-identical to the oracle (both evaluate in fp64
    and round once), and the bf16 copy is the RNE of the stored theta."""
    say("adamw specials", n, shift, gbf)
    rng = np.random.default_rng(n + shift)
    g_sp = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-40, np.inf, -np.inf, np.nan, 3e38, -3e38, 1e-30, 1.0],
                    np.float32)
    th_sp = np.array([0.0, -0.0, 1e-45, 1e-40, 1e30, -1e30, np.nan, np.inf, 3.4e38, 1.0], np.float32)
    v_sp = np.array([0.0, 1e-45, 1e-38, 1e30, np.inf, 1.0], np.float32)
    g = rng.normal(0, 1e-3, n).astype(np.float32)
    th = rng.normal(0, 0.02, n).astype(np.float32)
    m = rng.normal(0, 1e-3, n).astype(np.float32)
    v = (rng.normal(0, 1e-3, n) ** 2).astype(np.float32)
    idx = rng.permutation(n)
    g[idx[:600]] = g_sp[np.arange(600) % g_sp.size]
    th[idx[300:900]] = th_sp[np.arange(600) % th_sp.size]
    v[idx[500:1100]] = v_sp[np.arange(600) % v_sp.size]
    m[idx[700:1000]] = -m[idx[700:1000]] * 1e30
    gt_in = torch.from_numpy(g)
    if gbf:
        gt_in = gt_in.to(torch.bfloat16)
    G = [Guarded(n, torch.float32, shift=shift, fill=torch.from_numpy(x).cuda()) for x in (th, m, v)]
    Gg = Guarded(n, gt_in.dtype, shift=shift, fill=gt_in.cuda())
    P = Guarded(n, torch.bfloat16, shift=shift)
    for step in (1, 9):
        th0, m0, v0 = (x.t.cpu().numpy().copy() for x in G)
        g0 = bits(Gg.t) if gbf else Gg.t.cpu().numpy().copy()
        fs.fs_adamw_step(G[0].t, G[1].t, G[2].t, Gg.t, P.t, step=step)
        torch.cuda.synchronize()
        for x in G + [Gg, P]:
            x.check()
        rt, rm, rv, rp = oracle.adamw_step(th0, m0, v0, g0, oracle.AdamWHparams(step=step))
        for got, ref in zip((bits(x.t) for x in G), (rt, rm, rv)):
            nan_ref = np.isnan(ref)
            assert np.isnan(got.view(np.float32)[nan_ref]).all()
            np.testing.assert_array_equal(got[~nan_ref], ref.view(np.uint32)[~nan_ref])
        gp = bits(P.t)
        nan_p = np.isnan(rt)
        np.testing.assert_array_equal(gp[~nan_p], rp[~nan_p])
        assert ((gp[nan_p] & 0x7F80) == 0x7F80).all() and ((gp[nan_p] & 0x7F) != 0).all()


@pytest.mark.parametrize("n,N,A", [(16384 * 2 + 77, 8, 4), (3001, 3, 2)])
def test_reduce_adamw_fused_special_values(n, N, A):
    """The fused path on gradient slices holding NaN, infinities, signed zeros
    and subnormals, and state with extreme values: same NaN positions as the
    two-kernel path and bit-identical everywhere else."""
    say("fused specials", n, N, A)
    sl = _slices(n, N * A, seed=7, specials=True)
    rng = np.random.default_rng(n)
    th = rng.normal(0, 0.02, n).astype(np.float32)
    th[rng.integers(0, n, 64)] = np.array([np.inf, -0.0, 1e-45, 3e38], np.float32)[np.arange(64) % 4]
    m = rng.normal(0, 1e-3, n).astype(np.float32)
    v = (rng.normal(0, 1e-3, n) ** 2).astype(np.float32)
    v[rng.integers(0, n, 64)] = 0.0
    two = [Guarded(n, torch.float32, fill=torch.from_numpy(x).cuda()) for x in (th, m, v)]
    fused = [Guarded(n, torch.float32, fill=torch.from_numpy(x).cuda()) for x in (th, m, v)]
    g32, p2, pf, gf = (Guarded(n, torch.float32), Guarded(n, torch.bfloat16), Guarded(n, torch.bfloat16),
                       Guarded(n, torch.float32))
    fs.fs_reduce_shard([s.t for s in sl], g32.t, N, A)
    fs.fs_adamw_step(*[x.t for x in two], g32.t, p2.t, step=4)
    fs.fs_reduce_adamw_step([s.t for s in sl], *[x.t for x in fused], pf.t, gf.t, world=N, grad_acc=A, step=4)
    torch.cuda.synchronize()
    for x in two + fused + [g32, p2, pf, gf] + sl:
        x.check()
    for a, b in zip(two + [g32], fused + [gf]):
        ga, gb = bits(a.t), bits(b.t)
        na, nb = np.isnan(ga.view(np.float32)), np.isnan(gb.view(np.float32))
        np.testing.assert_array_equal(na, nb)
        np.testing.assert_array_equal(ga[~na], gb[~na])
    np.testing.assert_array_equal(bits(p2.t), bits(pf.t))


@pytest.mark.parametrize("n", [(1 << 20) + 4 * 256 * 3 + 4, (1 << 24) + 4 * 256 * 3 + 4],
                         ids=["small_grid", "capped_grid"])
def test_stream_read_fill_and_copy(n):
    """The measurement aids: fill writes its word everywhere (and only inside
    the buffer); read leaves its source untouched; copy reproduces its source
    bit for bit.  n is not a whole number of workgroups; the larger size is
    long enough for the launches' resident-workgroup caps to apply."""
    say("stream read / fill / copy", n)
    g = Guarded(n, torch.float32)
    fs.fs_stream_fill(g.t, 0x3F800000)
    torch.cuda.synchronize()
    g.check()
    assert (g.t == 1.0).all()
    src = Guarded(n, torch.float32, fill=synth.normal_f32(3, 2, n, 1.0, device="cuda"))
    before = bits(src.t)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    fs.fs_stream_read(src.t, sink)
    torch.cuda.synchronize()
    src.check()
    np.testing.assert_array_equal(bits(src.t), before)
    dst = Guarded(n, torch.float32)
    fs.fs_copy_bytes(dst.t, src.t)
    torch.cuda.synchronize()
    dst.check()
    np.testing.assert_array_equal(bits(dst.t), before)


def test_deterministic_across_runs_and_streams():
    """The fixed summation order makes every result reproducible: three runs,
    one on a side stream, give identical bits for the reduce, the bf16 reduce
    dtype, AdamW and the fused step."""
    n, N, A = 16384 * 5 + 123, 8, 4
    say("determinism", n, N, A)
    sl = _slices(n, N * A, seed=61)
    th0 = synth.normal_f32(61, synth.STREAM_MASTER, n, 0.02, device="cuda")
    m0 = synth.normal_f32(61, synth.STREAM_EXP_AVG, n, 1e-3, device="cuda")
    v0 = synth.normal_f32(61, synth.STREAM_EXP_AVG_SQ, n, 1e-3, device="cuda") ** 2
    side = torch.cuda.Stream()
    runs = []
    for r in range(3):
        st = side if r == 2 else torch.cuda.current_stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            g = torch.empty(n, device="cuda")
            g_rs = torch.empty(n, device="cuda")
            th, m, v = th0.clone(), m0.clone(), v0.clone()
            thf, mf, vf = th0.clone(), m0.clone(), v0.clone()
            p, pf = (torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(2))
            fs.fs_reduce_shard([s.t for s in sl], g, N, A)
            fs.fs_reduce_shard_ex([s.t for s in sl], g_rs, N, A, reduce_dtype="bf16")
            fs.fs_adamw_step(th, m, v, g, p, step=5)
            fs.fs_reduce_adamw_step([s.t for s in sl], thf, mf, vf, pf, None, world=N, grad_acc=A, step=5)
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        runs.append([bits(x) for x in (g, g_rs, th, m, v, p, thf, mf, vf, pf)])
    for r in (1, 2):
        for a, b in zip(runs[0], runs[r]):
            np.testing.assert_array_equal(a, b)


# ----------------------------------------------------- launch span boundaries --
#
# Calls longer than one launch's span run as consecutive launches over
# sub-ranges (32M elements for the reduce and the fused step, 16M for the bf16
# reduce dtype, 64M for AdamW).  Elements on both sides of every multiple of
# 16M, the first and the ragged last ones are compared with the oracle; the
# method is element-wise, so windows of the inputs give exact expected values.

SPAN_N = 2 * (32 << 20) + 4099
ADAM_SPAN_N = (64 << 20) + 4101


def _windows(n, step=16 << 20, half=2048):
    w = [(0, 2 * half)] + [(b - half, min(n, b + half)) for b in range(step, n, step)]
    return w + [(n - 2 * half, n)]


def _offset(t, shift):
    """A copy of t whose data starts `shift` elements past a 16-byte boundary."""
    raw = torch.empty(t.numel() + shift, dtype=t.dtype, device=t.device)
    v = raw[shift:]
    v.copy_(t)
    return v


@pytest.mark.parametrize("kind,shift", [("reduce", 0), ("reduce", 1), ("bf16_reduce_dtype", 0), ("fused", 0),
                                        ("fused", 3)])
def test_span_boundaries_reduce_family(kind, shift):
    n, N, A = SPAN_N, 8, 5                  # 40 terms: a 32-term pass, then 8
    say("span boundaries", kind, n, shift)
    sl = [_offset(synth.normal_bf16(7, 100 + t, n, 1e-3, device="cuda"), shift) for t in range(N * A)]
    W = _windows(n)
    hsl = [[bits(s[a:b]) for s in sl] for a, b in W]
    if kind == "fused":
        (T, M, V), _, P = _adam_inputs(n, seed=9, step=7, grad_bf16=False)
        st0 = [[bits(x.t[a:b]).view(np.float32) for x in (T, M, V)] for a, b in W]
        G = Guarded(n, torch.float32)
        fs.fs_reduce_adamw_step(sl, T.t, M.t, V.t, P.t, G.t, world=N, grad_acc=A, step=7)
        torch.cuda.synchronize()
        for g in (T, M, V, P, G):
            g.check()
        for (a, b), terms, (th0, m0, v0) in zip(W, hsl, st0):
            ref_g = oracle.reduce_shard(terms, N, A)
            np.testing.assert_array_equal(bits(G.t[a:b]), ref_g.view(np.uint32), err_msg=f"gradient [{a}, {b})")
            rt, rm, rv, rp = oracle.adamw_step(th0, m0, v0, ref_g, oracle.AdamWHparams(step=7))
            gt, gm, gv = (bits(x.t[a:b]).view(np.float32) for x in (T, M, V))
            assert np.all(np.abs(gt - rt) <= 1e-6 * np.maximum(np.abs(rt), np.abs(th0))), (a, b)
            assert np.all(np.abs(gm - rm) <= 1e-6 * np.abs(rm)), (a, b)
            assert np.all(np.abs(gv - rv) <= 1e-6 * np.abs(rv)), (a, b)
            assert np.all(np.abs(bits(P.t[a:b]).astype(np.int32) - rp.astype(np.int32)) <= 1), (a, b)
        return
    out = Guarded(n, torch.float32)
    if kind == "reduce":
        fs.fs_reduce_shard(sl, out.t, N, A)
    else:
        fs.fs_reduce_shard_ex(sl, out.t, N, A, reduce_dtype="bf16")
    torch.cuda.synchronize()
    out.check()
    for (a, b), terms in zip(W, hsl):
        ref = oracle.reduce_shard(terms, N, A) if kind == "reduce" else oracle.reduce_shard_bf16rs(terms, N, A)
        np.testing.assert_array_equal(bits(out.t[a:b]), ref.view(np.uint32), err_msg=f"{kind} [{a}, {b})")


@pytest.mark.parametrize("shift,gbf", [(0, False), (0, True), (2, False)])
def test_span_boundaries_adamw(shift, gbf):
    n = ADAM_SPAN_N
    say("span boundaries adamw", n, shift, gbf)
    (T, M, V), Gg, P = _adam_inputs(n, seed=5, step=11, grad_bf16=gbf, shift=shift)
    W = _windows(n)
    st0 = [[bits(x.t[a:b]).view(np.float32) for x in (T, M, V)] for a, b in W]
    g0 = [bits(Gg.t[a:b]) for a, b in W]
    fs.fs_adamw_step(T.t, M.t, V.t, Gg.t, P.t, step=11)
    torch.cuda.synchronize()
    for g in (T, M, V, P):
        g.check()
    for (a, b), (th0, m0, v0), gh in zip(W, st0, g0):
        grad = gh if gbf else gh.view(np.float32)
        rt, rm, rv, rp = oracle.adamw_step(th0, m0, v0, grad, oracle.AdamWHparams(step=11))
        gt, gm, gv = (bits(x.t[a:b]).view(np.float32) for x in (T, M, V))
        assert np.all(np.abs(gt - rt) <= 1e-6 * np.maximum(np.abs(rt), np.abs(th0))), (a, b)
        assert np.all(np.abs(gm - rm) <= 1e-6 * np.abs(rm)), (a, b)
        assert np.all(np.abs(gv - rv) <= 1e-6 * np.abs(rv)), (a, b)
        assert np.all(np.abs(bits(P.t[a:b]).astype(np.int32) - rp.astype(np.int32)) <= 1), (a, b)
