"""Pins for the oracle's reduce, AdamW, bf16 rounding and ledger.

Pins used (none retypes the oracle's formula):
  * ledger figures printed on the pages (golden/ledgers.json);
  * bf16 rounding against torch's float32 -> bfloat16 conversion (library);
  * reduce: N = A = 1 is exact widening (torch's bfloat16 -> float32); the
    data-parallel identity of "Data parallelism, ZeRO and FSDP" section 2.2
    on a tiny linear model with dyadic values, where every sum is exact, so
    the averaged shard must equal the full-batch gradient bit for bit;
    hand-derived sums whose value reveals the summation order;
  * AdamW: the closed form at t=1 with zero moments, the weight-decay-only
    case, torch.optim.AdamW in float64 as a library cross-check, and zero
    (pad) elements staying exactly +0.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- ledger --


def test_ledger_strategy_table():
    g = json.load(open(os.path.join(GOLDEN, "ledgers.json")))["strategy_table"]
    t = oracle.strategy_ledger(g["P"], g["N"], g["b"], g["bopt"])
    for s in ("FULL_SHARD", "SHARD_GRAD_OP", "NO_SHARD"):
        for k in ("resident", "peak", "comm"):
            assert t[s][k] / oracle.GB == pytest.approx(g[s][k], abs=5e-3), (s, k)
    assert oracle.ledger(g["P"], g["N"], g["b"], g["bopt"])["ddp"] / oracle.GB == pytest.approx(g["full_replica"])


@pytest.mark.parametrize("name", ["seven_b_16_bytes", "zero_paper_table"])
def test_ledger_zero_stages(name):
    g = json.load(open(os.path.join(GOLDEN, "ledgers.json")))[name]
    t = oracle.ledger(g["P"], g["N"], g["b"], g["bopt"])
    dec = g.get("printed_decimals", {})
    for k in ("ddp", "zero1", "zero2", "zero3"):
        got = t[k] / oracle.GB
        if k in dec:   # printed to a few significant figures
            assert abs(got - g[k]) <= 0.5 * 10 ** -dec[k] + 1e-9, (k, got)
        else:
            assert got == pytest.approx(g[k], rel=1e-12), (k, got)


def test_ledger_fp32_accumulation_term():
    """"Data parallelism, ZeRO and FSDP" section 9: fp32 gradient accumulation adds 4 bytes per parameter on
    the kept gradient part: 4P/N under ZeRO-2/3, 4P under DP and ZeRO-1."""
    P, N = 7e9, 8
    a = oracle.ledger(P, N, 2, 12, fp32_grad_acc=False)
    b = oracle.ledger(P, N, 2, 12, fp32_grad_acc=True)
    assert b["zero3"] - a["zero3"] == pytest.approx(4 * P / N)
    assert b["zero2"] - a["zero2"] == pytest.approx(4 * P / N)
    assert b["zero1"] - a["zero1"] == pytest.approx(4 * P)
    assert b["ddp"] - a["ddp"] == pytest.approx(4 * P)


# ----------------------------------------------------------- bf16 round --

def test_bf16_round_matches_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0xFF7FFFFF,
                        0x00000001, 0x807FFFFF, 0x3F808000, 0x3F818000, 0x3F80FFFF,
                        0x3F807FFF, 0x7F7F8000, 0x7F7F7FFF, 0x00008000, 0x00018000],
                       np.uint32)
    allbits = np.concatenate([bits, special])
    f = allbits.view(np.float32)
    got = oracle.bf16_round(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    finite = ~np.isnan(f)
    np.testing.assert_array_equal(got[finite], ref[finite])
    # NaN stays NaN (quiet), sign kept
    nan_out = got[~finite]
    assert ((nan_out & 0x7F80) == 0x7F80).all() and ((nan_out & 0x007F) != 0).all()
    assert ((nan_out & 0x8000) == (allbits[~finite] >> 16 & 0x8000)).all()


# ---------------------------------------------------------------- reduce --

def _bf16_bits(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_reduce_single_term_is_widening():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 16, size=50000, dtype=np.uint64).astype(np.uint16)
    out = oracle.reduce_shard([bits], world=1, grad_acc=1)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    fin = ~np.isnan(ref)
    np.testing.assert_array_equal(out.view(np.uint32)[fin], ref.view(np.uint32)[fin])
    assert np.isnan(out[~fin]).all()


def test_reduce_order_is_array_order():
    """2^24 + 1 rounds back to 2^24 (tie to even), so the position of the big
    term decides the sum: [2^24, 1, 1, 0] sums to 2^24, [1, 1, 2^24, 0] to
    2^24 + 2 (exact).  Divided by N = 4: 2^22 and 4194304.5."""
    big = 2.0 ** 24
    a = [_bf16_bits([v]) for v in (big, 1.0, 1.0, 0.0)]
    b = [_bf16_bits([v]) for v in (1.0, 1.0, big, 0.0)]
    assert oracle.reduce_shard(a, world=4, grad_acc=1)[0] == 2.0 ** 22
    assert oracle.reduce_shard(b, world=4, grad_acc=1)[0] == 4194304.5
    # micro-step outer, rank inner: slices[j*N + k]; N=2, A=2
    assert oracle.reduce_shard(a, world=2, grad_acc=2)[0] == 2.0 ** 23
    assert oracle.reduce_shard(b, world=2, grad_acc=2)[0] == 8388609.0


def test_reduce_signed_zero_and_specials():
    nz = _bf16_bits([-0.0])
    out = oracle.reduce_shard([nz, nz], world=2, grad_acc=1)
    assert out.view(np.uint32)[0] == 0x80000000          # -0 + -0 = -0, / 2 = -0
    inf, ninf, one = _bf16_bits([math.inf]), _bf16_bits([-math.inf]), _bf16_bits([1.0])
    assert np.isnan(oracle.reduce_shard([inf, ninf], 2, 1)[0])
    assert oracle.reduce_shard([inf, one], 2, 1)[0] == math.inf


def test_reduce_division_not_reciprocal():
    """One IEEE division by N: for N = 3 and a sum of 1, the result is
    fl32(1/3); 3 terms of 1/3 each exercise rounding of the quotient."""
    one = _bf16_bits([1.0])
    zero = _bf16_bits([0.0])
    assert oracle.reduce_shard([one, zero, zero], 3, 1)[0] == np.float32(1.0) / np.float32(3.0)
    seven = _bf16_bits([7.0])
    # 7/3 vs 7 * fl32(1/3): these differ in fp32
    assert np.float32(7.0) / np.float32(3.0) != np.float32(7.0) * (np.float32(1.0) / np.float32(3.0))
    assert oracle.reduce_shard([seven, zero, zero], 3, 1)[0] == np.float32(7.0) / np.float32(3.0)


def _round_to_f32_exact(q: Fraction) -> np.float32:
    """Correctly rounded (ties to even) fp32 of a rational, by exact compare."""
    c = np.float32(float(q))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - q)
        key = (d, int(np.array(cand).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


@pytest.mark.parametrize("world,grad_acc", [(1, 1), (2, 1), (3, 1), (4, 2), (8, 4), (5, 2), (8, 1)])
def test_reduce_linear_model_identity(world, grad_acc):
    """Data parallelism, ZeRO and FSDP, section 2.2: with equal samples per
    rank, the mean over ranks of the per-rank gradients of
    L_r = (N/B) sum_{i in S_r} l_i equals the full-batch gradient of
    L = (1/B) sum_i l_i.  With grad_acc micro-steps each micro-step loss is
    divided by A (section 5).  Model: l_i = 0.5*||x_i W - t_i||^2 with
    x in {-1,0,1}^D, small-integer W and t, m = 4 samples per micro-batch: all
    per-rank gradients are dyadic with few bits (exact in bf16) and their
    sums are exact in fp32, so the only rounding is the final fp32 result,
    which must equal the correctly rounded full-batch gradient.

    The gradient is laid out through the FSDP1 layout (two parameters W and
    a bias), and the reduce runs on every rank's shard."""
    rng = np.random.default_rng(100 + world * 10 + grad_acc)
    D, K, m = 4, 3, 4
    B = world * grad_acc * m
    X = rng.integers(-1, 2, size=(B, D))
    W = rng.integers(-3, 4, size=(D, K))
    bvec = rng.integers(-2, 3, size=(K,))
    T = rng.integers(-4, 5, size=(B, K))
    shapes = [(D, K), (K,)]
    L = oracle.fsdp1_layout(shapes, 2, world, use_orig_params=True)

    def grads(rows, scale: Fraction):
        R = X[rows] @ W + bvec - T[rows]                   # residuals (ints)
        gW = [[Fraction(int(v)) * scale for v in row] for row in (X[rows].T @ R)]
        gb = [Fraction(int(v)) * scale for v in R.sum(axis=0)]
        return [x for row in gW for x in row] + gb

    # micro-step j of rank k holds samples [(j*N + k)*m, +m); its loss is
    # (N/B') sum l_i / A with B' = N*m per micro-step -> scale 1/(m*A)
    slices_full = []
    for j in range(grad_acc):
        for k in range(world):
            rows = np.arange((j * world + k) * m, (j * world + k + 1) * m)
            g = grads(rows, Fraction(1, m * grad_acc))
            vals = np.array([float(x) for x in g], np.float32)
            bits = _bf16_bits(vals)
            assert (oracle.bf16_to_f32(bits) == vals).all()    # exact in bf16
            nw = D * K
            slices_full.append(oracle.pack(L, [bits[:nw], bits[nw:]]))
    full = grads(np.arange(B), Fraction(1, B))
    expect = np.array([_round_to_f32_exact(q) for q in full], np.float32)
    # every rank's shard
    avg = np.concatenate([
        oracle.reduce_shard([s[r * L.shard:(r + 1) * L.shard] for s in slices_full],
                            world, grad_acc)
        for r in range(world)])
    idx = L.index_map()
    np.testing.assert_array_equal(avg[idx].view(np.uint32), expect.view(np.uint32))
    mask = np.ones(avg.size, bool)
    mask[idx] = False
    assert (avg[mask].view(np.uint32) == 0).all()          # pads stay +0


# ----------------------------------------------------------------- AdamW --

def _f32_ulp_diff(a, b):
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


def test_adamw_closed_form_t1():
    """t=1, m=v=0: m' = (1-b1) g, v' = (1-b2) g^2, and m_hat = g,
    v_hat = g^2, so theta' = theta (1 - lr wd) - lr g / (|g| + eps)."""
    rng = np.random.default_rng(5)
    n = 20000
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    g[:5] = [0.0, -0.0, 1e-30, -3e-9, 5.0]
    z = np.zeros(n, np.float32)
    hp = oracle.AdamWHparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1)
    th1, m1, v1, p16 = oracle.adamw_step(th, z, z, g, hp)
    lr, b1, b2, eps, wd = (Fraction(float(np.float32(x))) for x in (hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay))
    for e in list(range(5)) + list(range(5, n, 97)):
        G, TH = Fraction(float(g[e])), Fraction(float(th[e]))
        m_exact = (1 - b1) * G
        v_exact = (1 - b2) * G * G
        upd = lr * G / (abs(G) + eps)   # |g| exact
        th_exact = TH * (1 - lr * wd) - upd
        assert _f32_ulp_diff(m1[e], _round_to_f32_exact(m_exact)) == 0, e
        assert _f32_ulp_diff(v1[e], _round_to_f32_exact(v_exact)) == 0 or v_exact == 0, e
        assert _f32_ulp_diff(th1[e], _round_to_f32_exact(th_exact)) <= 1, e
    ref16 = torch.from_numpy(th1.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(p16, ref16)


def test_adamw_weight_decay_only_and_pads():
    """g = m = v = 0: the update term is 0/(0+eps) = 0 and theta' is
    theta*(1 - lr*wd) rounded once; theta = 0 stays exactly +0 (pad)."""
    th = np.array([0.0, 0.5, -0.25, 3.0, 1e-3], np.float32)
    z = np.zeros_like(th)
    hp = oracle.AdamWHparams(lr=1e-2, weight_decay=0.1, step=7)
    th1, m1, v1, p16 = oracle.adamw_step(th, z, z, z, hp)
    f = 1 - Fraction(float(np.float32(1e-2))) * Fraction(float(np.float32(0.1)))
    for e in range(th.size):
        assert th1[e] == _round_to_f32_exact(Fraction(float(th[e])) * f)
    assert th1.view(np.uint32)[0] == 0 and m1.view(np.uint32).max() == 0
    assert v1.view(np.uint32).max() == 0 and p16[0] == 0


def _torch_adamw_f64(th, m, v, g, hp, steps=1):
    p = torch.nn.Parameter(torch.from_numpy(th.astype(np.float64)))
    opt = torch.optim.AdamW([p], lr=float(np.float32(hp.lr)),
                            betas=(float(np.float32(hp.beta1)), float(np.float32(hp.beta2))),
                            eps=float(np.float32(hp.eps)),
                            weight_decay=float(np.float32(hp.weight_decay)),
                            foreach=False, fused=False)
    st = opt.state[p]
    st["step"] = torch.tensor(float(hp.step - 1), dtype=torch.float64)
    st["exp_avg"] = torch.from_numpy(m.astype(np.float64))
    st["exp_avg_sq"] = torch.from_numpy(v.astype(np.float64))
    for _ in range(steps):
        p.grad = torch.from_numpy(g.astype(np.float64))
        opt.step()
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


@pytest.mark.parametrize("step", [1, 2, 10, 1000])
def test_adamw_vs_torch_float64(step):
    rng = np.random.default_rng(step)
    n = 50000
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32) if step > 1 else np.zeros(n, np.float32)
    v = ((rng.standard_normal(n) * 1e-3) ** 2).astype(np.float32) if step > 1 else np.zeros(n, np.float32)
    hp = oracle.AdamWHparams(step=step)
    th1, m1, v1, _ = oracle.adamw_step(th, m, v, g, hp)
    rt, rm, rv = _torch_adamw_f64(th, m, v, g, hp)
    # fp32 storage of a double result: within one rounding (plus the
    # double-vs-lerp/sqrt-split rounding noise of the library formula)
    assert np.all(np.abs(th1 - rt) <= 1e-6 * np.maximum(np.abs(rt), np.abs(th)) + 1e-30)
    assert np.all(np.abs(m1 - rm) <= 2 ** -23 * np.abs(rm) + 1e-38)
    assert np.all(np.abs(v1 - rv) <= 2 ** -23 * np.abs(rv) + 1e-44)


def test_adamw_bf16_grad_input():
    rng = np.random.default_rng(9)
    n = 1000
    g32 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    gb = oracle.bf16_round(g32)
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    z = np.zeros(n, np.float32)
    hp = oracle.AdamWHparams(step=3)
    a = oracle.adamw_step(th, z, z, gb, hp)
    b = oracle.adamw_step(th, z, z, oracle.bf16_to_f32(gb), hp)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# ------------------------------------------------- bf16 reduce dtype, cast --

def test_reduce_bf16rs_single_microstep_is_rounded_fp32_average():
    """A = 1: the delivered bf16 average is the bf16 rounding (torch's
    conversion) of the fp32 average, widened exactly."""
    rng = np.random.default_rng(12)
    for N in (1, 2, 3, 8):
        sl = [oracle.bf16_round((rng.standard_normal(20000) * 1e-3).astype(np.float32)) for _ in range(N)]
        f32 = oracle.reduce_shard(sl, N, 1)
        ref = torch.from_numpy(f32.copy()).to(torch.bfloat16).to(torch.float32).numpy()
        np.testing.assert_array_equal(oracle.reduce_shard_bf16rs(sl, N, 1).view(np.uint32), ref.view(np.uint32))


def test_reduce_bf16rs_rounds_each_microstep():
    """N = 2, A = 2, every micro-step's ranks hold 1 and 2^-8: the average
    0.5 + 2^-9 lies halfway between the bf16 neighbours 0.5 and 0.5 + 2^-8 and
    rounds to the even one, 0.5; two micro-steps give 1.0.  The fp32 path keeps
    1 + 2^-8."""
    one, tiny = _bf16_bits([1.0]), _bf16_bits([2.0 ** -8])
    sl = [one, tiny, one, tiny]
    assert oracle.reduce_shard_bf16rs(sl, 2, 2)[0] == 1.0
    assert oracle.reduce_shard(sl, 2, 2)[0] == 1.0 + 2.0 ** -8


@pytest.mark.parametrize("world,grad_acc", [(2, 2), (4, 2), (8, 4)])
def test_reduce_bf16rs_linear_model_identity(world, grad_acc):
    """With dyadic per-rank gradients whose micro-step averages are exact in
    bf16, the bf16 reduce dtype loses nothing: the result is the full-batch
    gradient of the data-parallel identity ("Data parallelism, ZeRO and
    FSDP" section 2.2)."""
    rng = np.random.default_rng(3 + world)
    D, K, m = 2, 2, 2
    B = world * grad_acc * m
    X = rng.integers(-1, 2, size=(B, D))
    W = rng.integers(-1, 2, size=(D, K))
    T = rng.integers(-1, 2, size=(B, K))
    slices = []
    for j in range(grad_acc):
        for k in range(world):
            rows = slice((j * world + k) * m, (j * world + k + 1) * m)
            g = (X[rows].T @ (X[rows] @ W - T[rows])).reshape(-1) / (m * grad_acc)
            slices.append(_bf16_bits(g.astype(np.float32)))
    full = (X.T @ (X @ W - T)).reshape(-1) / B
    # micro-step averages must be exact in bf16 for the identity to be exact
    for j in range(grad_acc):
        avg = sum(oracle.bf16_to_f32(slices[j * world + k]).astype(np.float64) for k in range(world)) / world
        assert np.array_equal(oracle.bf16_to_f32(oracle.bf16_round(avg.astype(np.float32))), avg.astype(np.float32))
    np.testing.assert_array_equal(oracle.reduce_shard_bf16rs(slices, world, grad_acc), full.astype(np.float32))


def test_pack_cast_is_pack_of_rounded_params():
    """The cast copy-in equals the bit copy-in of the params rounded to bf16
    by torch's conversion, for both layouts and every rank."""
    rng = np.random.default_rng(8)
    for kind, shapes, N, uo in (("f1", [(7,), (1,), (33,), (0,), (16,)], 4, True),
                                ("f1", [(7,), (1,), (33,), (0,), (16,)], 3, False),
                                ("f2", [(6, 3), (), (9,), (1, 5)], 4, None)):
        L = oracle.fsdp1_layout(shapes, 2, N, uo) if kind == "f1" else oracle.fsdp2_layout(shapes, 2, N)
        p32 = [(rng.standard_normal(int(n)) * 0.02).astype(np.float32) for n in L.numel]
        if p32[0].size:
            p32[0][0] = np.float32(np.nan)
        rounded = [torch.from_numpy(p.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                   for p in p32]
        ref = oracle.pack(L, rounded)
        got = oracle.pack_cast(L, p32)
        finite = ~np.isnan(oracle.bf16_to_f32(ref))
        np.testing.assert_array_equal(got[finite], ref[finite])
        assert np.isnan(oracle.bf16_to_f32(got[~finite])).all()
        for r in range(N):
            np.testing.assert_array_equal(oracle.pack_cast(L, p32, rank=r), got[r * L.shard:(r + 1) * L.shard])
