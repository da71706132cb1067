"""Host-side checks of the C-ABI library (no GPU call is made).

* libfsstate.so loads and exports every function include/*.h declares;
* the planner (fs_plan) lays out exactly what the oracle lays out, on the
  exhaustive tiny cases and on the workload shapes;
* the ledger fields equal the oracle's ledger;
* argument validation returns the documented error codes before touching
  the GPU.
"""
import ctypes
import itertools
import os
import re

import numpy as np
import pytest

import fsdp_sharded_state_amd as fs
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_symbol():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            hdr = open(os.path.join(ROOT, "include", h)).read()
            names |= set(re.findall(r"^\s*(?:int|void|const char\s*\*)\s*\*?\s*(fs_\w+)\s*\(", hdr, re.M))
    assert {"fs_plan", "fs_pack", "fs_unpack", "fs_reduce_shard", "fs_adamw_step", "fs_load_local",
            "fs_copy_bytes", "fs_stream_read", "fs_stream_fill"} <= names
    L = ctypes.CDLL(fs.LIB_PATH)
    missing = [n for n in sorted(names) if not hasattr(L, n)]
    assert not missing, missing


def _plan_index_map(plan):
    numels = [plan.param(i).numel for i in range(plan.n_params)]
    offs = np.concatenate([[0], np.cumsum(numels)]).astype(np.int64)
    out = np.full(int(offs[-1]), -1, np.int64)
    for dst, src, ln, p, r in plan.segments():
        assert ln > 0
        assert dst // plan.shard_numel == r and (dst + ln - 1) // plan.shard_numel == r
        tgt = out[offs[p] + src: offs[p] + src + ln]
        assert (tgt == -1).all(), "element placed twice"
        tgt[:] = np.arange(dst, dst + ln)
    assert (out >= 0).all(), "element never placed"
    return out


def _oracle_layout(kind, shapes, eb, N, uo):
    return (oracle.fsdp1_layout(shapes, eb, N, uo) if kind == "fsdp1"
            else oracle.fsdp2_layout(shapes, eb, N))


def _plan_index_sampled(plan, param, elem):
    """Plan's gathered index of sampled elements, after checking that the
    segments tile every parameter exactly once and never overlap in the
    gathered buffer."""
    segs = np.array(plan.segments(), np.int64).reshape(-1, 5)
    d = segs[np.argsort(segs[:, 0], kind="stable")]
    assert (d[1:, 0] >= d[:-1, 0] + d[:-1, 2]).all()            # disjoint in gathered
    out = np.empty(param.size, np.int64)
    for i in range(plan.n_params):
        si = segs[segs[:, 3] == i]
        si = si[np.argsort(si[:, 1])]
        numel = plan.param(i).numel
        if numel == 0:
            assert si.size == 0
            continue
        assert si[0, 1] == 0 and (si[1:, 1] == si[:-1, 1] + si[:-1, 2]).all()
        assert si[-1, 1] + si[-1, 2] == numel
        sel = param == i
        k = np.searchsorted(si[:, 1], elem[sel], side="right") - 1
        out[sel] = si[k, 0] + elem[sel] - si[k, 1]
    return out


def _compare(kind, shapes, eb, N, uo, grad_acc=1):
    P = fs.fs_plan(shapes, "bf16" if eb == 2 else "fp32", N, uo, kind, grad_acc)
    L = _oracle_layout(kind, shapes, eb, N, uo)
    assert P.shard_numel == L.shard
    assert P.gathered_numel == N * L.shard
    assert P.total_numel == int(L.numel.sum())
    if P.total_numel <= 1 << 20:
        np.testing.assert_array_equal(_plan_index_map(P), L.index_map())
    else:   # sampled elements, plus the first and last element of every parameter
        rng = np.random.default_rng(P.total_numel % 1000)
        nz = np.nonzero(L.numel)[0]
        param = np.concatenate([rng.choice(nz, 200000), nz, nz]).astype(np.int32)
        elem = (rng.random(param.size) * L.numel[param]).astype(np.int64)
        elem[200000:200000 + nz.size] = 0
        elem[200000 + nz.size:] = L.numel[nz] - 1
        np.testing.assert_array_equal(_plan_index_sampled(P, param, elem), L.index_at(param, elem))
    for i in range(len(shapes)):
        pl = P.param(i)
        assert pl.numel == L.numel[i]
        if kind == "fsdp1":
            assert pl.start == L.start[i]
        else:
            assert (pl.chunk_rows, pl.row, pl.pre) == (L.chunk_rows[i], L.row[i], L.pre[i])
    if kind == "fsdp1":
        assert P.flat_numel == L.flat_len
        assert P.align_pad == L.flat_len - P.total_numel
        assert P.tail_pad == N * L.shard - L.flat_len
    led = oracle.ledger(P.total_numel, N, eb, 12, fp32_grad_acc=grad_acc > 1)["zero3"]
    assert P.ledger_ideal_bytes == pytest.approx(led, rel=1e-12)
    return P


@pytest.mark.parametrize("eb", [2, 4])
@pytest.mark.parametrize("uo", [False, True])
def test_plan_matches_oracle_fsdp1_exhaustive(eb, uo):
    for n in (1, 2, 3):
        for numels in itertools.product(range(0, 10, 1 if n < 3 else 2), repeat=n):
            for N in (1, 2, 3, 4, 7, 8):
                _compare("fsdp1", [(x,) for x in numels], eb, N, uo)


def test_plan_matches_oracle_fsdp2_exhaustive():
    shapes_1 = [(d0, d1) for d0 in range(10) for d1 in (1, 3)] + [(5,), ()]
    for shapes in itertools.product(shapes_1, repeat=2):
        for N in (1, 2, 3, 4, 8):
            _compare("fsdp2", list(shapes), 2, N, False)


def test_plan_matches_oracle_workloads():
    _compare("fsdp1", synth.mlp_tiny_shapes(), 2, 4, True)
    _compare("fsdp2", synth.llama_block_shapes(), 2, 8, False, grad_acc=1)
    st = [(n,) for n in synth.padding_stress_numels()]
    for eb in (2, 4):
        for uo in (True, False):
            _compare("fsdp1", st, eb, 8, uo)
    for g in synth.llama_model_groups(1, 4096, 11008)[-1:]:
        _compare("fsdp2", g, 2, 8, False, grad_acc=4)


def test_seven_b_ledger_from_plans():
    """Sum of the 33 group plans of the 7B model at N=8: the pages' 16 B/param
    ZeRO-3 figure (14 GB for 7B) scales to this model's P = 6.738e9."""
    groups = synth.llama_model_groups(32, 4096, 11008)
    plans = [fs.fs_plan(g, "bf16", 8, False, "fsdp2", 1) for g in groups]
    P = sum(p.total_numel for p in plans)
    assert P == 6738411520
    ideal = sum(p.ledger_ideal_bytes for p in plans)
    assert ideal == pytest.approx(oracle.ledger(P, 8, 2, 12)["zero3"])
    assert sum(p.shard_numel for p in plans) == 842301440
    assert sum(p.tail_pad for p in plans) == 0


def test_plan_errors():
    L = fs.lib()
    h = ctypes.c_void_p()
    nd = (ctypes.c_int32 * 1)(1)
    dm = (ctypes.c_int64 * 1)(5)
    assert L.fs_plan(1, nd, dm, 0, 0, 0, 1, 1, ctypes.byref(h)) == fs.FS_E_INVAL      # N < 1
    assert L.fs_plan(1, nd, dm, 0, 4, 0, 1, 0, ctypes.byref(h)) == fs.FS_E_INVAL      # grad_acc < 1
    assert L.fs_plan(1, nd, dm, 7, 4, 0, 1, 1, ctypes.byref(h)) == fs.FS_E_DTYPE
    assert L.fs_plan(1, nd, dm, 0, 4, 1, 2, 1, ctypes.byref(h)) == fs.FS_E_UNSUPPORTED
    assert L.fs_plan(-1, nd, dm, 0, 4, 0, 1, 1, ctypes.byref(h)) == fs.FS_E_INVAL
    assert L.fs_plan(1, None, None, 0, 4, 0, 1, 1, ctypes.byref(h)) == fs.FS_E_INVAL
    assert L.fs_plan(1, nd, dm, 0, 4, 0, 3, 1, ctypes.byref(h)) == fs.FS_E_INVAL      # mode
    neg = (ctypes.c_int64 * 1)(-2)
    assert L.fs_plan(1, nd, neg, 0, 4, 0, 1, 1, ctypes.byref(h)) == fs.FS_E_INVAL
    big_nd = (ctypes.c_int32 * 1)(3)
    big = (ctypes.c_int64 * 3)(1 << 30, 1 << 30, 1 << 30)
    assert L.fs_plan(1, big_nd, big, 0, 4, 0, 1, 1, ctypes.byref(h)) == fs.FS_E_OVERFLOW
    nd9 = (ctypes.c_int32 * 1)(9)
    assert L.fs_plan(1, nd9, (ctypes.c_int64 * 9)(*[1] * 9), 0, 4, 0, 1, 1, ctypes.byref(h)) == fs.FS_E_INVAL
    assert b"world" in L.fs_last_error() or len(L.fs_last_error()) > 0


def test_empty_and_degenerate_plans():
    p = fs.fs_plan([], "bf16", 4, True, "fsdp1")
    assert p.shard_numel == 0 and p.gathered_numel == 0 and p.n_segments == 0
    p = fs.fs_plan([(0,), (0, 5)], "bf16", 4, False, "fsdp2")
    assert p.shard_numel == 0 and p.n_segments == 0
    p = fs.fs_plan([()], "fp32", 3, False, "fsdp2")       # scalar -> [1]
    assert p.shard_numel == 1 and p.segments() == [(0, 0, 1, 0, 0)]
    p = fs.fs_plan([(5,)], "bf16", 1, True, "fsdp1")      # N = 1
    assert p.shard_numel == 5 and p.segments() == [(0, 0, 5, 0, 0)]


def test_call_validation_before_gpu():
    """Invalid calls fail on the host; n = 0 calls succeed without a launch."""
    L = fs.lib()
    p = fs.fs_plan([(3,), (5,)], "bf16", 4, True, "fsdp1")
    # not uploaded
    assert L.fs_pack(p._h, ctypes.c_void_p(16), ctypes.c_void_p(16), -1, None) == fs.FS_E_INVAL
    assert L.fs_unpack(p._h, ctypes.c_void_p(16), ctypes.c_void_p(16), None) == fs.FS_E_INVAL
    assert L.fs_pack(None, None, None, -1, None) == fs.FS_E_INVAL
    sl = (ctypes.c_void_p * 2)(16, 32)
    assert L.fs_reduce_shard(-1, 2, 1, sl, ctypes.c_void_p(64), None) == fs.FS_E_INVAL
    assert L.fs_reduce_shard(8, 0, 1, sl, ctypes.c_void_p(64), None) == fs.FS_E_INVAL
    assert L.fs_reduce_shard(8, 2, 0, sl, ctypes.c_void_p(64), None) == fs.FS_E_INVAL
    assert L.fs_reduce_shard(0, 2, 1, sl, ctypes.c_void_p(64), None) == fs.FS_OK
    assert L.fs_reduce_shard(8, 2, 1, None, ctypes.c_void_p(64), None) == fs.FS_E_INVAL
    odd = (ctypes.c_void_p * 2)(17, 32)
    assert L.fs_reduce_shard(8, 2, 1, odd, ctypes.c_void_p(1 << 20), None) == fs.FS_E_ALIGN
    assert L.fs_reduce_shard(8, 2, 1, sl, ctypes.c_void_p((1 << 20) + 2), None) == fs.FS_E_ALIGN
    ov = (ctypes.c_void_p * 2)(1 << 20, 1 << 21)
    assert L.fs_reduce_shard(8, 2, 1, ov, ctypes.c_void_p((1 << 20) + 8), None) == fs.FS_E_INVAL   # overlap
    hp = fs.AdamWHparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 0, 1)
    f = ctypes.c_void_p(256)
    assert L.fs_adamw_step(8, f, f, f, f, 1, None, None, None) == fs.FS_E_INVAL
    assert L.fs_adamw_step(-1, f, f, f, f, 1, None, ctypes.byref(hp), None) == fs.FS_E_INVAL
    assert L.fs_adamw_step(8, f, f, f, f, 5, None, ctypes.byref(hp), None) == fs.FS_E_DTYPE
    assert L.fs_adamw_step(0, f, f, f, f, 1, None, ctypes.byref(hp), None) == fs.FS_OK
    bad = fs.AdamWHparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 0, 0)
    assert L.fs_adamw_step(8, f, f, f, f, 1, None, ctypes.byref(bad), None) == fs.FS_E_INVAL
    bad = fs.AdamWHparams(1e-3, 1.0, 0.999, 1e-8, 0.01, 0, 1)
    assert L.fs_adamw_step(8, f, f, f, f, 1, None, ctypes.byref(bad), None) == fs.FS_E_INVAL
    assert L.fs_adamw_step(8, ctypes.c_void_p(258), f, f, f, 1, None, ctypes.byref(hp), None) == fs.FS_E_ALIGN
    assert L.fs_copy_bytes(ctypes.c_void_p(256), ctypes.c_void_p(512), 15, None) == fs.FS_E_INVAL
    assert L.fs_copy_bytes(ctypes.c_void_p(264), ctypes.c_void_p(512), 16, None) == fs.FS_E_ALIGN
    assert L.fs_stream_read(ctypes.c_void_p(256), 15, ctypes.c_void_p(512), None) == fs.FS_E_INVAL
    assert L.fs_stream_read(ctypes.c_void_p(264), 16, ctypes.c_void_p(512), None) == fs.FS_E_ALIGN
    assert L.fs_stream_read(ctypes.c_void_p(256), 16, None, None) == fs.FS_E_INVAL
    assert L.fs_stream_fill(ctypes.c_void_p(256), -16, 0, None) == fs.FS_E_INVAL
    assert L.fs_stream_fill(ctypes.c_void_p(260), 16, 0, None) == fs.FS_E_ALIGN
    assert L.fs_stream_fill(ctypes.c_void_p(256), 0, 0, None) == fs.FS_OK           # nothing to do


def test_adamw_rejects_arrays_that_share_memory():
    """AdamW updates element k of every array from element k of the others:
    any two of theta, m, v, the gradient and the bf16 copy that share memory
    are refused on the host, for the fused step as well.  n = 2**40 is more
    than one launch covers, so a call that passes every check still fails
    (FS_E_OVERFLOW) before launching anything: no call here reaches a GPU."""
    L = fs.lib()
    hp = fs.AdamWHparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 0, 1)
    n = 1 << 40
    A, B, C, G, P, S = (k << 44 for k in range(1, 7))          # disjoint, 16 TiB apart
    vp = ctypes.c_void_p

    def adamw(th, m, v, g, p, gdt=fs.FS_FP32):
        return L.fs_adamw_step(n, vp(th), vp(m), vp(v), vp(g), gdt, vp(p), ctypes.byref(hp), None)

    assert adamw(A, B, C, G, P) == fs.FS_E_OVERFLOW                           # disjoint: only the size fails
    for args, name in [((A, A, C, G, P), b"exp_avg"), ((A, B, B + 4 * n - 16, G, P), b"exp_avg_sq"),
                       ((A, B, C, A + 16, P), b"grad"), ((A, B, C, G, C + 4 * n - 2), b"param_bf16")]:
        assert adamw(*args) == fs.FS_E_INVAL, name
        assert name in L.fs_last_error() and b"overlaps" in L.fs_last_error()
    assert adamw(A, A + 4 * n, C, G, P) == fs.FS_E_OVERFLOW                   # adjacent, not overlapping
    assert adamw(A, B, C, G, G + 2 * n, fs.FS_BF16) == fs.FS_E_OVERFLOW       # a bf16 gradient is 2n bytes
    assert adamw(A, B, C, G, G + 2 * n, fs.FS_FP32) == fs.FS_E_INVAL          # an fp32 one is 4n

    sl = (ctypes.c_void_p * 2)(S, S + (1 << 43))
    for fused in (L.fs_reduce_adamw_step, L.fs_reduce_adamw_step_noalloc):
        def call(th, m, v, p, go=None):
            extra = (vp(go),) if fused is L.fs_reduce_adamw_step else ()
            return fused(n, 2, 1, sl, vp(th), vp(m), vp(v), vp(p), *extra, ctypes.byref(hp), None)
        assert call(A, B, C, P) == fs.FS_E_OVERFLOW
        for args, name in [((A, B, A, P), b"exp_avg_sq"), ((A, B, C, A + 2), b"param_bf16")]:
            assert call(*args) == fs.FS_E_INVAL, name
            assert name in L.fs_last_error() and b"overlaps" in L.fs_last_error()
    assert L.fs_reduce_adamw_step(n, 2, 1, sl, vp(A), vp(B), vp(C), vp(P), vp(B + 8), ctypes.byref(hp),
                                  None) == fs.FS_E_INVAL
    assert b"grad_out" in L.fs_last_error()

def test_fused_call_validation_before_gpu():
    L = fs.lib()
    hp = fs.AdamWHparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 0, 1)
    f = ctypes.c_void_p(1 << 24)
    sl = (ctypes.c_void_p * 2)(1 << 20, 1 << 21)
    assert L.fs_reduce_adamw_step(-1, 2, 1, sl, f, f, f, None, None, ctypes.byref(hp), None) == fs.FS_E_INVAL
    assert L.fs_reduce_adamw_step(8, 0, 1, sl, f, f, f, None, None, ctypes.byref(hp), None) == fs.FS_E_INVAL
    assert L.fs_reduce_adamw_step(8, 2, 1, sl, f, f, f, None, None, None, None) == fs.FS_E_INVAL
    assert L.fs_reduce_adamw_step(0, 2, 1, sl, f, f, f, None, None, ctypes.byref(hp), None) == fs.FS_OK
    big = (ctypes.c_void_p * 40)(*[(1 << 20) * (k + 1) for k in range(40)])
    assert L.fs_reduce_adamw_step(8, 8, 5, big, ctypes.c_void_p(1 << 30), ctypes.c_void_p(1 << 31),
                                  ctypes.c_void_p(1 << 32), None, None, ctypes.byref(hp), None) == fs.FS_E_INVAL
    assert b"grad_out" in L.fs_last_error()
    assert L.fs_reduce_adamw_step(8, 2, 1, sl, ctypes.c_void_p((1 << 24) + 2), f, f, None, None,
                                  ctypes.byref(hp), None) == fs.FS_E_ALIGN
    # an output overlapping a slice
    assert L.fs_reduce_adamw_step(8, 2, 1, sl, ctypes.c_void_p((1 << 20) + 4), ctypes.c_void_p(1 << 25),
                                  ctypes.c_void_p(1 << 26), None, None, ctypes.byref(hp), None) == fs.FS_E_INVAL


def test_reduce_ex_and_pack_cast_validation_before_gpu():
    L = fs.lib()
    sl = (ctypes.c_void_p * 2)(1 << 20, 1 << 21)
    out = ctypes.c_void_p(1 << 24)
    assert L.fs_reduce_shard_ex(8, 2, 1, 7, sl, out, None) == fs.FS_E_DTYPE
    assert L.fs_reduce_shard_ex(-1, 2, 1, fs.FS_BF16, sl, out, None) == fs.FS_E_INVAL
    assert L.fs_reduce_shard_ex(0, 2, 1, fs.FS_BF16, sl, out, None) == fs.FS_OK
    many = (ctypes.c_void_p * 33)(*[(1 << 20) * (k + 1) for k in range(33)])
    assert L.fs_reduce_shard_ex(8, 33, 1, fs.FS_BF16, many, ctypes.c_void_p(1 << 30), None) == fs.FS_E_UNSUPPORTED
    p32 = fs.fs_plan([(3,), (5,)], "fp32", 4, True, "fsdp1")
    assert L.fs_pack_cast(p32._h, ctypes.c_void_p(16), fs.FS_BF16, ctypes.c_void_p(16), -1, None) == fs.FS_E_UNSUPPORTED
    p16 = fs.fs_plan([(3,), (5,)], "bf16", 4, True, "fsdp1")
    assert L.fs_pack_cast(p16._h, ctypes.c_void_p(16), fs.FS_FP32, ctypes.c_void_p(16), -1, None) == fs.FS_E_INVAL  # not uploaded
    assert L.fs_pack_cast(p16._h, ctypes.c_void_p(16), 9, ctypes.c_void_p(16), -1, None) == fs.FS_E_DTYPE


@pytest.mark.parametrize("dtype,eb", [("bf16", 2), ("fp32", 4)])
@pytest.mark.parametrize("grad_acc", [1, 4])
def test_plan_ledger_fields_match_oracle(dtype, eb, grad_acc):
    """Every per-rank ledger field of a plan equals the oracle's ledger for
    the group's P, N, b and bopt = 12."""
    for N in (1, 2, 8, 64):
        p = fs.fs_plan(synth.llama_block_shapes(), dtype, N, False, "fsdp2", grad_acc)
        P = p.total_numel
        led = oracle.ledger(P, N, eb, 12, fp32_grad_acc=grad_acc > 1)
        strat = oracle.strategy_ledger(P, N, eb, 12)
        assert p.ledger_ddp_bytes == pytest.approx(led["ddp"], rel=1e-12)
        assert p.ledger_zero1_bytes == pytest.approx(led["zero1"], rel=1e-12)
        assert p.ledger_zero2_bytes == pytest.approx(led["zero2"], rel=1e-12)
        assert p.ledger_ideal_bytes == pytest.approx(led["zero3"], rel=1e-12)
        assert p.comm_full_shard_bytes == pytest.approx(strat["FULL_SHARD"]["comm"], rel=1e-12, abs=1e-9)
        assert p.comm_shard_grad_op_bytes == pytest.approx(strat["SHARD_GRAD_OP"]["comm"], rel=1e-12, abs=1e-9)
        if grad_acc == 1:
            assert p.peak_full_shard_bytes == pytest.approx(strat["FULL_SHARD"]["peak"], rel=1e-12)


def test_seven_b_strategy_table_from_plans():
    """The 7B model at N = 8 through the plans, with the pages' 8 B/param
    optimizer convention of the strategy table restored (bopt 12 -> 8 moves
    every sharded figure by 4P/N and the replicated one by 4P): the FULL_SHARD
    communication and the replica sizes scale from the page's 7e9 to this
    model's P exactly."""
    groups = synth.llama_model_groups(32, 4096, 11008)
    plans = [fs.fs_plan(g, "bf16", 8, False, "fsdp2", 1) for g in groups]
    P = sum(p.total_numel for p in plans)
    comm = sum(p.comm_full_shard_bytes for p in plans)
    assert comm == pytest.approx(36.75e9 * P / 7e9, rel=1e-12)
    ddp_bopt8 = sum(p.ledger_ddp_bytes for p in plans) - 4 * P
    assert ddp_bopt8 == pytest.approx(84e9 * P / 7e9, rel=1e-12)


def test_reshard_plan_validation():
    L = fs.lib()
    a = fs.fs_plan([(3,), (5,)], "bf16", 4, True, "fsdp1")
    b = fs.fs_plan([(3,), (6,)], "bf16", 2, False, "fsdp2")
    c = fs.fs_plan([(3,), (5,)], "fp32", 2, False, "fsdp2")
    d = fs.fs_plan([(3,)], "bf16", 2, False, "fsdp2")
    h = ctypes.c_void_p()
    assert L.fs_reshard_plan(a._h, b._h, ctypes.byref(h)) == fs.FS_E_INVAL
    assert L.fs_reshard_plan(a._h, c._h, ctypes.byref(h)) == fs.FS_E_DTYPE
    assert L.fs_reshard_plan(a._h, d._h, ctypes.byref(h)) == fs.FS_E_INVAL
    assert L.fs_reshard_plan(None, a._h, ctypes.byref(h)) == fs.FS_E_INVAL
    r = fs.fs_reshard_plan(a, fs.fs_plan([(3,), (5,)], "bf16", 3, False, "fsdp2"))
    assert r.n_segments >= 2 and r.workspace_bytes >= 256
    assert L.fs_reshard(r._h, ctypes.c_void_p(16), ctypes.c_void_p(1 << 20), None) == fs.FS_E_INVAL  # not uploaded
    # identical layouts collapse to one segment per parameter run
    same = fs.fs_reshard_plan(fs.fs_plan([(40,), (24,)], "bf16", 8, False, "fsdp1"),
                              fs.fs_plan([(40,), (24,)], "bf16", 8, False, "fsdp1"))
    assert same.n_segments == 1


def test_planner_is_thread_safe_and_errors_are_per_thread():
    """Plans made concurrently from 8 threads (ctypes releases the GIL during
    the C call) match the oracle, and each thread's fs_last_error names its
    own failure."""
    import threading
    L = fs.lib()
    errors, failures = {}, []
    barrier = threading.Barrier(8)

    def work(tid):
        try:
            barrier.wait()
            for rep in range(20):
                shapes = [((tid * 7 + rep * 3 + k) % 13 + 1, (k % 3) + 1) for k in range(5)]
                N = 1 + (tid + rep) % 8
                _compare("fsdp2", shapes, 2, N, False)
                _compare("fsdp1", [(int(np.prod(s)),) for s in shapes], 4, N, bool(rep & 1))
            h = ctypes.c_void_p()
            nd = (ctypes.c_int32 * 1)(1)
            dm = (ctypes.c_int64 * 1)(5)
            if tid % 2:
                rc = L.fs_plan(1, nd, dm, 0, 0, 0, 1, 1, ctypes.byref(h))       # world < 1
            else:
                rc = L.fs_plan(1, nd, dm, 0, 4, 1, 2, 1, ctypes.byref(h))       # use_orig_params in FSDP2
            barrier.wait()      # every thread has failed before any reads its message
            errors[tid] = (rc, L.fs_last_error().decode())
        except Exception as e:  # noqa: BLE001 -- reported below
            failures.append((tid, repr(e)))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not failures, failures
    for tid, (rc, msg) in errors.items():
        if tid % 2:
            assert rc == fs.FS_E_INVAL and "world" in msg, (tid, msg)
        else:
            assert rc == fs.FS_E_UNSUPPORTED and "use_orig_params" in msg, (tid, msg)


# ------------------------------------------------------ randomized planner --

from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

_dims = st.integers(min_value=0, max_value=97)
_shape = st.one_of(st.tuples(), st.tuples(_dims), st.tuples(_dims, st.integers(1, 9)),
                   st.tuples(_dims, st.integers(1, 5), st.integers(1, 3)))


@settings(max_examples=300, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(shapes=st.lists(_shape, min_size=0, max_size=12), N=st.integers(1, 64),
       eb=st.sampled_from([2, 4]), uo=st.booleans(), mode=st.sampled_from(["fsdp1", "fsdp2"]))
def test_planner_matches_oracle_randomized(shapes, N, eb, uo, mode):
    """Random parameter lists (scalars, empty and 1- to 3-D shapes) and N up
    to 64: the library's plan places every element where the oracle does."""
    _compare(mode, shapes, eb, N, uo and mode == "fsdp1")


def test_bench_launch_spans_match_the_library():
    """bench.py's launch-count arithmetic mirrors the library's span constants."""
    import re
    import bench
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "fsdp_sharded_state_amd", "csrc", "fs_kernels.hip")).read()
    def span(name):
        m = re.search(r"constexpr int64_t %s = (\d+)ll << (\d+);" % name, src)
        assert m, name
        return int(m.group(1)) << int(m.group(2))
    assert bench.LAUNCH_SPAN["reduce"] == span("kSpan")
    assert bench.LAUNCH_SPAN["reduce_adamw_fused"] == span("kSpan")
    assert bench.LAUNCH_SPAN["reduce_bf16_reduce_dtype"] == span("kRsSpan")
    assert bench.LAUNCH_SPAN["adamw"] == span("kAdamSpan")
    S = 842_301_440
    assert bench.launches_per_call("reduce", S, 32, 8) == 26
    assert bench.launches_per_call("reduce", S, 40, 8) == 52
    assert bench.launches_per_call("reduce_bf16_reduce_dtype", S, 32, 8) == 51
    assert bench.launches_per_call("adamw", S) == 13


@pytest.mark.parametrize("kind,uo", [("fsdp1", True), ("fsdp1", False), ("fsdp2", False)])
def test_plan_twin_keeps_element_positions(kind, uo):
    """fs_plan_twin: the twin places every element where the plan does (equal to
    the oracle's layout of the plan's dtype), with the other element size; for
    FSDP2 and FSDP1 without use_orig_params it equals the plan made directly
    with that dtype, and with use_orig_params it does not (the alignment
    follows the parameter dtype)."""
    shapes = [(6, 3), (9,), (1, 1), (13, 5), (0, 2), (33, 16), (7,)]
    for N in (1, 3, 4, 8):
        P = fs.fs_plan(shapes, "bf16", N, uo, kind, 2)
        T = P.twin("fp32")
        assert T.info.elem_bytes == 4 and T.info.dtype == fs.FS_FP32
        for f in ("mode", "world", "use_orig_params", "grad_acc", "n_params", "total_numel", "flat_numel",
                  "shard_numel", "gathered_numel", "align_pad", "tail_pad", "n_segments"):
            assert getattr(T.info, f) == getattr(P.info, f), f
        assert T.segments() == P.segments()
        L = _oracle_layout(kind, shapes, 2, N, uo)
        np.testing.assert_array_equal(_plan_index_map(T), L.with_elem_bytes(4).index_map())
        D = fs.fs_plan(shapes, "fp32", N, uo, kind, 2)
        if kind == "fsdp1" and uo:
            assert D.segments() != T.segments()
        else:
            assert D.segments() == T.segments()
            assert D.info.workspace_bytes == T.info.workspace_bytes
            assert abs(D.info.ledger_ideal_bytes - T.info.ledger_ideal_bytes) < 1e-6
        back = T.twin("bf16")
        assert back.segments() == P.segments() and back.info.workspace_bytes == P.info.workspace_bytes
    L = fs.lib()
    assert L.fs_plan_twin(None, fs.FS_FP32, ctypes.byref(ctypes.c_void_p())) == fs.FS_E_INVAL
    assert L.fs_plan_twin(P._h, 7, ctypes.byref(ctypes.c_void_p())) == fs.FS_E_DTYPE
