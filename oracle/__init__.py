"""CPU oracle for the per-rank state-sharding engine.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this package.  It shares no
code with the HIP library (``fsdp_sharded_state_amd``); neither imports the
other.  The arithmetic lives in plain C loops (``fs_oracle.c``, built with
gcc, no fast-math, no FMA contraction); this module only marshals numpy arrays
into those loops, plus the memory ledger, which is plain arithmetic.

Sources, cited by page title and section:
  "FSDP1 vs FSDP2" -- section 01 (per-rank ledger), section 03 (layouts),
      the strategy ledger table (FULL_SHARD / SHARD_GRAD_OP / NO_SHARD),
      Table 3 (worked example).
  "Data parallelism, ZeRO and FSDP" -- sections 1, 2.1, 5, 9 and 9.4.
  "ZeRO/FSDP explainer" (AI infra KB M036) -- sections 03 (7B, 8 cards), 04.

The C source builds twice: liboracle.so (single-threaded, what every check
uses) and liboracle_omp.so (the same loops under OpenMP, used only to time
the oracle on all host cores; pass parallel=True).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, replace
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fs_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_LIB_OMP = os.path.join(_HERE, "liboracle_omp.so")

# gcc flags: each C operator is one IEEE operation (no contraction into FMA,
# no fast-math reassociation), so the loops compute exactly what they say.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile fs_oracle.c with gcc (host only) into liboracle.so and, with
    -fopenmp, into liboracle_omp.so."""
    for path, extra in ((_LIB, []), (_LIB_OMP, ["-fopenmp"])):
        if force or not os.path.exists(path):
            tmp = path + ".tmp"
            subprocess.run(["gcc", *CFLAGS, *extra, _SRC, "-o", tmp, "-lm"], check=True)
            os.replace(tmp, path)
    return _LIB


_libs = {}


def lib(parallel: bool = False) -> ctypes.CDLL:
    """The single-threaded oracle library, or (parallel=True) its OpenMP build."""
    if parallel not in _libs:
        path = _LIB_OMP if parallel else _LIB
        if not os.path.exists(path):
            build(force=False)
        L = ctypes.CDLL(path)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        f32 = ctypes.c_float
        L.oracle_fsdp1_layout.argtypes = [i32, vp, i32, i32, i32, vp, vp, vp]
        L.oracle_fsdp1_layout.restype = ctypes.c_int
        L.oracle_fsdp2_layout.argtypes = [i32, vp, vp, i32, vp, vp, vp]
        L.oracle_fsdp2_layout.restype = ctypes.c_int
        L.oracle_index_map.argtypes = [vp, vp]
        L.oracle_index_map.restype = None
        L.oracle_index_at.argtypes = [vp, i64, vp, vp, vp]
        L.oracle_index_at.restype = None
        L.oracle_pack.argtypes = [vp, vp, vp, i32]
        L.oracle_pack.restype = None
        L.oracle_unpack.argtypes = [vp, vp, vp]
        L.oracle_unpack.restype = None
        L.oracle_bf16_round.argtypes = [f32]
        L.oracle_bf16_round.restype = ctypes.c_uint16
        L.oracle_bf16_round_array.argtypes = [i64, vp, vp]
        L.oracle_bf16_round_array.restype = None
        L.oracle_reduce.argtypes = [i64, i32, i32, vp, vp]
        L.oracle_reduce.restype = None
        L.oracle_reduce_bf16rs.argtypes = [i64, i32, i32, vp, vp]
        L.oracle_reduce_bf16rs.restype = None
        L.oracle_reshard.argtypes = [vp, vp, vp, vp]
        L.oracle_reshard.restype = None
        L.oracle_pack_cast.argtypes = [vp, vp, vp, i32]
        L.oracle_pack_cast.restype = None
        L.oracle_adamw.argtypes = [i64, vp, vp, vp, vp, i32, vp,
                                   f32, f32, f32, f32, f32, i64]
        L.oracle_adamw.restype = None
        L.oracle_threads.argtypes = []
        L.oracle_threads.restype = ctypes.c_int
        _libs[parallel] = L
    return _libs[parallel]


def threads(parallel: bool = False) -> int:
    """Threads the element loops of that build use."""
    return int(lib(parallel).oracle_threads())


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# --------------------------------------------------------------------------
# Layouts
# --------------------------------------------------------------------------

FSDP1 = 1
FSDP2 = 2


class _CLayout(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("n_params", ctypes.c_int32),
                ("world", ctypes.c_int32), ("elem_bytes", ctypes.c_int32),
                ("shard", ctypes.c_int64),
                ("numel", ctypes.c_void_p), ("start", ctypes.c_void_p),
                ("chunk_rows", ctypes.c_void_p), ("row", ctypes.c_void_p),
                ("pre", ctypes.c_void_p)]


def _numel(shape: Sequence[int]) -> int:
    n = 1
    for d in shape:
        n *= int(d)
    return n


@dataclass
class Layout:
    """A planned layout: which gathered-buffer index each element occupies.

    mode: FSDP1 or FSDP2; shard: elements per rank (c or T); world: N.
    FSDP1 fills `start` and `flat_len`; FSDP2 fills chunk_rows / row / pre.
    """
    mode: int
    world: int
    elem_bytes: int
    numel: np.ndarray
    shard: int
    flat_len: int = 0
    start: Optional[np.ndarray] = None
    chunk_rows: Optional[np.ndarray] = None
    row: Optional[np.ndarray] = None
    pre: Optional[np.ndarray] = None

    @property
    def n_params(self) -> int:
        return len(self.numel)

    @property
    def gathered_numel(self) -> int:
        return self.world * self.shard

    def _c(self) -> _CLayout:
        z = np.zeros(max(1, self.n_params), np.int64)
        self._keep = [np.ascontiguousarray(x if x is not None else z)
                      for x in (self.numel, self.start, self.chunk_rows,
                                self.row, self.pre)]
        k = self._keep
        return _CLayout(self.mode, self.n_params, self.world, self.elem_bytes,
                        self.shard, _ptr(k[0]), _ptr(k[1]), _ptr(k[2]),
                        _ptr(k[3]), _ptr(k[4]))

    def with_elem_bytes(self, elem_bytes: int) -> "Layout":
        """The same element positions holding elements of `elem_bytes` bytes:
        the layout of state kept element for element beside the parameters
        (the fp32 master, m and v of bf16 parameters, "Data parallelism, ZeRO
        and FSDP" sections 1 and 9.1).  Only the copies change."""
        assert elem_bytes in (2, 4)
        return replace(self, elem_bytes=elem_bytes)

    def index_map(self) -> np.ndarray:
        """Gathered index of every parameter element, parameters in order."""
        out = np.empty(int(self.numel.sum()), np.int64)
        c = self._c()
        lib().oracle_index_map(ctypes.byref(c), _ptr(out))
        return out


    def index_at(self, param: np.ndarray, elem: np.ndarray) -> np.ndarray:
        """Gathered index of element elem[k] of parameter param[k]."""
        param = np.ascontiguousarray(param, np.int32)
        elem = np.ascontiguousarray(elem, np.int64)
        assert ((elem >= 0) & (elem < self.numel[param])).all()
        out = np.empty(max(1, param.size), np.int64)
        c = self._c()
        lib().oracle_index_at(ctypes.byref(c), param.size, _ptr(param), _ptr(elem), _ptr(out))
        return out[:param.size]


def fsdp1_layout(shapes: Sequence[Sequence[int]], elem_bytes: int, world: int,
                 use_orig_params: bool) -> Layout:
    """FSDP1 FlatParameter layout ["FSDP1 vs FSDP2", section 03 and Table 3]."""
    numel = np.array([_numel(s) for s in shapes], np.int64)
    n = len(numel)
    start = np.zeros(max(1, n), np.int64)
    flat_len = np.zeros(1, np.int64)
    shard = np.zeros(1, np.int64)
    rc = lib().oracle_fsdp1_layout(n, _ptr(numel) if n else None, elem_bytes,
                                   world, int(bool(use_orig_params)),
                                   _ptr(start), _ptr(flat_len), _ptr(shard))
    if rc != 0:
        raise ValueError("invalid FSDP1 layout arguments")
    return Layout(FSDP1, world, elem_bytes, numel, int(shard[0]),
                  flat_len=int(flat_len[0]), start=start[:n])


def fsdp2_layout(shapes: Sequence[Sequence[int]], elem_bytes: int,
                 world: int) -> Layout:
    """FSDP2 per-parameter dim-0 layout ["FSDP1 vs FSDP2", section 03 and Table 3].

    A 0-d parameter is taken as shape [1]; row = product of dims 1.."""
    d0 = np.array([int(s[0]) if len(s) else 1 for s in shapes], np.int64)
    row = np.array([_numel(s[1:]) if len(s) else 1 for s in shapes], np.int64)
    numel = d0 * row
    n = len(d0)
    cr = np.zeros(max(1, n), np.int64)
    pre = np.zeros(max(1, n), np.int64)
    shard = np.zeros(1, np.int64)
    rc = lib().oracle_fsdp2_layout(n, _ptr(d0) if n else None,
                                   _ptr(row) if n else None, world,
                                   _ptr(cr), _ptr(pre), _ptr(shard))
    if rc != 0:
        raise ValueError("invalid FSDP2 layout arguments")
    return Layout(FSDP2, world, elem_bytes, numel, int(shard[0]),
                  chunk_rows=cr[:n], row=row, pre=pre[:n])


def pack(layout: Layout, params: Sequence[np.ndarray], rank: int = -1, parallel: bool = False) -> np.ndarray:
    """All-gather copy-in.  params: 1-D arrays of the layout's element size
    (uint16 for bf16 bits, uint32/float32 for fp32).  Returns the gathered
    buffer (rank < 0) or rank's shard, same dtype as the params."""
    dt = np.uint16 if layout.elem_bytes == 2 else np.uint32
    ps = [np.ascontiguousarray(p).view(dt).reshape(-1) for p in params]
    for p, n in zip(ps, layout.numel):
        assert p.size == n
    size = layout.shard if rank >= 0 else layout.gathered_numel
    out = np.empty(max(1, size), dt)
    ptrs = (ctypes.c_void_p * max(1, len(ps)))(*[_ptr(p) for p in ps])
    c = layout._c()
    lib(parallel).oracle_pack(ctypes.byref(c), ptrs, _ptr(out), int(rank))
    return out[:size]


def pack_cast(layout: Layout, params: Sequence[np.ndarray], rank: int = -1) -> np.ndarray:
    """Copy-in with the fp32 -> bf16 parameter cast.  layout: a bf16 layout;
    params: float32 arrays.  Returns bf16 bits (uint16)."""
    assert layout.elem_bytes == 2
    ps = [np.ascontiguousarray(p, np.float32).reshape(-1) for p in params]
    for p, n in zip(ps, layout.numel):
        assert p.size == n
    size = layout.shard if rank >= 0 else layout.gathered_numel
    out = np.empty(max(1, size), np.uint16)
    ptrs = (ctypes.c_void_p * max(1, len(ps)))(*[_ptr(p) for p in ps])
    c = layout._c()
    lib().oracle_pack_cast(ctypes.byref(c), ptrs, _ptr(out), int(rank))
    return out[:size]


def reshard(src_layout: Layout, dst_layout: Layout, gathered: np.ndarray) -> np.ndarray:
    """Move a gathered buffer from src_layout to dst_layout (same parameters,
    same element size); dst pads are zero."""
    assert src_layout.elem_bytes == dst_layout.elem_bytes
    assert list(src_layout.numel) == list(dst_layout.numel)
    dt = np.uint16 if src_layout.elem_bytes == 2 else np.uint32
    g = np.ascontiguousarray(gathered).view(dt).reshape(-1)
    assert g.size == src_layout.gathered_numel
    out = np.empty(max(1, dst_layout.gathered_numel), dt)
    cs, cd = src_layout._c(), dst_layout._c()
    keep = (src_layout._keep, dst_layout._keep)   # noqa: F841 (arrays behind the structs)
    gsrc = g if g.size else np.zeros(1, dt)
    lib().oracle_reshard(ctypes.byref(cs), ctypes.byref(cd), _ptr(gsrc), _ptr(out))
    return out[:dst_layout.gathered_numel]


def unpack(layout: Layout, gathered: np.ndarray, parallel: bool = False) -> List[np.ndarray]:
    """All-gather copy-out: per-parameter 1-D arrays from a gathered buffer."""
    dt = np.uint16 if layout.elem_bytes == 2 else np.uint32
    g = np.ascontiguousarray(gathered).view(dt).reshape(-1)
    assert g.size == layout.gathered_numel
    outs = [np.empty(max(1, int(n)), dt) for n in layout.numel]
    ptrs = (ctypes.c_void_p * max(1, len(outs)))(*[_ptr(o) for o in outs])
    c = layout._c()
    lib(parallel).oracle_unpack(ctypes.byref(c), _ptr(g) if g.size else _ptr(np.zeros(1, dt)), ptrs)
    return [o[:int(n)] for o, n in zip(outs, layout.numel)]


# --------------------------------------------------------------------------
# Reduce and AdamW
# --------------------------------------------------------------------------

def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, np.float32).reshape(-1)
    out = np.empty(max(1, x.size), np.uint16)
    lib().oracle_bf16_round_array(x.size, _ptr(x), _ptr(out))
    return out[:x.size]


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits (uint16) to float32."""
    b = np.ascontiguousarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def reduce_shard(slices: Sequence[np.ndarray], world: int, grad_acc: int, parallel: bool = False) -> np.ndarray:
    """Average slices[j*world + k] (bf16 bits, uint16) into an fp32 shard
    ["Data parallelism, ZeRO and FSDP", sections 2.1, 5 and 9.2]."""
    assert len(slices) == world * grad_acc
    ss = [np.ascontiguousarray(s, np.uint16).reshape(-1) for s in slices]
    n = ss[0].size
    assert all(s.size == n for s in ss)
    out = np.empty(max(1, n), np.float32)
    ptrs = (ctypes.c_void_p * len(ss))(*[_ptr(s) for s in ss])
    lib(parallel).oracle_reduce(n, world, grad_acc, ptrs, _ptr(out))
    return out[:n]


def reduce_shard_bf16rs(slices: Sequence[np.ndarray], world: int, grad_acc: int) -> np.ndarray:
    """Average with a bf16 reduce dtype: each micro-step's N-way average is
    delivered as bf16, then accumulated in fp32 ["FSDP1 vs FSDP2", mixed
    precision; "Data parallelism, ZeRO and FSDP", section 9.2]."""
    assert len(slices) == world * grad_acc
    ss = [np.ascontiguousarray(s, np.uint16).reshape(-1) for s in slices]
    n = ss[0].size
    assert all(s.size == n for s in ss)
    out = np.empty(max(1, n), np.float32)
    ptrs = (ctypes.c_void_p * len(ss))(*[_ptr(s) for s in ss])
    lib().oracle_reduce_bf16rs(n, world, grad_acc, ptrs, _ptr(out))
    return out[:n]


@dataclass
class AdamWHparams:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    step: int = 1


def adamw_step(master: np.ndarray, exp_avg: np.ndarray, exp_avg_sq: np.ndarray,
               grad: np.ndarray, hp: AdamWHparams, want_bf16: bool = True, parallel: bool = False):
    """One AdamW step ["Data parallelism, ZeRO and FSDP", sections 1 and 9.1;
    "ZeRO/FSDP explainer", section 04].

    Returns new copies (master, exp_avg, exp_avg_sq, param_bf16 or None); the
    inputs are not modified.  grad: float32 array, or uint16 bf16 bits."""
    th = np.array(master, np.float32, copy=True).reshape(-1)
    m = np.array(exp_avg, np.float32, copy=True).reshape(-1)
    v = np.array(exp_avg_sq, np.float32, copy=True).reshape(-1)
    g = np.ascontiguousarray(grad).reshape(-1)
    is_bf16 = g.dtype == np.uint16
    if not is_bf16:
        g = g.astype(np.float32, copy=False)
    n = th.size
    assert m.size == n and v.size == n and g.size == n
    p16 = np.empty(max(1, n), np.uint16) if want_bf16 else None
    dummy = np.zeros(1, np.float32)
    lib(parallel).oracle_adamw(n, _ptr(th) if n else _ptr(dummy), _ptr(m) if n else _ptr(dummy),
                       _ptr(v) if n else _ptr(dummy), _ptr(g) if n else _ptr(dummy),
                       int(is_bf16), _ptr(p16) if want_bf16 else None,
                       hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay,
                       int(hp.step))
    return th, m, v, (p16[:n] if want_bf16 else None)


# --------------------------------------------------------------------------
# Memory ledger (plain arithmetic)
# --------------------------------------------------------------------------

GB = 1e9  # the pages count decimal GB ("FSDP1 vs FSDP2", section 01 calculator)


def ledger(P: float, N: int, b: float, bopt: float, fp32_grad_acc: bool = False) -> dict:
    """Per-rank resident bytes of each scheme ["FSDP1 vs FSDP2", section 01
    table; "Data parallelism, ZeRO and FSDP", section 9; "ZeRO/FSDP
    explainer", section 03].

    P parameters, N data-parallel ranks, b bytes per parameter and per
    gradient, bopt optimizer bytes per parameter.  With fp32 gradient
    accumulation the gradient term grows by 4 bytes per parameter on the
    part each scheme keeps of the gradient ("Data parallelism, ZeRO and FSDP",
    section 9)."""
    acc = 4.0 if fp32_grad_acc else 0.0
    return {
        "ddp": P * (2 * b + bopt) + acc * P,
        "zero1": 2 * P * b + P * bopt / N + acc * P,
        "zero2": P * b + P * (b + bopt) / N + acc * P / N,
        "zero3": P * (2 * b + bopt) / N + acc * P / N,
    }


def strategy_ledger(P: float, N: int, b: float, bopt: float) -> dict:
    """FSDP1 strategy table ["FSDP1 vs FSDP2", strategy ledger]: resident, worst-case peak
    (resident plus one full parameter copy while it is gathered) and
    communication bytes per iteration per card (3P(N-1)/N elements for
    FULL_SHARD, 2P(N-1)/N for SHARD_GRAD_OP and NO_SHARD)."""
    sharded = P * (2 * b + bopt) / N
    full = P * (2 * b + bopt)
    frac = (N - 1) / N
    return {
        "FULL_SHARD": {"resident": sharded, "peak": sharded + P * b,
                       "comm": 3 * P * frac * b},
        "SHARD_GRAD_OP": {"resident": sharded, "peak": sharded + P * b,
                          "comm": 2 * P * frac * b},
        "NO_SHARD": {"resident": full, "peak": full, "comm": 2 * P * frac * b},
    }
