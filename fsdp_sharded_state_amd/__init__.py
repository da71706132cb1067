"""Python binding of the per-rank state-sharding engine (libfsstate.so).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in include/fs.h.  torch supplies device memory and
streams.  There is no fallback: if the library is missing, importing its
functions raises.

    plan = fs_plan(shapes, "bf16", world=8, mode="fsdp2")
    plan.upload()                         # segment/tile tables -> device
    fs_pack(plan, params, gathered)       # all-gather copy-in (all N ranks)
    fs_unpack(plan, gathered, outs)       # all-gather copy-out
    fs_reduce_shard(slices, grad32, world=8, grad_acc=4)
    fs_adamw_step(master, m, v, grad32, p16, lr=1e-3, step=1)
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfsstate.so")

FS_OK = 0
FS_E_INVAL, FS_E_UNSUPPORTED, FS_E_DTYPE, FS_E_OVERFLOW, FS_E_ALIGN, FS_E_HIP, FS_E_NOMEM = range(-1, -8, -1)
_CODES = {0: "FS_OK", -1: "FS_E_INVAL", -2: "FS_E_UNSUPPORTED", -3: "FS_E_DTYPE",
          -4: "FS_E_OVERFLOW", -5: "FS_E_ALIGN", -6: "FS_E_HIP", -7: "FS_E_NOMEM"}
FS_BF16, FS_FP32 = 0, 1
NOALLOC_MAX_NUMEL = 16777216   # scratch capacity of fs_reduce_adamw_step_noalloc (fp32 elements)
FS_FSDP1_FLAT, FS_FSDP2_PER_PARAM = 1, 2


class FsError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_CODES.get(code, code)}: {msg}")
        self.code = code


class PlanInfo(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("dtype", ctypes.c_int32), ("world", ctypes.c_int32),
                ("use_orig_params", ctypes.c_int32), ("grad_acc", ctypes.c_int32),
                ("n_params", ctypes.c_int32), ("elem_bytes", ctypes.c_int32), ("bopt", ctypes.c_int32),
                ("total_numel", ctypes.c_int64), ("flat_numel", ctypes.c_int64),
                ("shard_numel", ctypes.c_int64), ("gathered_numel", ctypes.c_int64),
                ("align_pad", ctypes.c_int64), ("tail_pad", ctypes.c_int64),
                ("n_segments", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("ledger_ideal_bytes", ctypes.c_double), ("ledger_padded_bytes", ctypes.c_double),
                ("ledger_ddp_bytes", ctypes.c_double), ("ledger_zero1_bytes", ctypes.c_double),
                ("ledger_zero2_bytes", ctypes.c_double), ("peak_full_shard_bytes", ctypes.c_double),
                ("comm_full_shard_bytes", ctypes.c_double), ("comm_shard_grad_op_bytes", ctypes.c_double)]


class Segment(ctypes.Structure):
    _fields_ = [("dst_off", ctypes.c_int64), ("src_off", ctypes.c_int64), ("len", ctypes.c_int64),
                ("param", ctypes.c_int32), ("rank", ctypes.c_int32)]


class ParamLayout(ctypes.Structure):
    _fields_ = [("numel", ctypes.c_int64), ("start", ctypes.c_int64), ("chunk_rows", ctypes.c_int64),
                ("row", ctypes.c_int64), ("pre", ctypes.c_int64)]


class AdamWHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("reserved", ctypes.c_int32),
                ("step", ctypes.c_int64)]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libfsstate.so (built by `python -m fsdp_sharded_state_amd.build`)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m fsdp_sharded_state_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    L.fs_plan.argtypes = [i32, vp, vp, i32, i32, i32, i32, i32, ctypes.POINTER(vp)]
    L.fs_plan_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    L.fs_plan_param.argtypes = [vp, i32, ctypes.POINTER(ParamLayout)]
    L.fs_plan_segments.argtypes = [vp, vp, i64, ctypes.POINTER(i64)]
    L.fs_plan_upload.argtypes = [vp, vp, sz, vp]
    L.fs_plan_destroy.argtypes = [vp]
    L.fs_plan_destroy.restype = None
    L.fs_plan_twin.argtypes = [vp, i32, ctypes.POINTER(vp)]
    L.fs_pack.argtypes = [vp, vp, vp, i32, vp]
    L.fs_unpack.argtypes = [vp, vp, vp, vp]
    L.fs_reduce_shard.argtypes = [i64, i32, i32, vp, vp, vp]
    L.fs_adamw_step.argtypes = [i64, vp, vp, vp, vp, i32, vp, ctypes.POINTER(AdamWHparams), vp]
    L.fs_reshard_plan.argtypes = [vp, vp, ctypes.POINTER(vp)]
    L.fs_reshard_info.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.fs_reshard_upload.argtypes = [vp, vp, sz, vp]
    L.fs_reshard.argtypes = [vp, vp, vp, vp]
    L.fs_reshard_destroy.argtypes = [vp]
    L.fs_reshard_destroy.restype = None
    L.fs_reduce_shard_ex.argtypes = [i64, i32, i32, i32, vp, vp, vp]
    L.fs_pack_cast.argtypes = [vp, vp, i32, vp, i32, vp]
    L.fs_load_local.argtypes = [vp, i32, vp, vp, vp]
    L.fs_reduce_adamw_step_noalloc.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp, ctypes.POINTER(AdamWHparams), vp]
    L.fs_reduce_adamw_step.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp, vp, ctypes.POINTER(AdamWHparams), vp]
    L.fs_copy_bytes.argtypes = [vp, vp, i64, vp]
    L.fs_stream_read.argtypes = [vp, i64, vp, vp]
    L.fs_stream_fill.argtypes = [vp, i64, ctypes.c_uint32, vp]
    L.fs_last_error.argtypes = []
    L.fs_last_error.restype = ctypes.c_char_p
    for name in ("fs_plan", "fs_plan_twin", "fs_plan_info", "fs_plan_param", "fs_plan_segments", "fs_plan_upload",
                 "fs_pack", "fs_unpack", "fs_reduce_shard", "fs_adamw_step", "fs_reduce_adamw_step",
                 "fs_reduce_shard_ex", "fs_pack_cast", "fs_reshard_plan", "fs_reshard_info",
                 "fs_reshard_upload", "fs_reshard", "fs_load_local", "fs_reduce_adamw_step_noalloc",
                 "fs_copy_bytes", "fs_stream_read", "fs_stream_fill"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int):
    if rc != FS_OK:
        raise FsError(rc, lib().fs_last_error().decode())


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(dtype) -> int:
    if dtype in ("bf16", torch.bfloat16, FS_BF16):
        return FS_BF16
    if dtype in ("fp32", torch.float32, FS_FP32):
        return FS_FP32
    raise ValueError(f"unsupported dtype {dtype!r}")


def _mode_code(mode) -> int:
    if mode in ("fsdp1", FS_FSDP1_FLAT):
        return FS_FSDP1_FLAT
    if mode in ("fsdp2", FS_FSDP2_PER_PARAM):
        return FS_FSDP2_PER_PARAM
    raise ValueError(f"unsupported mode {mode!r}")


def _dev_ptr(t: torch.Tensor, what: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


class Plan:
    """An uploaded-or-not layout plan (wraps fs_plan_t)."""

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)
        self._destroy = lib().fs_plan_destroy   # kept for interpreter shutdown
        info = PlanInfo()
        _check(lib().fs_plan_info(self._h, ctypes.byref(info)))
        self.info = info
        self.workspace: Optional[torch.Tensor] = None
        self._ptr_cache = {}
        self._pinned = set()        # pointer-table keys a captured graph or another stream may still read
        self._pieces = {}           # rank -> local piece element counts
        self.numels = [self.param(i).numel for i in range(info.n_params)]
        self.shapes: Optional[List[tuple]] = None   # set by fs_plan()

    def close(self):
        """Release the plan's host memory (also done on garbage collection)."""
        h = self.__dict__.pop("_h", None)
        if h is not None and h.value:
            self._destroy(h)

    def __del__(self):
        self.close()

    # summary
    def __getattr__(self, name):
        info = self.__dict__.get("info")
        if info is not None and name in dict(PlanInfo._fields_):
            return getattr(info, name)
        raise AttributeError(name)

    def param(self, i: int) -> ParamLayout:
        out = ParamLayout()
        _check(lib().fs_plan_param(self._h, i, ctypes.byref(out)))
        return out

    def segments(self) -> List[tuple]:
        n = ctypes.c_int64()
        _check(lib().fs_plan_segments(self._h, None, 0, ctypes.byref(n)))
        arr = (Segment * max(1, n.value))()
        _check(lib().fs_plan_segments(self._h, arr, n.value, ctypes.byref(n)))
        return [(s.dst_off, s.src_off, s.len, s.param, s.rank) for s in arr[:n.value]]

    def local_pieces(self, rank: int) -> List[Optional[tuple]]:
        """Where each parameter's elements held by `rank` sit: per parameter,
        (offset in the rank's shard, first element of the flattened
        parameter, count), or None when the rank holds none of it.  A
        parameter's elements on one rank are always one contiguous run, in
        both layouts."""
        if not 0 <= rank < self.info.world:
            raise ValueError(f"rank {rank} out of range [0, {self.info.world})")
        c = self.info.shard_numel
        out: List[Optional[tuple]] = [None] * self.info.n_params
        for dst, src, ln, p, r in self.segments():
            if r == rank:
                if out[p] is not None:
                    raise RuntimeError(f"parameter {p} has two runs on rank {rank}")
                out[p] = (dst - r * c, src, ln)
        return out

    def twin(self, dtype) -> "Plan":
        """The plan of `dtype` elements at this plan's element positions
        (fs_plan_twin): lays out the fp32 master, m and v of this plan's bf16
        parameters element for element (not uploaded)."""
        h = ctypes.c_void_p()
        _check(lib().fs_plan_twin(self._h, _dtype_code(dtype), ctypes.byref(h)))
        t = Plan(h.value)
        t.shapes = self.shapes
        return t

    def local_views(self, shard: torch.Tensor, rank: int) -> List[torch.Tensor]:
        """The sharded state dict of `rank`, zero-copy: for each parameter,
        the view of `shard` (that rank's shard buffer, shard_numel elements:
        parameters, gradients or optimizer state laid out by this plan) that
        holds the parameter's local elements.  FSDP2: shaped (rows, *shape[1:])
        -- the rank's dim-0 chunk, empty when it has no rows; FSDP1: 1-D, the
        flattened parameter's elements that fall in the rank's flat shard."""
        if shard.dim() != 1 or shard.numel() != self.info.shard_numel:
            raise ValueError(f"shard must be 1-D with {self.info.shard_numel} elements")
        if shard.element_size() != self.info.elem_bytes:
            raise ValueError(f"shard element size {shard.element_size()} != plan's {self.info.elem_bytes}")
        fsdp2 = self.info.mode == FS_FSDP2_PER_PARAM
        views = []
        for i, piece in enumerate(self.local_pieces(rank)):
            off, _, ln = piece if piece is not None else (0, 0, 0)
            v = shard[off:off + ln]
            tail = tuple(self.shapes[i][1:]) if fsdp2 and self.shapes and self.shapes[i] else ()
            row = math.prod(tail)
            views.append(v.view((ln // row,) + tail) if fsdp2 and row else v)
        return views

    def local_numels(self, rank: int) -> List[int]:
        """Element count of every parameter's local piece on `rank`."""
        if rank not in self._pieces:
            self._pieces[rank] = [0 if pc is None else pc[2] for pc in self.local_pieces(rank)]
        return self._pieces[rank]

    def load_local(self, shard: torch.Tensor, rank: int, tensors: Sequence[torch.Tensor], stream=None):
        """Import a sharded state dict (fs_load_local): write each parameter's
        local tensor (shaped as local_views returns it, or flat) into its place
        in `shard` (that rank's shard buffer on the GPU) and zero the pads."""
        if not 0 <= rank < self.info.world:
            raise ValueError(f"rank {rank} out of range [0, {self.info.world})")
        if shard.dim() != 1 or shard.numel() != self.info.shard_numel:
            raise ValueError(f"shard must be 1-D with {self.info.shard_numel} elements")
        if shard.element_size() != self.info.elem_bytes:
            raise ValueError(f"shard element size {shard.element_size()} != plan's {self.info.elem_bytes}")
        want = self.local_numels(rank)
        if len(tensors) != len(want):
            raise ValueError(f"expected {len(want)} local tensors, got {len(tensors)}")
        for i, (t, n) in enumerate(zip(tensors, want)):
            if t.numel() != n:
                raise ValueError(f"local tensor {i}: {t.numel()} elements, rank {rank} holds {n}")
        tab = self.ptr_table(tensors, "local tensors", numels=want, stream=stream)
        _check(lib().fs_load_local(self._h, int(rank), tab.data_ptr(),
                                   _dev_ptr(shard, "shard") if shard.numel() else 0, _stream(stream)))

    def upload(self, device="cuda", stream=None) -> "Plan":
        ws = torch.empty(max(16, self.info.workspace_bytes), dtype=torch.uint8, device=device)
        _check(lib().fs_plan_upload(self._h, ws.data_ptr(), ws.numel(), _stream(stream)))
        self.workspace = ws
        return self

    def ptr_table(self, tensors: Sequence[torch.Tensor], what: str, elem_bytes: Optional[int] = None,
                  numels: Optional[Sequence[int]] = None, stream=None) -> torch.Tensor:
        """Device array of the tensors' data pointers (cached per pointer set).
        Every tensor must hold `numels[i]` elements (default: its parameter's
        element count) of `elem_bytes` bytes (default: the plan's).

        The kernels read the table when they run, not when they are enqueued,
        so a table must outlive every launch that uses it.  A few recent sets
        are kept; the oldest is released when a new one is made, which is safe
        for launches on the current stream (the allocator reuses its memory in
        stream order).  A table used while a graph is being captured, or with
        a stream given as a raw handle, is pinned for the plan's lifetime; one
        used on another torch stream is recorded on that stream.  A new set
        cannot be made during capture (its upload would be a captured copy
        from host memory): run the call once before capturing."""
        if len(tensors) != self.info.n_params:
            raise ValueError(f"{what}: expected {self.info.n_params} tensors, got {len(tensors)}")
        esz = self.info.elem_bytes if elem_bytes is None else elem_bytes
        want = self.numels if numels is None else numels
        ptrs = []
        for i, t in enumerate(tensors):
            if t.element_size() != esz:
                raise ValueError(f"{what}[{i}]: element size {t.element_size()} != {esz}")
            if t.numel() != want[i]:
                raise ValueError(f"{what}[{i}]: numel {t.numel()} != {want[i]}")
            ptrs.append(_dev_ptr(t, f"{what}[{i}]") if t.numel() else 0)
        key = (tuple(ptrs), str(tensors[0].device) if tensors else "")
        capturing = torch.cuda.is_available() and torch.cuda.is_current_stream_capturing()
        tab = self._ptr_cache.get(key)
        if tab is None:
            if capturing:
                raise RuntimeError(f"{what}: a pointer set not seen before, during graph capture; run the same "
                                   "call once before capturing so that its device pointer table exists")
            dev = tensors[0].device if tensors else torch.device("cuda")
            tab = torch.tensor(ptrs or [0], dtype=torch.int64, device=dev)
            if len(self._ptr_cache) >= 8:          # keep a few pointer sets (pack and unpack sides)
                old = next((k for k in self._ptr_cache if k not in self._pinned), None)
                if old is not None:
                    self._ptr_cache.pop(old)
            self._ptr_cache[key] = tab
        if capturing:
            self._pinned.add(key)
        if stream is not None:
            if isinstance(stream, torch.cuda.Stream):
                if stream != torch.cuda.current_stream(tab.device):
                    tab.record_stream(stream)
            else:
                self._pinned.add(key)
        return tab


def fs_plan(shapes: Sequence[Sequence[int]], dtype="bf16", world: int = 1, use_orig_params: bool = False,
            mode="fsdp1", grad_acc: int = 1) -> Plan:
    """Plan one FSDP group's shard layout (fs_plan)."""
    n = len(shapes)
    ndim = (ctypes.c_int32 * max(1, n))(*[len(s) for s in shapes])
    flat = [int(d) for s in shapes for d in s]
    dims = (ctypes.c_int64 * max(1, len(flat)))(*flat)
    h = ctypes.c_void_p()
    _check(lib().fs_plan(n, ndim, dims, _dtype_code(dtype), int(world), int(bool(use_orig_params)),
                         _mode_code(mode), int(grad_acc), ctypes.byref(h)))
    plan = Plan(h.value)
    plan.shapes = [tuple(int(d) for d in s) for s in shapes]
    return plan


class Reshard:
    """Relayout plan from one group plan to another (wraps fs_reshard_t)."""

    def __init__(self, src: "Plan", dst: "Plan"):
        h = ctypes.c_void_p()
        _check(lib().fs_reshard_plan(src._h, dst._h, ctypes.byref(h)))
        self._h = h
        self._destroy = lib().fs_reshard_destroy
        self.src_info, self.dst_info = src.info, dst.info
        wb, ns = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().fs_reshard_info(h, ctypes.byref(wb), ctypes.byref(ns)))
        self.workspace_bytes, self.n_segments = wb.value, ns.value
        self.workspace: Optional[torch.Tensor] = None

    def close(self):
        h = self.__dict__.pop("_h", None)
        if h is not None and h.value:
            self._destroy(h)

    def __del__(self):
        self.close()

    def upload(self, device="cuda", stream=None) -> "Reshard":
        ws = torch.empty(max(16, self.workspace_bytes), dtype=torch.uint8, device=device)
        _check(lib().fs_reshard_upload(self._h, ws.data_ptr(), ws.numel(), _stream(stream)))
        self.workspace = ws
        return self


def fs_reshard_plan(src: "Plan", dst: "Plan") -> Reshard:
    """Plan moving a group's gathered buffer from plan src (N) to plan dst (N')."""
    return Reshard(src, dst)


def fs_reshard(r: Reshard, src_gathered: torch.Tensor, dst_gathered: torch.Tensor, stream=None):
    """dst_gathered <- src_gathered re-laid from the src plan to the dst plan."""
    if src_gathered.numel() != r.src_info.gathered_numel or dst_gathered.numel() != r.dst_info.gathered_numel:
        raise ValueError("fs_reshard: buffer sizes do not match the plans")
    _check(lib().fs_reshard(r._h, _dev_ptr(src_gathered, "src_gathered") if src_gathered.numel() else 0,
                            _dev_ptr(dst_gathered, "dst_gathered") if dst_gathered.numel() else 0,
                            _stream(stream)))


def fs_pack(plan: Plan, params: Sequence[torch.Tensor], out: torch.Tensor, rank: int = -1, stream=None):
    """All-gather copy-in: params -> out (whole gathered buffer, or rank's shard)."""
    want = plan.info.gathered_numel if rank < 0 else plan.info.shard_numel
    if out.numel() != want or out.element_size() != plan.info.elem_bytes:
        raise ValueError(f"fs_pack: out must hold {want} elements of {plan.info.elem_bytes} bytes")
    tab = plan.ptr_table(params, "params", stream=stream)
    _check(lib().fs_pack(plan._h, tab.data_ptr(), _dev_ptr(out, "out") if want else 0, int(rank), _stream(stream)))


def fs_pack_cast(plan: Plan, params: Sequence[torch.Tensor], out: torch.Tensor, rank: int = -1, stream=None):
    """Copy-in with the parameter-dtype cast: fp32 params into a bf16 plan's
    gathered buffer (or rank's shard), rounded to nearest even."""
    want = plan.info.gathered_numel if rank < 0 else plan.info.shard_numel
    if out.numel() != want or out.dtype != torch.bfloat16:
        raise ValueError(f"fs_pack_cast: out must be bfloat16 with {want} elements")
    if not params:
        raise ValueError("fs_pack_cast: no parameters")
    dt = params[0].dtype
    if any(p.dtype != dt for p in params):
        raise ValueError("fs_pack_cast: parameters must share one dtype")
    tab = plan.ptr_table(params, "params", elem_bytes=params[0].element_size(), stream=stream)
    _check(lib().fs_pack_cast(plan._h, tab.data_ptr(), _dtype_code(dt), _dev_ptr(out, "out") if want else 0,
                              int(rank), _stream(stream)))


def fs_unpack(plan: Plan, gathered: torch.Tensor, params: Sequence[torch.Tensor], stream=None):
    """All-gather copy-out: gathered -> params."""
    if gathered.numel() != plan.info.gathered_numel or gathered.element_size() != plan.info.elem_bytes:
        raise ValueError("fs_unpack: gathered has the wrong size or element size")
    tab = plan.ptr_table(params, "params", stream=stream)
    _check(lib().fs_unpack(plan._h, _dev_ptr(gathered, "gathered") if gathered.numel() else 0,
                           tab.data_ptr(), _stream(stream)))


def fs_reduce_shard(slices: Sequence[torch.Tensor], out: torch.Tensor, world: int, grad_acc: int = 1, stream=None):
    """Average slices[j*world + k] (bf16, n each) into out (fp32, n)."""
    n = out.numel()
    if out.dtype != torch.float32:
        raise ValueError("fs_reduce_shard: out must be float32")
    if len(slices) != world * grad_acc:
        raise ValueError(f"fs_reduce_shard: need world*grad_acc = {world * grad_acc} slices")
    ptrs = []
    for k, s in enumerate(slices):
        if s.dtype != torch.bfloat16 or s.numel() != n:
            raise ValueError(f"fs_reduce_shard: slice {k} must be bf16 with {n} elements")
        ptrs.append(_dev_ptr(s, f"slices[{k}]") if n else 0)
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
    _check(lib().fs_reduce_shard(n, int(world), int(grad_acc), arr, _dev_ptr(out, "out") if n else 0,
                                 _stream(stream)))


def fs_reduce_shard_ex(slices: Sequence[torch.Tensor], out: torch.Tensor, world: int, grad_acc: int = 1,
                       reduce_dtype="fp32", stream=None):
    """fs_reduce_shard with a reduce dtype: "fp32" (same as fs_reduce_shard)
    or "bf16" (each micro-step's average delivered in bf16, accumulated in fp32)."""
    n = out.numel()
    if out.dtype != torch.float32:
        raise ValueError("fs_reduce_shard_ex: out must be float32")
    if len(slices) != world * grad_acc:
        raise ValueError(f"fs_reduce_shard_ex: need world*grad_acc = {world * grad_acc} slices")
    ptrs = []
    for k, s in enumerate(slices):
        if s.dtype != torch.bfloat16 or s.numel() != n:
            raise ValueError(f"fs_reduce_shard_ex: slice {k} must be bf16 with {n} elements")
        ptrs.append(_dev_ptr(s, f"slices[{k}]") if n else 0)
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
    _check(lib().fs_reduce_shard_ex(n, int(world), int(grad_acc), _dtype_code(reduce_dtype), arr,
                                    _dev_ptr(out, "out") if n else 0, _stream(stream)))


def fs_adamw_step(master: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor, grad: torch.Tensor,
                  param_bf16: Optional[torch.Tensor] = None, *, lr: float = 1e-3, beta1: float = 0.9,
                  beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.01, step: int = 1,
                  stream=None):
    """One AdamW step over the fp32 shard (in place), writing the bf16 copy."""
    n = master.numel()
    for name, t in (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        if t.dtype != torch.float32 or t.numel() != n:
            raise ValueError(f"fs_adamw_step: {name} must be float32 with {n} elements")
    if grad.numel() != n or grad.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("fs_adamw_step: grad must be float32 or bfloat16 with n elements")
    if param_bf16 is not None and (param_bf16.dtype != torch.bfloat16 or param_bf16.numel() != n):
        raise ValueError("fs_adamw_step: param_bf16 must be bfloat16 with n elements")
    hp = AdamWHparams(lr, beta1, beta2, eps, weight_decay, 0, int(step))
    ptr = (lambda t, w: _dev_ptr(t, w) if n else 0)
    _check(lib().fs_adamw_step(n, ptr(master, "master"), ptr(exp_avg, "exp_avg"), ptr(exp_avg_sq, "exp_avg_sq"),
                               ptr(grad, "grad"), FS_BF16 if grad.dtype == torch.bfloat16 else FS_FP32,
                               ptr(param_bf16, "param_bf16") if param_bf16 is not None else None,
                               ctypes.byref(hp), _stream(stream)))


def fs_reduce_adamw_step(slices: Sequence[torch.Tensor], master: torch.Tensor, exp_avg: torch.Tensor,
                         exp_avg_sq: torch.Tensor, param_bf16: Optional[torch.Tensor] = None,
                         grad_out: Optional[torch.Tensor] = None, *, world: int, grad_acc: int = 1,
                         lr: float = 1e-3, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                         weight_decay: float = 0.01, step: int = 1, stream=None):
    """Fused reduce + AdamW: average slices[j*world + k] (bf16) and apply one
    AdamW step to the fp32 shard in place; the averaged gradient goes to
    grad_out only if given."""
    n = master.numel()
    for name, t in (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        if t.dtype != torch.float32 or t.numel() != n:
            raise ValueError(f"fs_reduce_adamw_step: {name} must be float32 with {n} elements")
    if len(slices) != world * grad_acc:
        raise ValueError(f"fs_reduce_adamw_step: need world*grad_acc = {world * grad_acc} slices")
    ptrs = []
    for k, s in enumerate(slices):
        if s.dtype != torch.bfloat16 or s.numel() != n:
            raise ValueError(f"fs_reduce_adamw_step: slice {k} must be bf16 with {n} elements")
        ptrs.append(_dev_ptr(s, f"slices[{k}]") if n else 0)
    if param_bf16 is not None and (param_bf16.dtype != torch.bfloat16 or param_bf16.numel() != n):
        raise ValueError("fs_reduce_adamw_step: param_bf16 must be bfloat16 with n elements")
    if grad_out is not None and (grad_out.dtype != torch.float32 or grad_out.numel() != n):
        raise ValueError("fs_reduce_adamw_step: grad_out must be float32 with n elements")
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
    hp = AdamWHparams(lr, beta1, beta2, eps, weight_decay, 0, int(step))
    ptr = (lambda t, w: (_dev_ptr(t, w) if n else 0) if t is not None else None)
    _check(lib().fs_reduce_adamw_step(n, int(world), int(grad_acc), arr, ptr(master, "master"),
                                      ptr(exp_avg, "exp_avg"), ptr(exp_avg_sq, "exp_avg_sq"),
                                      ptr(param_bf16, "param_bf16"), ptr(grad_out, "grad_out"),
                                      ctypes.byref(hp), _stream(stream)))


def fs_reduce_adamw_step_noalloc(slices: Sequence[torch.Tensor], master: torch.Tensor, exp_avg: torch.Tensor,
                                 exp_avg_sq: torch.Tensor, param_bf16: Optional[torch.Tensor] = None, *, world: int,
                                 grad_acc: int = 1, lr: float = 1e-3, beta1: float = 0.9, beta2: float = 0.999,
                                 eps: float = 1e-8, weight_decay: float = 0.01, step: int = 1, stream=None):
    """fs_reduce_adamw_step without grad_out, for callers that cannot
    allocate: with more than 32 terms the partial sums go to the library's
    per-GPU scratch array (at most NOALLOC_MAX_NUMEL elements)."""
    n = master.numel()
    for name, t in (("master", master), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        if t.dtype != torch.float32 or t.numel() != n:
            raise ValueError(f"fs_reduce_adamw_step_noalloc: {name} must be float32 with {n} elements")
    if len(slices) != world * grad_acc:
        raise ValueError(f"fs_reduce_adamw_step_noalloc: need world*grad_acc = {world * grad_acc} slices")
    ptrs = []
    for k, s in enumerate(slices):
        if s.dtype != torch.bfloat16 or s.numel() != n:
            raise ValueError(f"fs_reduce_adamw_step_noalloc: slice {k} must be bf16 with {n} elements")
        ptrs.append(_dev_ptr(s, f"slices[{k}]") if n else 0)
    if param_bf16 is not None and (param_bf16.dtype != torch.bfloat16 or param_bf16.numel() != n):
        raise ValueError("fs_reduce_adamw_step_noalloc: param_bf16 must be bfloat16 with n elements")
    arr = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
    hp = AdamWHparams(lr, beta1, beta2, eps, weight_decay, 0, int(step))
    ptr = (lambda t, w: (_dev_ptr(t, w) if n else 0) if t is not None else None)
    _check(lib().fs_reduce_adamw_step_noalloc(n, int(world), int(grad_acc), arr, ptr(master, "master"),
                                              ptr(exp_avg, "exp_avg"), ptr(exp_avg_sq, "exp_avg_sq"),
                                              ptr(param_bf16, "param_bf16"), ctypes.byref(hp), _stream(stream)))


def fs_copy_bytes(dst: torch.Tensor, src: torch.Tensor, stream=None):
    """Plain streaming copy (measurement aid): src -> dst, same byte size."""
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("fs_copy_bytes: size mismatch")
    _check(lib().fs_copy_bytes(_dev_ptr(dst, "dst"), _dev_ptr(src, "src"), nb, _stream(stream)))


def fs_stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None):
    """Read-only stream over src's bytes (measurement aid); sink: a device
    tensor of at least 4 bytes that may receive an unspecified value."""
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("fs_stream_read: sink needs 4 bytes")
    _check(lib().fs_stream_read(_dev_ptr(src, "src"), src.numel() * src.element_size(), _dev_ptr(sink, "sink"),
                                _stream(stream)))


def fs_stream_fill(dst: torch.Tensor, value: int, stream=None):
    """Write-only stream: every 32-bit word of dst becomes `value` (measurement aid)."""
    _check(lib().fs_stream_fill(_dev_ptr(dst, "dst"), dst.numel() * dst.element_size(), int(value) & 0xFFFFFFFF,
                                _stream(stream)))
