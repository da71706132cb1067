"""Seeded synthetic inputs for the state-sharding engine.

This module serves both sides of every parity check -- the CPU oracle and the
HIP library -- and holds none of the method's arithmetic: it only turns
(seed, stream, element index) into numbers.

The generator is counter-based, so any element can be produced on its own and
the same bits come out on the CPU and on the GPU:

  * word(seed, stream, i, c) = fmix32(fmix32(lo(i) ^ K) ^ (hi(i) + c*0x9E3779B9 + K2))
    where fmix32 is MurmurHash3's 32-bit finalizer (Appleby), K/K2 are 32-bit
    keys derived from (seed, stream) by the same finalizer, and c in {0, 1}
    picks one of two words per element.  All arithmetic is exact integer
    arithmetic on int64 tensors kept below 2^63.
  * uniform 16-bit patterns: the low half of word c=0 (NaN payloads included).
  * an approximately normal value with standard deviation sigma: the four
    16-bit halves of words 0 and 1 are summed (Irwin-Hall, n=4), centred,
    converted exactly to fp32 and multiplied once, in fp32, by
    fp32(sigma / sd) with sd = sqrt(4 * (2^32 - 1) / 12).  One IEEE multiply
    with round-to-nearest-even gives the same bits on both devices.
  * bf16 values are torch's round-to-nearest-even conversion of those fp32
    values.

Stream numbering used by the tests and the benchmark: 1 parameters (index =
element position in the concatenation of a model's parameters), 2 fp32
master, 3 first moment, 4 second moment, 100 + j*N + k the gradient slice of
micro-step j, logical rank k.
"""
from __future__ import annotations

import math

import numpy as np
import torch

_M32 = 0xFFFFFFFF
_SD4 = math.sqrt(4.0 * (2.0 ** 32 - 1.0) / 12.0)  # sd of a sum of four U{0..65535}

STREAM_PARAMS = 1
STREAM_MASTER = 2
STREAM_EXP_AVG = 3
STREAM_EXP_AVG_SQ = 4


def stream_grad(j: int, k: int, world: int) -> int:
    return 100 + j * world + k


def _fmix32_int(x: int) -> int:
    x &= _M32
    x ^= x >> 16
    x = (x * 0x85EBCA6B) & _M32
    x ^= x >> 13
    x = (x * 0xC2B2AE35) & _M32
    x ^= x >> 16
    return x


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    # (x * c) mod 2^32 for 0 <= x, c < 2^32 with every product below 2^48
    lo = x & 0xFFFF
    hi = x >> 16
    return (lo * c + (((hi * c) & 0xFFFF) << 16)) & _M32


def _fmix32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x85EBCA6B)
    x = x ^ (x >> 13)
    x = _mul32(x, 0xC2B2AE35)
    x = x ^ (x >> 16)
    return x


def _keys(seed: int, stream: int):
    k1 = _fmix32_int(_fmix32_int(seed) ^ ((stream * 0x27D4EB2F) & _M32))
    k2 = _fmix32_int(k1 ^ 0x165667B1)
    return k1, k2


def words(seed: int, stream: int, idx: torch.Tensor, c: int) -> torch.Tensor:
    """32-bit word c of elements `idx` (int64 tensor), as int64 in [0, 2^32)."""
    k1, k2 = _keys(seed, stream)
    lo = idx & _M32
    hi = idx >> 32
    a = _fmix32(lo ^ k1)
    b = (hi + ((c * 0x9E3779B9 + k2) & _M32)) & _M32
    return _fmix32(a ^ b)


def _index(start: int, count: int, device) -> torch.Tensor:
    return torch.arange(start, start + count, dtype=torch.int64, device=device)


def bits16_at(seed: int, stream: int, idx: torch.Tensor) -> torch.Tensor:
    """Uniform 16-bit patterns (int16 tensor) at element indices idx."""
    w = words(seed, stream, idx, 0) & 0xFFFF
    return (w - ((w >> 15) << 16)).to(torch.int16)


def bits32_at(seed: int, stream: int, idx: torch.Tensor) -> torch.Tensor:
    """Uniform 32-bit patterns (int32 tensor) at element indices idx."""
    w = words(seed, stream, idx, 0)
    return (w - ((w >> 31) << 32)).to(torch.int32)


def normal_f32_at(seed: int, stream: int, idx: torch.Tensor, sigma: float) -> torch.Tensor:
    """Approximately N(0, sigma^2) fp32 values at element indices idx."""
    w0 = words(seed, stream, idx, 0)
    w1 = words(seed, stream, idx, 1)
    s = (w0 & 0xFFFF) + (w0 >> 16) + (w1 & 0xFFFF) + (w1 >> 16) - 2 * 65535
    scale = torch.tensor(sigma / _SD4, dtype=torch.float32, device=idx.device)
    return s.to(torch.float32) * scale


def normal_bf16_at(seed: int, stream: int, idx: torch.Tensor, sigma: float) -> torch.Tensor:
    return normal_f32_at(seed, stream, idx, sigma).to(torch.bfloat16)


# ---- contiguous ranges, chunked so the int64 temporaries stay bounded ----

_CHUNK = 1 << 25


def _fill(out: torch.Tensor, start: int, fn) -> torch.Tensor:
    n = out.numel()
    flat = out.view(-1)
    for off in range(0, n, _CHUNK):
        cnt = min(_CHUNK, n - off)
        flat[off:off + cnt] = fn(_index(start + off, cnt, out.device))
    return out


def bits16(seed: int, stream: int, count: int, device="cpu", start: int = 0) -> torch.Tensor:
    out = torch.empty(count, dtype=torch.int16, device=device)
    return _fill(out, start, lambda i: bits16_at(seed, stream, i))


def bits32(seed: int, stream: int, count: int, device="cpu", start: int = 0) -> torch.Tensor:
    out = torch.empty(count, dtype=torch.int32, device=device)
    return _fill(out, start, lambda i: bits32_at(seed, stream, i))


def normal_f32(seed: int, stream: int, count: int, sigma: float, device="cpu",
               start: int = 0) -> torch.Tensor:
    out = torch.empty(count, dtype=torch.float32, device=device)
    return _fill(out, start, lambda i: normal_f32_at(seed, stream, i, sigma))


def normal_bf16(seed: int, stream: int, count: int, sigma: float, device="cpu",
                start: int = 0) -> torch.Tensor:
    out = torch.empty(count, dtype=torch.bfloat16, device=device)
    return _fill(out, start, lambda i: normal_bf16_at(seed, stream, i, sigma))


def fill_normal(out: torch.Tensor, seed: int, stream: int, sigma: float, start: int = 0) -> torch.Tensor:
    """Fill `out` (fp32 or bf16, any device, contiguous) in place with the
    same values normal_f32 / normal_bf16 would return for this range."""
    if out.dtype == torch.float32:
        return _fill(out, start, lambda i: normal_f32_at(seed, stream, i, sigma))
    if out.dtype == torch.bfloat16:
        return _fill(out, start, lambda i: normal_bf16_at(seed, stream, i, sigma))
    raise ValueError(f"fill_normal: unsupported dtype {out.dtype}")


def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a CPU tensor as numpy uint16 (2-byte) or uint32 (4-byte)."""
    t = t.detach().contiguous().cpu()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)


# ---- workload shapes ------------------------------------------------------

def mlp_tiny_shapes():
    """Tiny 2-layer MLP parameter list: W_in, W_out, bias, LN weight."""
    return [(64, 256), (256, 64), (256,), (64,)]


def llama_block_shapes(d: int = 4096, f: int = 11008, kv: int = None):
    """One Llama-style block, shapes as the workload lists them: q, k, v, o
    (d x d, or d x kv for grouped k/v), gate and up (d x f), down (f x d) and
    two RMSNorm weights (d)."""
    kv = d if kv is None else kv
    return [(d, d), (d, kv), (d, kv), (d, d), (d, f), (d, f), (f, d), (d,), (d,)]


def llama_model_groups(n_blocks: int, d: int, f: int, vocab: int = 32000, kv: int = None):
    """FSDP2 groups of a Llama-style model: one group per block, then the
    root group (token embedding and LM head, vocab x d each)."""
    groups = [llama_block_shapes(d, f, kv) for _ in range(n_blocks)]
    groups.append([(vocab, d), (vocab, d)])
    return groups


def padding_stress_numels(seed: int = 3, count: int = 97, log2_max: float = 22.0):
    """Element counts log-uniform in [1, 2^22]: numel = max(1, floor(2^u)),
    u ~ U[0, log2_max), drawn with numpy PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    u = rng.uniform(0.0, log2_max, size=count)
    return [max(1, int(math.floor(2.0 ** x))) for x in u]
