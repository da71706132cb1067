"""Randomized GPU parity: seeded random parameter lists (scalars, empty
tensors, 1- to 3-D shapes of awkward sizes), random N, dtype, mode and
use_orig_params, random 0..7-element misalignment of every buffer.  Pack
(all ranks and one rank), unpack and re-shard to another random plan must
equal the oracle bit for bit; all outputs sit in canary guard bands.
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
