"""fs_reduce_adamw_step_noalloc (for callers that cannot allocate device
memory) against fs_reduce_adamw_step with a caller-supplied grad_out, bit for
bit, on two calls in a row, the second smaller; more than 32 terms, so the
partial sums go through the library's scratch array.  Also: an aligned and a
misaligned case, the 32-term path that needs no scratch, the largest size the
scratch holds, and the size limit."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import Guarded, bits, say

pytestmark = pytest.mark.gpu

fs = pytest.importorskip("fsdp_sharded_state_amd")


def _inputs(n, N, A, seed, shift=0):
    sl = [Guarded(n, torch.bfloat16, shift=shift,
                  fill=synth.normal_bf16(seed, synth.stream_grad(j, k, N), n, 1e-3, device="cuda"))
          for j in range(A) for k in range(N)]
    th = synth.normal_f32(seed, synth.STREAM_MASTER, n, 0.02, device="cuda")
    m = synth.normal_f32(seed, synth.STREAM_EXP_AVG, n, 1e-3, device="cuda")
    v = synth.normal_f32(seed, synth.STREAM_EXP_AVG_SQ, n, 1e-3, device="cuda") ** 2
    return sl, (th, m, v)


def _run_pair(n, N, A, seed, shift=0, step=7):
    say("no-alloc fused step", n, N, A, shift)
    sl, state = _inputs(n, N, A, seed, shift)
    ref = [Guarded(n, torch.float32, shift=shift, fill=x) for x in state]
    got = [Guarded(n, torch.float32, shift=shift, fill=x) for x in state]
    p_ref, p_got = Guarded(n, torch.bfloat16, shift=shift), Guarded(n, torch.bfloat16, shift=shift)
    g_ref = Guarded(n, torch.float32, shift=shift)
    fs.fs_reduce_adamw_step([s.t for s in sl], *(x.t for x in ref), p_ref.t, g_ref.t, world=N, grad_acc=A, step=step)
    fs.fs_reduce_adamw_step_noalloc([s.t for s in sl], *(x.t for x in got), p_got.t, world=N, grad_acc=A, step=step)
    torch.cuda.synchronize()
    for g in ref + got + [p_ref, p_got, g_ref] + sl:
        g.check()
    for a, b in zip(ref + [p_ref], got + [p_got]):
        np.testing.assert_array_equal(bits(a.t), bits(b.t))


def test_noalloc_matches_fused_with_grad_out_two_calls():
    # 40 terms over 5M elements, then 36 terms over a smaller, ragged n
    _run_pair(5_000_003, 8, 5, seed=11)
    _run_pair(40_007, 3, 12, seed=12)


def test_noalloc_misaligned_and_single_pass():
    _run_pair(30_011, 5, 7, seed=13, shift=1)    # 35 terms, misaligned buffers: the general kernels
    _run_pair(65_539, 8, 4, seed=14)             # 32 terms: one pass, no scratch needed


def test_noalloc_at_the_scratch_capacity():
    # the largest n the scratch array holds, 40 terms: every partial sum it can keep is written and read
    _run_pair(fs.NOALLOC_MAX_NUMEL, 8, 5, seed=15)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    n = fs.NOALLOC_MAX_NUMEL + 1
    one = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    st = [torch.zeros(n, device="cuda") for _ in range(3)]
    with pytest.raises(fs.FsError, match="scratch"):
        fs.fs_reduce_adamw_step_noalloc([one] * 33, *st, world=33, grad_acc=1)
    # one pass (at most 32 terms) needs no scratch: the same size is accepted
    fs.fs_reduce_adamw_step_noalloc([one] * 32, *st, world=32, grad_acc=1)
    torch.cuda.synchronize()
