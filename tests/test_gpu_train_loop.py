"""Several sharded training steps end to end on the GPU, against the oracle
running the same sequence on the CPU.

One FSDP group (FSDP2 per-parameter chunks, or the FSDP1 flat parameter with
or without use_orig_params) with N logical ranks and grad_acc micro-steps,
all ranks' state held in gathered-layout buffers (each rank's shard is its
slice, as "FSDP1 vs FSDP2" section 03 lays them out): per step,

  1. unpack the gathered bf16 parameters (the all-gather copy-out),
  2. pack every (micro-step j, rank k) gradient into the gathered layout --
     what the reduce-scatter delivers, one slice per term,
  3. average the N * grad_acc terms into the fp32 gradient ("Data
     parallelism, ZeRO and FSDP", sections 2.1, 5 and 9.2),
  4. AdamW on the fp32 master, moments and the bf16 copy, which is written
     straight into the gathered buffer the next step unpacks (section 9.1).

Steps 3 and 4 run as two kernels, as the fused reduce + AdamW (the fp32
gradient never stored), or with the bf16 reduce dtype (each micro-step's
average delivered in bf16, "FSDP1 vs FSDP2", mixed precision).  The
gradients are seeded synthetic values (the same counter-based streams on
both sides), not functions of the parameters.  Every intermediate is
compared bit for bit after each step; pads stay zero throughout.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import bits, say

pytestmark = pytest.mark.gpu
fs = pytest.importorskip("fsdp_sharded_state_amd")

MIXED = [(6, 3), (9,), (1, 1), (13, 5), (0, 2), (33, 16)]
CASES = [
    # (name, mode, use_orig_params, shapes, N, grad_acc, steps)
    ("fsdp2_mixed_pads", "fsdp2", False, MIXED, 4, 2, 3),
    ("fsdp2_llama_block_d256", "fsdp2", False, synth.llama_block_shapes(256, 688), 8, 4, 3),
    ("fsdp1_orig_params_mixed", "fsdp1", True, MIXED, 4, 2, 3),
    ("fsdp1_flat_mixed", "fsdp1", False, MIXED, 3, 3, 2),
]


def _grad_stream(j, k, N, t):
    return synth.stream_grad(j, k, N) + 1000 * t


@pytest.mark.parametrize("variant", ["two_kernels", "fused", "bf16_reduce_dtype"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_training_steps_match_oracle(case, variant):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    name, mode, uo, shapes, N, A, steps = case
    say("train loop", name, variant, N, A, steps)
    plan = fs.fs_plan(shapes, "bf16", N, uo, mode, A).upload()
    L = oracle.fsdp2_layout(shapes, 2, N) if mode == "fsdp2" else oracle.fsdp1_layout(shapes, 2, N, uo)
    numel = [int(np.prod(s)) if len(s) else 1 for s in shapes]
    n = plan.gathered_numel

    # initial parameters -> gathered bf16 buffer (both sides)
    p0 = [synth.to_numpy_bits(synth.normal_bf16(21, synth.STREAM_PARAMS, k, 0.02, start=sum(numel[:i])))
          for i, k in enumerate(numel)]
    g_host = oracle.pack(L, p0)
    gathered = torch.from_numpy(g_host.view(np.int16)).cuda().view(torch.bfloat16)
    # fp32 master = the bf16 values widened; moments start at zero
    th_host = (g_host.astype(np.uint32) << 16).view(np.float32)
    m_host = np.zeros(n, np.float32)
    v_host = np.zeros(n, np.float32)
    th = torch.from_numpy(th_host.copy()).cuda()
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    grad = torch.empty(n, dtype=torch.float32, device="cuda")
    outs = [torch.empty(k, dtype=torch.bfloat16, device="cuda") for k in numel]
    gpack = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(N * A)]

    for t in range(1, steps + 1):
        hp = oracle.AdamWHparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=t)
        # 1. copy-out
        fs.fs_unpack(plan, gathered, outs)
        params_host = oracle.unpack(L, g_host)
        # 2. per-(micro-step, rank) gradients, packed
        terms_host = []
        for j in range(A):
            for k in range(N):
                gh = [synth.to_numpy_bits(synth.normal_bf16(21, _grad_stream(j, k, N, t), c, 1e-3,
                                                             start=sum(numel[:i])))
                      for i, c in enumerate(numel)]
                gd = [torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16).reshape(s)
                      for x, s in zip(gh, shapes)]
                fs.fs_pack(plan, gd, gpack[j * N + k])
                terms_host.append(oracle.pack(L, gh))
        # 3. average and 4. AdamW, bf16 copy into the gathered buffer
        adam = dict(lr=hp.lr, beta1=hp.beta1, beta2=hp.beta2, eps=hp.eps, weight_decay=hp.weight_decay, step=t)
        if variant == "fused":
            fs.fs_reduce_adamw_step(gpack, th, m, v, gathered, grad, world=N, grad_acc=A, **adam)
            grad_host = oracle.reduce_shard(terms_host, N, A)
        else:
            if variant == "bf16_reduce_dtype":
                fs.fs_reduce_shard_ex(gpack, grad, N, A, reduce_dtype="bf16")
                grad_host = oracle.reduce_shard_bf16rs(terms_host, N, A)
            else:
                fs.fs_reduce_shard(gpack, grad, N, A)
                grad_host = oracle.reduce_shard(terms_host, N, A)
            fs.fs_adamw_step(th, m, v, grad, gathered, **adam)
        th_host, m_host, v_host, g_host = oracle.adamw_step(th_host, m_host, v_host, grad_host, hp)
        torch.cuda.synchronize()

        for i, (o, ph) in enumerate(zip(outs, params_host)):
            np.testing.assert_array_equal(bits(o), ph, err_msg=f"{name} step {t}: unpacked parameter {i}")
        for k in range(N * A):
            np.testing.assert_array_equal(bits(gpack[k]), terms_host[k], err_msg=f"{name} step {t}: term {k}")
        np.testing.assert_array_equal(bits(grad), grad_host.view(np.uint32), err_msg=f"{name} step {t}: gradient")
        for got, want, what in ((th, th_host, "master"), (m, m_host, "exp_avg"), (v, v_host, "exp_avg_sq")):
            np.testing.assert_array_equal(bits(got), want.view(np.uint32), err_msg=f"{name} step {t}: {what}")
        np.testing.assert_array_equal(bits(gathered), g_host, err_msg=f"{name} step {t}: bf16 parameters")
        pads = np.ones(n, bool)
        pads[L.index_map()] = False
        assert not np.any(bits(gathered)[pads]), f"{name} step {t}: a pad of the gathered buffer is not zero"


RESUME_CASES = [
    # (name, mode, use_orig_params, shapes, N, N2); the fp32 state is laid out by the bf16
    # plans' fp32 twins (fs_plan_twin), at the bf16 elements' positions
    ("fsdp2_mixed_4_to_2", "fsdp2", False, MIXED, 4, 2),
    ("fsdp2_llama_block_d256_8_to_2", "fsdp2", False, synth.llama_block_shapes(256, 688), 8, 2),
    ("fsdp1_flat_mixed_4_to_2", "fsdp1", False, MIXED, 4, 2),
    ("fsdp1_orig_params_mixed_4_to_2", "fsdp1", True, MIXED, 4, 2),
]


def _scaled_bits(x, scale):
    """bf16 bits times a power of two, exactly."""
    f = (x.astype(np.uint32) << 16).view(np.float32) * np.float32(scale)
    b = f.view(np.uint32)
    assert not np.any(b & 0xFFFF), "scaling left the bf16 grid"
    return (b >> 16).astype(np.uint16)


@pytest.mark.parametrize("variant", ["two_kernels", "fused"])
@pytest.mark.parametrize("case", RESUME_CASES, ids=lambda c: c[0])
def test_resume_at_another_rank_count(case, variant):
    """Resuming from a sharded state on a different number of ranks (the FSDP
    tutorial page, section 3.3, loads a checkpoint at another card count).
    Two steps run at N ranks with one micro-step each; then theta, m, v and
    the bf16 parameters are re-sharded to N2 ranks (fs_reshard) and the third
    step runs there with grad_acc = N / N2, micro-step j of rank k carrying
    the original rank j*N2 + k's gradient scaled by N2 / N (the 1/grad_acc
    that the micro-step loss holds, "Data parallelism, ZeRO and FSDP" section
    5).  Power-of-two scaling is exact in bf16 and fp32 and the terms are
    summed in the original rank order, so the averaged gradient and the whole
    state equal, bit for bit, the oracle's three steps at N ranks re-laid for
    N2 ranks by the oracle's re-shard.  The resumed step runs as the reduce
    and AdamW kernels, or as the fused reduce + AdamW."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    name, mode, uo, shapes, N, N2 = case
    A2 = N // N2
    say("resume at another rank count", name, variant, N, N2)

    def layout(n):
        return oracle.fsdp2_layout(shapes, 2, n) if mode == "fsdp2" else oracle.fsdp1_layout(shapes, 2, n, uo)

    P, Q = (fs.fs_plan(shapes, "bf16", n, uo, mode) for n in (N, N2))
    Pf, Qf = P.twin("fp32").upload(), Q.twin("fp32").upload()
    P.upload()
    Q.upload()
    L, M = layout(N), layout(N2)
    Lf, Mf = L.with_elem_bytes(4), M.with_elem_bytes(4)
    numel = [int(np.prod(s)) if len(s) else 1 for s in shapes]
    n, n2 = P.gathered_numel, Q.gathered_numel

    def grads(t, k):
        return [synth.to_numpy_bits(synth.normal_bf16(21, _grad_stream(0, k, N, t), c, 1e-3, start=sum(numel[:i])))
                for i, c in enumerate(numel)]

    def dev(host_bits, shape):
        return torch.from_numpy(host_bits.view(np.int16)).cuda().view(torch.bfloat16).reshape(shape)

    p0 = [synth.to_numpy_bits(synth.normal_bf16(21, synth.STREAM_PARAMS, k, 0.02, start=sum(numel[:i])))
          for i, k in enumerate(numel)]
    g_host = oracle.pack(L, p0)
    gathered = torch.from_numpy(g_host.view(np.int16)).cuda().view(torch.bfloat16)
    th_host = (g_host.astype(np.uint32) << 16).view(np.float32)
    m_host = np.zeros(n, np.float32)
    v_host = np.zeros(n, np.float32)
    th = torch.from_numpy(th_host.copy()).cuda()
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    grad = torch.empty(n, device="cuda")
    gpack = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(N)]
    adam = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)

    # the oracle runs three steps at N ranks; the GPU runs the first two there
    for t in (1, 2, 3):
        hp = oracle.AdamWHparams(step=t, **adam)
        grad_host = oracle.reduce_shard([oracle.pack(L, grads(t, k)) for k in range(N)], N, 1)
        th_host, m_host, v_host, g_host = oracle.adamw_step(th_host, m_host, v_host, grad_host, hp)
        if t < 3:
            for k in range(N):
                fs.fs_pack(P, [dev(x, s) for x, s in zip(grads(t, k), shapes)], gpack[k])
            fs.fs_reduce_shard(gpack, grad, N, 1)
            fs.fs_adamw_step(th, m, v, grad, gathered, step=t, **adam)

    # re-shard the state to N2 ranks
    rf, rb = fs.fs_reshard_plan(Pf, Qf).upload(), fs.fs_reshard_plan(P, Q).upload()
    th2, m2, v2, grad2 = (torch.empty(n2, device="cuda") for _ in range(4))
    gathered2 = torch.empty(n2, dtype=torch.bfloat16, device="cuda")
    for src, dst in ((th, th2), (m, m2), (v, v2)):
        fs.fs_reshard(rf, src, dst)
    fs.fs_reshard(rb, gathered, gathered2)

    # third step at N2 ranks, grad_acc A2
    gpack2 = [torch.empty(n2, dtype=torch.bfloat16, device="cuda") for _ in range(N)]
    for j in range(A2):
        for k in range(N2):
            gd = [dev(_scaled_bits(x, 1.0 / A2), s) for x, s in zip(grads(3, j * N2 + k), shapes)]
            fs.fs_pack(Q, gd, gpack2[j * N2 + k])
    if variant == "fused":
        fs.fs_reduce_adamw_step(gpack2, th2, m2, v2, gathered2, grad2, world=N2, grad_acc=A2, step=3, **adam)
    else:
        fs.fs_reduce_shard(gpack2, grad2, N2, A2)
        fs.fs_adamw_step(th2, m2, v2, grad2, gathered2, step=3, **adam)
    torch.cuda.synchronize()

    relaid = lambda x: oracle.reshard(Lf, Mf, x.view(np.uint32))
    np.testing.assert_array_equal(bits(grad2), relaid(grad_host), err_msg=f"{name}: gradient at {N2} ranks")
    for got, want, what in ((th2, th_host, "master"), (m2, m_host, "exp_avg"), (v2, v_host, "exp_avg_sq")):
        np.testing.assert_array_equal(bits(got), relaid(want), err_msg=f"{name}: {what} at {N2} ranks")
    np.testing.assert_array_equal(bits(gathered2), oracle.reshard(L, M, g_host), err_msg=f"{name}: bf16 parameters")
