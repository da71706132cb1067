"""The oracle's sharded training chain against plain data-parallel AdamW.

"Data parallelism, ZeRO and FSDP" (sections 2.2 and 9) states that data
parallelism over N ranks with grad_acc micro-steps is the large-batch step on
the averaged gradient, and that ZeRO-3 / FSDP only partitions where the
parameters, gradients and optimizer state live -- the update is unchanged.
So several steps of the oracle's sharded chain (pack the per-rank gradients
into the gathered layout, average, AdamW on the sharded fp32 state, unpack)
must match torch.optim.AdamW in float64 on the unsharded parameters, fed the
average of the same gradients, to within fp32 rounding (the hyperparameters
enter as the fp32 values the AdamW hyperparameter struct holds, so the
reference gets those same values); and the parameters
read back through the layout's index map must land on the right elements
(a misplaced element meets a different gradient and fails the comparison).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

MIXED = [(6, 3), (9,), (1, 1), (13, 5), (0, 2), (33, 16)]
CASES = [
    ("fsdp2", False, MIXED, 4, 2),
    ("fsdp1", True, MIXED, 4, 2),
    ("fsdp1", False, MIXED, 3, 3),
]
STEPS = 4


def _bf16_to_f64(bits16):
    return (bits16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_uo{int(c[1])}_N{c[3]}_A{c[4]}")
def test_sharded_chain_equals_unsharded_adamw(case):
    mode, uo, shapes, N, A = case
    L = oracle.fsdp2_layout(shapes, 2, N) if mode == "fsdp2" else oracle.fsdp1_layout(shapes, 2, N, uo)
    numel = [int(np.prod(s)) if len(s) else 1 for s in shapes]
    P = sum(numel)
    imap = L.index_map()                       # gathered index of every parameter element, in order
    p0 = synth.to_numpy_bits(synth.normal_bf16(31, synth.STREAM_PARAMS, P, 0.02))
    p0_list = np.split(p0, np.cumsum(numel)[:-1])

    # sharded chain (all ranks' shards in one gathered-layout buffer)
    g_bits = oracle.pack(L, p0_list)
    th = (g_bits.astype(np.uint32) << 16).view(np.float32).copy()
    m = np.zeros_like(th)
    v = np.zeros_like(th)

    # unsharded reference: float64 AdamW over the concatenated parameters
    ref = torch.nn.Parameter(torch.from_numpy(_bf16_to_f64(p0)))
    f32 = lambda x: float(np.float32(x))
    opt = torch.optim.AdamW([ref], lr=f32(1e-3), betas=(f32(0.9), f32(0.999)), eps=f32(1e-8),
                            weight_decay=f32(0.01), foreach=False, fused=False)

    for t in range(1, STEPS + 1):
        terms, full = [], np.zeros(P, np.float64)
        for j in range(A):
            for k in range(N):
                g = synth.to_numpy_bits(synth.normal_bf16(31, synth.stream_grad(j, k, N) + 100 * t, P, 1e-3))
                terms.append(oracle.pack(L, np.split(g, np.cumsum(numel)[:-1])))
                full += _bf16_to_f64(g)
        grad = oracle.reduce_shard(terms, N, A)
        hp = oracle.AdamWHparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=t)
        th, m, v, g_bits = oracle.adamw_step(th, m, v, grad, hp)

        ref.grad = torch.from_numpy(full / N)
        opt.step()

        # the averaged gradient, read through the layout, is the unsharded one
        np.testing.assert_allclose(grad[imap], full / N, rtol=2e-6, atol=1e-12)
        # the state after the step, read through the layout
        want = ref.detach().numpy()
        got = th[imap].astype(np.float64)
        np.testing.assert_allclose(got, want, rtol=0, atol=2e-8 * t)
        st = opt.state[ref]
        # fp32 state against float64: relative 1e-5, with absolute floors at the
        # fp32 rounding scale of the moments' magnitudes (m ~ 1e-4, v ~ 1e-9),
        # since a moment that passes near zero has no relative accuracy left
        np.testing.assert_allclose(m[imap], st["exp_avg"].numpy(), rtol=1e-5, atol=1e-10)
        np.testing.assert_allclose(v[imap], st["exp_avg_sq"].numpy(), rtol=1e-5, atol=1e-15)
        # pads carry no state
        pads = np.ones(th.size, bool)
        pads[imap] = False
        assert not np.any(th[pads]) and not np.any(m[pads]) and not np.any(v[pads]) and not np.any(g_bits[pads])


@pytest.mark.parametrize("mode,uo,N,N2", [("fsdp2", False, 4, 2), ("fsdp2", False, 8, 2), ("fsdp1", False, 4, 2),
                                          ("fsdp1", True, 4, 2), ("fsdp1", True, 8, 2)])
def test_resume_at_another_rank_count(mode, uo, N, N2):
    """Re-sharding the state to N2 ranks and continuing there with
    grad_acc = N / N2 (micro-step gradients scaled by N2 / N, the 1/grad_acc of
    "Data parallelism, ZeRO and FSDP" section 5) gives exactly the state of
    continuing at N ranks, re-laid: power-of-two scaling is exact and the
    terms keep their order.  Pins reshard against the chain: a re-shard that
    moves an element to another's place, or a reduce that reorders terms or
    divides by the wrong count, breaks the equality.  The fp32 state sits at
    the bf16 elements' positions (Layout.with_elem_bytes), which FSDP1's
    use_orig_params alignment makes differ from a 4-byte layout's."""
    A2 = N // N2
    lay = lambda n: oracle.fsdp2_layout(MIXED, 2, n) if mode == "fsdp2" else oracle.fsdp1_layout(MIXED, 2, n, uo)
    L, M = lay(N), lay(N2)
    Lf, Mf = L.with_elem_bytes(4), M.with_elem_bytes(4)
    numel = [int(np.prod(s)) if len(s) else 1 for s in MIXED]
    split = lambda x: np.split(x, np.cumsum(numel)[:-1])
    grads = lambda t, k: split(synth.to_numpy_bits(synth.normal_bf16(37, synth.stream_grad(0, k, N) + 100 * t,
                                                                      sum(numel), 1e-3)))
    half = lambda x: ((((x.astype(np.uint32) << 16).view(np.float32) * np.float32(1.0 / A2)).view(np.uint32)) >> 16
                      ).astype(np.uint16)
    p0 = synth.to_numpy_bits(synth.normal_bf16(37, synth.STREAM_PARAMS, sum(numel), 0.02))
    g = oracle.pack(L, split(p0))
    th = (g.astype(np.uint32) << 16).view(np.float32).copy()
    m, v = np.zeros_like(th), np.zeros_like(th)
    hp = lambda t: oracle.AdamWHparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=t)
    for t in (1, 2):
        th, m, v, g = oracle.adamw_step(th, m, v, oracle.reduce_shard([oracle.pack(L, grads(t, k)) for k in range(N)],
                                                                      N, 1), hp(t))
    gA = oracle.reduce_shard([oracle.pack(L, grads(3, k)) for k in range(N)], N, 1)
    A = oracle.adamw_step(th, m, v, gA, hp(3))
    relaid = lambda x: oracle.reshard(Lf, Mf, x.view(np.uint32))
    th2, m2, v2 = (relaid(x).view(np.float32) for x in (th, m, v))
    terms = [oracle.pack(M, [half(x) for x in grads(3, j * N2 + k)]) for j in range(A2) for k in range(N2)]
    gB = oracle.reduce_shard(terms, N2, A2)
    B = oracle.adamw_step(th2, m2, v2, gB, hp(3))
    np.testing.assert_array_equal(gB.view(np.uint32), relaid(gA))
    for a, b in zip(A[:3], B[:3]):
        np.testing.assert_array_equal(b.view(np.uint32), relaid(a))
    np.testing.assert_array_equal(B[3], oracle.reshard(L, M, A[3]))
