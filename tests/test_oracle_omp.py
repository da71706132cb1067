"""The OpenMP build of the oracle (used only to time it on every host core)
computes exactly what the single-threaded build computes: same source, its
element loops split across threads, no arithmetic changed."""
import numpy as np

import oracle
import synth


def _bits16(n, seed):
    return np.random.default_rng(seed).integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)


def test_omp_build_runs_on_several_threads():
    assert oracle.threads(False) == 1
    assert oracle.threads(True) >= 1


def test_omp_reduce_bit_identical():
    n, N, A = 200_003, 8, 4
    sl = [synth.to_numpy_bits(synth.normal_bf16(5, synth.stream_grad(j, k, N), n, 1e-3))
          for j in range(A) for k in range(N)]
    a = oracle.reduce_shard(sl, N, A)
    b = oracle.reduce_shard(sl, N, A, parallel=True)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


def test_omp_adamw_bit_identical():
    n = 150_001
    th = synth.normal_f32(6, synth.STREAM_MASTER, n, 0.02).numpy()
    m = synth.normal_f32(6, synth.STREAM_EXP_AVG, n, 1e-3).numpy()
    v = synth.normal_f32(6, synth.STREAM_EXP_AVG_SQ, n, 1e-3).numpy() ** 2
    g = synth.normal_f32(6, 100, n, 1e-3).numpy()
    hp = oracle.AdamWHparams(step=1000)
    for grad in (g, oracle.bf16_round(g)):
        ra = oracle.adamw_step(th, m, v, grad, hp)
        rb = oracle.adamw_step(th, m, v, grad, hp, parallel=True)
        for x, y in zip(ra, rb):
            np.testing.assert_array_equal(x.view(np.uint32 if x.dtype == np.float32 else np.uint16),
                                          y.view(np.uint32 if y.dtype == np.float32 else np.uint16))


def test_omp_pack_unpack_bit_identical():
    shapes = [(1000, 37), (513,), (3, 333), (4097,)]
    for L in (oracle.fsdp1_layout(shapes, 2, 8, True), oracle.fsdp2_layout(shapes, 2, 8)):
        params = [_bits16(int(n), k) for k, n in enumerate(L.numel)]
        for rank in (-1, 3):
            np.testing.assert_array_equal(oracle.pack(L, params, rank), oracle.pack(L, params, rank, parallel=True))
        g = oracle.pack(L, params)
        for x, y in zip(oracle.unpack(L, g), oracle.unpack(L, g, parallel=True)):
            np.testing.assert_array_equal(x, y)
