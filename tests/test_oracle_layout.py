"""Pins for the oracle's layouts (FSDP1 FlatParameter, FSDP2 per-parameter).

What pins them, none of it the oracle's own arithmetic:
  * the worked example printed in "FSDP1 vs FSDP2", Table 3 (golden file);
  * closed-form invariants stated on the same page, section 03: alignment
    unit a = 16/bytes, at most a-1 pad elements, aligned starts, equal
    chunks, FSDP2 shard = sum of ceil(d0/N) rows;
  * brute force: a constructive model that appends elements and PAD markers
    and cuts with torch.chunk (tests/brute_layout.py), compared on every
    element over exhaustive tiny parameter lists.
"""
import itertools
import json
import os
import random

import numpy as np
import pytest

import oracle
from brute_layout import PAD, fsdp1_gathered, fsdp2_gathered, index_map_from

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example_table3():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    shapes, N, w = g["shapes"], g["world"], g["elem_bytes"]
    per = g["elements_per_rank"]
    f1f = oracle.fsdp1_layout(shapes, w, N, use_orig_params=False)
    f1t = oracle.fsdp1_layout(shapes, w, N, use_orig_params=True)
    f2 = oracle.fsdp2_layout(shapes, w, N)
    assert f1f.shard == per["fsdp1_use_orig_params_false"]
    assert f1t.shard == per["fsdp1_use_orig_params_true"]
    assert f2.shard == per["fsdp2"]
    # the table's alignment pad ahead of the second parameter, then its world pad
    assert f1t.start[1] - 3 == g["fsdp1_use_orig_params_true_align_pad_before_second_param"]
    assert f1t.world * f1t.shard - f1t.flat_len == g["fsdp1_use_orig_params_true_world_pad"]
    assert list(f2.chunk_rows * f2.row) == g["fsdp2_per_param_chunk_elements"]


def _rand_shapes(rng, n, maxnumel):
    return [(rng.randint(0, maxnumel),) for _ in range(n)]


@pytest.mark.parametrize("elem_bytes", [2, 4])
@pytest.mark.parametrize("use_orig", [False, True])
def test_fsdp1_closed_forms(elem_bytes, use_orig):
    rng = random.Random(11 + elem_bytes + 7 * use_orig)
    a = 16 // elem_bytes if use_orig else 1
    for _ in range(300):
        N = rng.randint(1, 16)
        shapes = _rand_shapes(rng, rng.randint(1, 12), 40)
        L = oracle.fsdp1_layout(shapes, elem_bytes, N, use_orig)
        numel = [s[0] for s in shapes]
        prev_end = 0
        for i, n in enumerate(numel):
            pad = L.start[i] - prev_end
            assert 0 <= pad <= a - 1
            if i == 0:
                assert L.start[0] == 0
            else:
                assert L.start[i] % a == 0
            prev_end = L.start[i] + n
        assert L.flat_len == prev_end
        c = L.shard
        assert N * c >= L.flat_len
        if L.flat_len > 0:
            assert N * (c - 1) < L.flat_len
            assert N * c - L.flat_len <= N - 1   # world pad below N
        else:
            assert c == 0


def test_fsdp2_closed_forms():
    rng = random.Random(5)
    for _ in range(300):
        N = rng.randint(1, 16)
        shapes = [tuple(rng.randint(0, 20) for _ in range(rng.randint(0, 3)))
                  for _ in range(rng.randint(1, 8))]
        L = oracle.fsdp2_layout(shapes, 2, N)
        T = 0
        for s, cr, rw, pre in zip(shapes, L.chunk_rows, L.row, L.pre):
            d0 = s[0] if len(s) else 1
            assert pre == T
            assert cr * N >= d0 and (d0 == 0 or (cr - 1) * N < d0)
            T += cr * rw
        assert L.shard == T


def _check_against_brute(L, gathered, shard, numels):
    assert L.shard == shard
    assert len(gathered) == L.world * shard
    np.testing.assert_array_equal(L.index_map(), np.array(index_map_from(gathered, numels), np.int64))


@pytest.mark.parametrize("elem_bytes", [2, 4])
@pytest.mark.parametrize("use_orig", [False, True])
def test_fsdp1_brute_force_exhaustive(elem_bytes, use_orig):
    """Every list of 1-3 parameters with 0..9 elements, N = 1..8."""
    count = 0
    for n in (1, 2, 3):
        for numels in itertools.product(range(10), repeat=n):
            shapes = [(x,) for x in numels]
            for N in range(1, 9):
                L = oracle.fsdp1_layout(shapes, elem_bytes, N, use_orig)
                g, shard = fsdp1_gathered(shapes, elem_bytes, N, use_orig)
                _check_against_brute(L, g, shard, numels)
                count += 1
    assert count == (10 + 100 + 1000) * 8


@pytest.mark.parametrize("use_orig", [False, True])
def test_fsdp1_brute_force_random_long(use_orig):
    rng = random.Random(21 + use_orig)
    for _ in range(400):
        shapes = [tuple(rng.randint(1, 4) for _ in range(rng.randint(0, 3)))
                  for _ in range(rng.randint(4, 9))]
        for eb in (2, 4):
            N = rng.randint(1, 12)
            L = oracle.fsdp1_layout(shapes, eb, N, use_orig)
            g, shard = fsdp1_gathered(shapes, eb, N, use_orig)
            _check_against_brute(L, g, shard, [int(np.prod(s)) for s in shapes])


def test_fsdp2_brute_force_exhaustive():
    """Every list of 1-2 parameters shaped [d0, d1] with d0 in 0..9, d1 in 1..3,
    plus 1-D and 0-d parameters, N = 1..8."""
    shapes_1 = [(d0, d1) for d0 in range(10) for d1 in (1, 2, 3)] + [(5,), ()]
    count = 0
    for n in (1, 2):
        for shapes in itertools.product(shapes_1, repeat=n):
            for N in range(1, 9):
                L = oracle.fsdp2_layout(list(shapes), 2, N)
                g, shard = fsdp2_gathered(list(shapes), N)
                _check_against_brute(L, g, shard, [int(np.prod(s)) for s in shapes])
                count += 1
    assert count == (32 + 32 * 32) * 8


def test_fsdp2_brute_force_random_3d():
    rng = random.Random(99)
    for _ in range(300):
        shapes = [tuple(rng.randint(0, 7) for _ in range(rng.randint(0, 3)))
                  for _ in range(rng.randint(1, 6))]
        N = rng.randint(1, 10)
        L = oracle.fsdp2_layout(shapes, 4, N)
        g, shard = fsdp2_gathered(shapes, N)
        _check_against_brute(L, g, shard, [int(np.prod(s)) if len(s) else 1 for s in shapes])


def test_pack_unpack_roundtrip_and_pads():
    """Pack places every element once, pads are zero, unpack inverts it, and
    a rank's shard is its slice of the gathered buffer."""
    rng = np.random.default_rng(7)
    cases = [("f1", [(3,), (5,)], 4, True), ("f1", [(3,), (5,)], 4, False),
             ("f2", [(6, 3), (1,), (0, 2), (9,)], 4, None),
             ("f1", [(17,), (1,), (0,), (33,)], 3, True)]
    for kind, shapes, N, uo in cases:
        for eb in (2, 4):
            L = (oracle.fsdp1_layout(shapes, eb, N, uo) if kind == "f1"
                 else oracle.fsdp2_layout(shapes, eb, N))
            dt = np.uint16 if eb == 2 else np.uint32
            # nonzero patterns so pads (zero) are distinguishable
            params = [rng.integers(1, 2 ** (8 * eb), size=int(n), dtype=np.uint64).astype(dt)
                      for n in L.numel]
            gath = oracle.pack(L, params)
            idx = L.index_map()
            mask = np.zeros(L.gathered_numel, bool)
            mask[idx] = True
            assert (gath[~mask] == 0).all()
            np.testing.assert_array_equal(gath[idx], np.concatenate(params) if params else [])
            back = oracle.unpack(L, gath)
            for p, q in zip(params, back):
                np.testing.assert_array_equal(p, q)
            for r in range(N):
                np.testing.assert_array_equal(oracle.pack(L, params, rank=r),
                                              gath[r * L.shard:(r + 1) * L.shard])


def test_padding_stress_invariants():
    """97 log-uniform parameters, N=8: the closed-form invariants at the size
    the pack/unpack parity tests use (brute force is exhaustive only on tiny
    lists)."""
    import synth
    numels = synth.padding_stress_numels()
    shapes = [(n,) for n in numels]
    for eb in (2, 4):
        a = 16 // eb
        for uo in (True, False):
            L = oracle.fsdp1_layout(shapes, eb, 8, uo)
            ends = L.start + np.array(numels)
            pads = L.start[1:] - ends[:-1]
            assert (pads >= 0).all() and (pads <= (a - 1 if uo else 0)).all()
            if uo:
                assert (L.start % a == 0).all()
            assert 8 * L.shard >= L.flat_len > 8 * (L.shard - 1)


def test_reshard_is_unpack_then_pack():
    """Re-sharding equals copy-out under the old layout followed by copy-in
    under the new one, for rank-count changes, mode changes and both element
    sizes; re-sharding to the same layout reproduces the gathered buffer."""
    rng = np.random.default_rng(13)
    shapes = [(6, 3), (1,), (0, 2), (9,), (), (17, 2)]
    for eb in (2, 4):
        dt = np.uint16 if eb == 2 else np.uint32
        layouts = [oracle.fsdp2_layout(shapes, eb, N) for N in (1, 3, 4, 8)]
        layouts += [oracle.fsdp1_layout(shapes, eb, N, uo) for N in (2, 5) for uo in (False, True)]
        params = [rng.integers(1, 2 ** (8 * eb), size=int(n), dtype=np.uint64).astype(dt)
                  for n in layouts[0].numel]
        for Ls in layouts:
            g = oracle.pack(Ls, params)
            np.testing.assert_array_equal(oracle.reshard(Ls, Ls, g), g)
            for Ld in layouts:
                np.testing.assert_array_equal(oracle.reshard(Ls, Ld, g), oracle.pack(Ld, oracle.unpack(Ls, g)))


def test_layout_with_other_element_size():
    """Layout.with_elem_bytes keeps every element's gathered index and copies
    elements of the new size: for FSDP2 and FSDP1 without use_orig_params it
    is the layout built with that size; with use_orig_params (alignment by the
    parameter dtype) the 4-byte layout built directly places elements
    elsewhere, the derived one where the 2-byte layout does.  Pack and unpack
    round-trip 4-byte elements at those positions with zero pads."""
    shapes = [(6, 3), (9,), (1, 1), (13, 5), (0, 2), (33, 16), (7,)]
    rng = np.random.default_rng(4)
    for N in (1, 3, 8):
        for build, uo in ((lambda eb: oracle.fsdp2_layout(shapes, eb, N), False),
                          (lambda eb: oracle.fsdp1_layout(shapes, eb, N, False), False),
                          (lambda eb: oracle.fsdp1_layout(shapes, eb, N, True), True)):
            L2, L4 = build(2), build(4)
            T = L2.with_elem_bytes(4)
            np.testing.assert_array_equal(T.index_map(), L2.index_map())
            assert T.gathered_numel == L2.gathered_numel and T.elem_bytes == 4
            if uo:
                assert not np.array_equal(L4.index_map(), T.index_map())
            else:
                np.testing.assert_array_equal(L4.index_map(), T.index_map())
            params = [rng.integers(1, 1 << 32, size=int(n), dtype=np.uint64).astype(np.uint32) for n in T.numel]
            g = oracle.pack(T, params)
            assert g.dtype == np.uint32
            pads = np.ones(g.size, bool)
            pads[T.index_map()] = False
            assert not g[pads].any()
            np.testing.assert_array_equal(g[T.index_map()], np.concatenate(params))
            for a, b in zip(oracle.unpack(T, g), params):
                np.testing.assert_array_equal(a, b)
