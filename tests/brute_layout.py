"""Constructive (brute-force) layout model used to pin the oracle's layouts.

It builds the gathered buffer element by element, as the pages describe the
construction, with PAD markers, and cuts it with torch.chunk -- the routine
the pages name for both FSDP1 (flatten().chunk(N), chunks padded to
chunks[0].numel()) and FSDP2 (chunk on dim 0, every rank's piece padded to
the first chunk's row count, missing chunks empty).  Source: "FSDP1 vs
FSDP2", section 03 and Table 3.

It shares nothing with the oracle's closed-form offsets: no start/pre/ceil
arithmetic appears here, only appending and torch.chunk.
"""
from typing import List, Sequence, Tuple

import torch

PAD = None


def _prod(shape):
    n = 1
    for d in shape:
        n *= int(d)
    return n


def fsdp1_gathered(shapes: Sequence[Sequence[int]], elem_bytes: int, world: int,
                   use_orig_params: bool) -> Tuple[List, int]:
    """Return (gathered list of (param, elem) or PAD, shard length)."""
    align = 16 // elem_bytes if use_orig_params else 1
    flat: List = []
    for i, shape in enumerate(shapes):
        if i > 0:
            while len(flat) % align != 0:   # pad before every later parameter
                flat.append(PAD)
        flat.extend((i, e) for e in range(_prod(shape)))
    if use_orig_params:
        while len(flat) % world != 0:       # pad the whole flat to a multiple of N
            flat.append(PAD)
    # torch.chunk over the flat's positions, then pad every chunk to chunks[0]
    chunks = list(torch.arange(len(flat)).chunk(world))
    shard = chunks[0].numel()
    gathered: List = []
    for r in range(world):
        piece = [flat[int(x)] for x in chunks[r]] if r < len(chunks) else []
        piece += [PAD] * (shard - len(piece))
        gathered.extend(piece)
    return gathered, shard


def fsdp2_gathered(shapes: Sequence[Sequence[int]], world: int) -> Tuple[List, int]:
    """Return (gathered list of (param, elem) or PAD, shard length T)."""
    per_rank: List[List] = [[] for _ in range(world)]
    for i, shape in enumerate(shapes):
        shape = tuple(shape) if len(shape) else (1,)
        ids = torch.arange(_prod(shape)).reshape(shape)
        chunks = list(ids.chunk(world, dim=0))
        full_rows = chunks[0].shape[0]
        row = _prod(shape[1:])
        for r in range(world):
            piece = [(i, int(e)) for e in chunks[r].reshape(-1)] if r < len(chunks) else []
            piece += [PAD] * (full_rows * row - len(piece))
            per_rank[r].extend(piece)
    shard = len(per_rank[0])
    assert all(len(p) == shard for p in per_rank)
    gathered = [x for p in per_rank for x in p]
    return gathered, shard


def index_map_from(gathered: List, numels: Sequence[int]) -> List[int]:
    """Gathered index of every parameter element, parameters in order."""
    where = {}
    for x, item in enumerate(gathered):
        if item is not PAD:
            assert item not in where, "element placed twice"
            where[item] = x
    out = []
    for i, n in enumerate(numels):
        for e in range(n):
            out.append(where[(i, e)])
    assert len(where) == len(out), "stray element"
    return out
