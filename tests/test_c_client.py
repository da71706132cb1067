"""The engine used from plain C (tests/c/fs_c_client.c): include/fs.h
compiles as C99 and links, and a C caller gets the same plans, error codes
and GPU results as the Python binding.

* host mode (no GPU): the worked example of "FSDP1 vs FSDP2" (Table 3) under
  the three layouts -- elements per rank, pads, and every segment's placement
  checked against the oracle's index map -- and the documented error codes;
* gpu mode: pack / unpack / reduce / AdamW on the tiny MLP group through the C
  ABI and the HIP runtime only, checked inside the program against what the
  method fixes (placement, zero pads, round trip, exact average, the
  first-step AdamW closed form).
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "c"))
import build_client  # noqa: E402

GOLDEN = json.load(open(os.path.join(HERE, "golden", "worked_example.json")))
FS_E_INVAL, FS_E_UNSUPPORTED, FS_E_DTYPE = -1, -2, -3


@pytest.fixture(scope="module")
def client():
    return build_client.build(force=False)


def _check_segments(rec, L, shard):
    got = np.full(L.gathered_numel, -1, np.int64)
    offs = np.concatenate([[0], np.cumsum(L.numel)]).astype(np.int64)
    for dst, src, ln, p, r in rec["segments"]:
        assert ln > 0 and dst // shard == r and (dst + ln - 1) // shard == r
        got[dst:dst + ln] = offs[p] + src + np.arange(ln)
    want = np.full(L.gathered_numel, -1, np.int64)
    want[L.index_map()] = np.arange(int(offs[-1]))
    np.testing.assert_array_equal(got, want)


def test_c_client_host_worked_example(client):
    out = subprocess.run([client, "host"], capture_output=True, text=True, timeout=60, check=True).stdout
    rec = json.loads(out)
    assert rec["rc"] == [0, 0, 0]
    shapes, N, eb = [tuple(s) for s in GOLDEN["shapes"]], GOLDEN["world"], GOLDEN["elem_bytes"]
    per_rank = GOLDEN["elements_per_rank"]
    for key, L in (("fsdp1_use_orig_params_false", oracle.fsdp1_layout(shapes, eb, N, False)),
                   ("fsdp1_use_orig_params_true", oracle.fsdp1_layout(shapes, eb, N, True)),
                   ("fsdp2", oracle.fsdp2_layout(shapes, eb, N))):
        assert rec[key]["shard_numel"] == per_rank[key]
        assert rec[key]["gathered_numel"] == N * per_rank[key]
        _check_segments(rec[key], L, per_rank[key])
    t = rec["fsdp1_use_orig_params_true"]
    assert t["align_pad"] == GOLDEN["fsdp1_use_orig_params_true_align_pad_before_second_param"]
    assert t["tail_pad"] == GOLDEN["fsdp1_use_orig_params_true_world_pad"]
    rank0 = [s for s in rec["fsdp2"]["segments"] if s[4] == 0]
    assert [s[2] for s in sorted(rank0, key=lambda s: s[3])] == GOLDEN["fsdp2_per_param_chunk_elements"]
    assert rec["errors"] == {"world_0": FS_E_INVAL, "use_orig_params_fsdp2": FS_E_UNSUPPORTED,
                             "negative_dim": FS_E_INVAL, "grad_acc_0": FS_E_INVAL,
                             "twin_bad_dtype": FS_E_DTYPE, "twin_null": FS_E_INVAL, "last_error_nonempty": 1}


def test_c_client_host_fp32_twin(client):
    """From C, the fp32 twin of the worked example's use_orig_params plan
    keeps the bf16 plan's positions (the 16-byte alignment counted in 2-byte
    elements: 5 pad elements before the second parameter, 4 elements per
    rank), while the plan made directly with FS_FP32 aligns 4-byte elements
    (1 pad element, 3 per rank): "FSDP1 vs FSDP2", section 03."""
    rec = json.loads(subprocess.run([client, "host"], capture_output=True, text=True, timeout=60,
                                    check=True).stdout)
    assert rec["twin_rc"] == [0, 0] and rec["twin_elem_bytes"] == 4
    shapes, N = [tuple(s) for s in GOLDEN["shapes"]], GOLDEN["world"]
    bf, tw, d32 = (rec["fsdp1_use_orig_params_true" + k] for k in ("", "_fp32_twin", "_fp32_direct"))
    for k in ("shard_numel", "gathered_numel", "align_pad", "tail_pad", "segments"):
        assert tw[k] == bf[k]
    L = oracle.fsdp1_layout(shapes, 2, N, True)
    _check_segments(tw, L.with_elem_bytes(4), tw["shard_numel"])
    D = oracle.fsdp1_layout(shapes, 4, N, True)
    assert d32["shard_numel"] == 3 and d32["gathered_numel"] == 12 and d32["align_pad"] == 1
    _check_segments(d32, D, 3)


@pytest.mark.gpu
def test_c_client_gpu_step(client):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[gpu] C client: tiny MLP step through the C ABI", file=sys.stderr, flush=True)
    res = subprocess.run([client, "gpu"], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stdout + res.stderr
