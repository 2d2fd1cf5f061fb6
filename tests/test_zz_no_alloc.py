"""duo_decode_static (split-K partials and arrival counters in the library's static
device array, no allocation) against duo_decode (the same kernels over the handle's
workspace), through the C ABI: two calls in a row, the second with a smaller input."""

import numpy as np
import pytest

from mixed_head_kv_amd import inputs as I

from parity_util import device_synth, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _filled(w, n):
    """A handle of workload w holding positions [0, n) appended through kv_append."""
    from mixed_head_kv_amd.binding import DuoKV
    kv = DuoKV.for_workload(w)
    kv.append(0, device_synth(w, 0, "k", 0, n), device_synth(w, 0, "v", 0, n))
    return kv


# A long context (many retrieval splits, so the merge runs from the static array), then a
# shorter one with fewer heads; bf16 MHA and int4 GQA.
CASES = [
    ("bf16 GQA, 40000 keys", I.Workload("na_big", 61, 1, 32, 8, 128, "bf16", "same", 64, 256, 40000, 0, 4, 4), 40000),
    ("int4 GQA, 3000 keys", I.Workload("na_small", 62, 1, 8, 4, 128, "bf16", "int4", 4, 64, 3000, 0, 4, 2), 3000),
]


def test_static_scratch_decode_matches_workspace_decode(torch_cuda):
    from mixed_head_kv_amd import binding as B
    for label, w, n in CASES:
        say(f"no-alloc decode: {label}")
        a, b = _filled(w, n), _filled(w, n)
        for step in range(2):
            t = n + step
            q = device_synth(w, 0, "q", t, 1)[0]
            k = device_synth(w, 0, "k", t, 1)[0]
            v = device_synth(w, 0, "v", t, 1)[0]
            out_ws = torch_cuda.empty_like(q)
            out_st = torch_cuda.full_like(q, float("nan"))
            B.duo_decode(a.h, 0, q, k, v, out_ws)            # appends into a
            B.duo_decode_static(b.h, 0, q, k, v, out_st)     # appends into b
            torch_cuda.cuda.synchronize()
            assert torch_cuda.equal(out_ws, out_st), (label, step)
            # attend again without appending: the same token, no state change
            out2 = torch_cuda.full_like(q, float("nan"))
            B.duo_decode_static(b.h, 0, q, None, None, out2)
            torch_cuda.cuda.synchronize()
            assert torch_cuda.equal(out_ws, out2), (label, step, "no append")
        assert a.length(0) == b.length(0) == n + 2
        a.close()
        b.close()


def test_static_scratch_decode_rejects_what_does_not_fit(torch_cuda):
    """32 sequences x 1024 query heads: one split of every query head needs
    32 * 1024 * 130 * 4 bytes (17 MB), above the 16 MiB array: DUO_E_CAPACITY, and
    nothing is appended.  (The workspace's own partial buffer makes this handle ~35 GB.)"""
    from mixed_head_kv_amd import binding as B
    w = I.Workload("na_wide", 63, 1, 1024, 64, 128, "bf16", "same", 4, 16, 64, 0, 1, 32)
    say("no-alloc decode: 32 x 1024 query heads (rejected)")
    kv = B.DuoKV.for_workload(w, batch=32)
    q = torch_cuda.zeros((32, 1024, 128), dtype=torch_cuda.bfloat16, device="cuda")
    k = torch_cuda.zeros((32, 64, 128), dtype=torch_cuda.bfloat16, device="cuda")
    with pytest.raises(B.DuoError) as e:
        B.duo_decode_static(kv.h, 0, q, k, k, q)
    assert e.value.code == B.DUO_E_CAPACITY
    assert kv.length(0) == 0
    kv.close()
    del kv
    torch_cuda.cuda.empty_cache()
