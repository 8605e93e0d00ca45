"""The allocation-free paged decode (attn_sink_fwd_decode_paged_noalloc, on the
library's own device scratch) against attn_sink_fwd_decode_paged with a
caller workspace: two calls in a row on one device, the second with a
smaller input, then the first input again.  Both entry points run the same
kernels with the same split plan, so their outputs must agree bit for bit
(which is within every tolerance against the oracle)."""

import math

import pytest
import torch

from softmax_learnable_sink_amd import synth
from tests.gpu_util import dev_tensor, need_gpu, say

pytestmark = pytest.mark.gpu


def _dev(case):
    return dict(q=dev_tensor(case["q"], synth.BF16), k=dev_tensor(case["k_cache"], synth.BF16),
                v=dev_tensor(case["v_cache"], synth.BF16),
                bt=torch.from_numpy(case["block_table"]).cuda(),
                sl=torch.from_numpy(case["seqlens"]).cuda(),
                sink=torch.from_numpy(case["sink"]).cuda())


def _both(d, window, num_splits=0):
    from softmax_learnable_sink_amd import binding
    D = d["q"].shape[-1]
    args = (d["q"], d["k"], d["v"], d["bt"], d["sl"], d["sink"])
    kw = dict(softmax_scale=1.0 / math.sqrt(D), window=window, num_splits=num_splits)
    o_ref, l_ref = binding.attn_sink_fwd_decode_paged(*args, **kw)
    out = torch.empty_like(d["q"])
    lse = torch.empty(d["q"].shape[:2], dtype=torch.float32, device=d["q"].device)
    o_na, l_na = binding.attn_sink_fwd_decode_paged_noalloc(*args, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    assert o_na.data_ptr() == out.data_ptr() and l_na.data_ptr() == lse.data_ptr()
    return (o_ref, l_ref), (o_na, l_na)


def _same(a, b):
    (o1, l1), (o2, l2) = a, b
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "O differs"
    assert torch.equal(l1, l2), "LSE differs"


def test_noalloc_decode_equals_workspace_decode():
    need_gpu()
    # 1: equal token ranges (32 sequences, L in [1024, 16384], 64/8 heads, D 64)
    say("case: noalloc decode B32 H64/8 D64 P16 L~U[1024,16384] (equal ranges), seed 11")
    big = synth.decode_case(32, 64, 8, 64, 16, 1024, 16384, seed=11)
    db = _dev(big)
    ref1, got1 = _both(db, None)
    _same(ref1, got1)
    # 2: smaller input, chunks, first/last window at D 128
    say("case: noalloc decode B3 H32/8 D128 P16 L~U[100,3000] window (64, 512), seed 12")
    small = synth.decode_case(3, 32, 8, 128, 16, 100, 3000, seed=12)
    ds = _dev(small)
    ref2, got2 = _both(ds, (64, 512))
    _same(ref2, got2)
    # 3: explicit split count on the small input, then the first input again
    say("case: noalloc decode, small input with 5 splits, then the first input again")
    ref3, got3 = _both(ds, (64, 512), num_splits=5)
    _same(ref3, got3)
    ref4, got4 = _both(db, None)
    _same(ref4, got4)
    _same(ref1, got4)
