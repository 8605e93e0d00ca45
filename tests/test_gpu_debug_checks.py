"""The debug library (device-side precondition checks) on valid inputs: every
paged and packed entry point gives the release library's outputs bit for bit
and records no violation.  (Invalid inputs are exercised on the CPU only, in
tests/test_device_checks.py.)"""

import math

import numpy as np
import pytest
import torch

from softmax_learnable_sink_amd import synth
from tests.gpu_util import dev_tensor, need_gpu, say

pytestmark = pytest.mark.gpu


def _i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _both(monkeypatch, fn):
    """fn() with the release library, then with the debug library; the debug
    library's device check flags after it."""
    from softmax_learnable_sink_amd import binding
    ref = fn()
    torch.cuda.synchronize()
    dbg = binding.debug_lib()
    monkeypatch.setattr(binding, "_lib", dbg)
    binding.attn_sink_device_check_flags(clear=True, handle=dbg)
    got = fn()
    torch.cuda.synchronize()
    flags = binding.attn_sink_device_check_flags(clear=True, handle=dbg)
    monkeypatch.undo()
    return ref, got, flags


def _same(ref, got):
    for a, b in zip(ref, got):
        if a is None:
            assert b is None
            continue
        x = a.view(torch.int16) if a.dtype == torch.bfloat16 else a
        y = b.view(torch.int16) if b.dtype == torch.bfloat16 else b
        assert torch.equal(x, y)


@pytest.mark.parametrize("B,Hq,Hkv,D,lo,hi,window,splits", [
    (64, 64, 8, 64, 500, 3000, None, 0),           # equal token ranges
    (3, 32, 8, 128, 100, 3000, (64, 512), 0),      # chunks, with the window
    (4, 8, 2, 64, 1, 700, None, 3),                # explicit split count
])
def test_debug_decode_matches_release(monkeypatch, B, Hq, Hkv, D, lo, hi, window, splits):
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say(f"case: debug-checked decode B{B} H{Hq}/{Hkv} D{D} L~U[{lo},{hi}] window={window} "
        f"splits={splits}")
    c = synth.decode_case(B, Hq, Hkv, D, 16, lo, hi, seed=B + D)
    args = (dev_tensor(c["q"], synth.BF16), dev_tensor(c["k_cache"], synth.BF16),
            dev_tensor(c["v_cache"], synth.BF16), _i32(c["block_table"]), _i32(c["seqlens"]),
            torch.from_numpy(c["sink"]).cuda())
    ref, got, flags = _both(monkeypatch, lambda: binding.attn_sink_fwd_decode_paged(
        *args, softmax_scale=1 / math.sqrt(D), window=window, num_splits=splits))
    assert flags == 0
    _same(ref, got)


def test_debug_extend_and_index_rows_match_release(monkeypatch):
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say("case: debug-checked extend B3 H8/2 D64 P16 and index rows, seed 7")
    c = synth.extend_case(3, 8, 2, 64, 16, 1, 150, 0, 300, seed=7)
    q, kc, vc = (dev_tensor(c[n], synth.BF16) for n in ("q", "k_cache", "v_cache"))
    bt, cu, sl = _i32(c["block_table"]), _i32(c["cu_seqlens_q"]), _i32(c["seqlens"])
    sink = torch.from_numpy(c["sink"]).cuda()
    ref, got, flags = _both(monkeypatch, lambda: binding.attn_sink_fwd_extend_paged(
        q, kc, vc, bt, cu, sl, c["max_seqlen_q"], sink, softmax_scale=0.125, window=(16, 64)))
    assert flags == 0
    _same(ref, got)
    # per-query lists: every row lists its first 40 positions (entries past the
    # context are empty)
    tq = q.shape[0]
    idx = _i32(np.tile(np.arange(40, dtype=np.int32), (tq, 1)))
    ref, got, flags = _both(monkeypatch, lambda: binding.attn_sink_fwd_index_rows_paged(
        q, kc, vc, bt, cu, sl, idx, sink, softmax_scale=0.125))
    assert flags == 0
    _same(ref, got)


def test_debug_varlen_forward_backward_match_release(monkeypatch):
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say("case: debug-checked varlen fwd+bwd 3 sequences of 40..150 tokens H8/2 D64, seed 2")
    c = synth.varlen_case(3, 8, 2, 64, 40, 150, seed=2, dout=True)
    q, k, v, do = (dev_tensor(c[n], synth.BF16) for n in ("q", "k", "v", "dout"))
    sink = torch.from_numpy(c["sink"]).cuda()
    cq, ck = _i32(c["cu_seqlens_q"]), _i32(c["cu_seqlens_k"])

    def run():
        o, lse = binding.attn_sink_fwd_varlen(q, k, v, cq, ck, c["max_seqlen_q"], sink,
                                              softmax_scale=0.125)
        g = binding.attn_sink_bwd_varlen(q, k, v, o, do, lse, cq, ck, c["max_seqlen_q"],
                                         c["max_seqlen_k"], sink, softmax_scale=0.125)
        return (o, lse) + tuple(g)
    ref, got, flags = _both(monkeypatch, run)
    assert flags == 0
    _same(ref, got)
