"""GPU parity of the forward prefill (C ABI via the binding) against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
from softmax_learnable_sink_amd import synth
from tests.gpu_util import (TOL_F32, TOL_LSE, TOL_O, check_close, dev_tensor, host64, need_gpu,
                            say, vals)

pytestmark = pytest.mark.gpu


def _run(case, scale, causal, window, use_sink=True):
    from softmax_learnable_sink_amd import binding
    dt = case["dtype"]
    q, k, v = (dev_tensor(case[n], dt) for n in ("q", "k", "v"))
    sink = torch.from_numpy(case["sink"]).cuda() if (use_sink and case["sink"] is not None) else None
    o, lse = binding.attn_sink_fwd_prefill(q, k, v, sink, causal=causal, softmax_scale=scale,
                                           window=window)
    torch.cuda.synchronize()
    return o, lse


def _oracle(case, scale, causal, window, use_sink=True):
    dt = case["dtype"]
    sink = case["sink"] if use_sink else None
    return oracle.prefill(vals(case["q"], dt), vals(case["k"], dt), vals(case["v"], dt), sink,
                          scale, causal=causal, window=window)


def test_fp32_tiny_workload():
    """B1, S128, 2 heads / 2 KV heads, D64, causal, fp32, scale 1/8, seed 0: <= 1e-5."""
    need_gpu()
    say("case: fp32 B1 S128 H2/2 D64 causal seed0")
    case = synth.prefill_case(1, 128, 128, 2, 2, 64, dtype=synth.F32, seed=0)
    o, lse = _run(case, 0.125, True, None)
    ro, rl = _oracle(case, 0.125, True, None)
    check_close("O", host64(o), ro, TOL_F32)
    check_close("LSE", host64(lse), rl, TOL_F32)


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,D,causal,window", [
    (2, 300, 300, 8, 2, 64, True, None),     # g=4, ragged tail, several tiles
    (1, 200, 200, 4, 4, 64, True, None),     # MHA
    (1, 130, 130, 6, 3, 64, True, None),     # g=2
    (1, 100, 100, 3, 1, 64, True, None),     # g=3
    (1, 257, 257, 16, 2, 128, True, None),   # D=128, g=8
    (2, 77, 333, 8, 1, 64, True, None),      # Sq < Sk, bottom-right causal
    (1, 190, 260, 8, 2, 64, False, None),    # non-causal
    (1, 100, 60, 4, 2, 64, True, None),      # Sq > Sk: first rows see no key
    (1, 400, 400, 8, 2, 64, True, (70, 100)),  # first/last window
    (1, 333, 333, 8, 2, 64, True, (0, 64)),  # pure sliding window
    (1, 300, 300, 4, 1, 128, True, (5, 37)),  # window, D=128
    (1, 1, 1, 4, 4, 64, True, None),         # single token
    (1, 5, 0, 4, 2, 64, False, None),        # no keys at all
    # group size a multiple of 8: two 4-head workgroups per KV head
    (1, 300, 300, 16, 2, 64, True, None),    # g=8, ragged tail
    (2, 190, 260, 8, 1, 64, False, None),    # g=8, non-causal, Sq < Sk
    (1, 100, 60, 8, 1, 64, True, None),      # g=8, Sq > Sk: first rows see no key
    (1, 400, 400, 16, 2, 64, True, (70, 100)),  # g=8, first/last window
    (1, 333, 333, 8, 1, 64, True, (0, 64)),  # g=8, sliding window
    (1, 1, 1, 8, 1, 64, True, None),         # g=8, single token
    (1, 5, 0, 8, 1, 64, False, None),        # g=8, no keys at all
    (1, 130, 130, 32, 2, 64, True, None),    # g=16: two 8-head workgroups per KV head
])
@pytest.mark.parametrize("use_sink", [True, False])
def test_prefill_bf16_matches_oracle(B, Sq, Sk, Hq, Hkv, D, causal, window, use_sink):
    need_gpu()
    say(f"case: bf16 B{B} Sq{Sq} Sk{Sk} H{Hq}/{Hkv} D{D} causal={causal} window={window} sink={use_sink}")
    case = synth.prefill_case(B, Sq, Sk, Hq, Hkv, D, seed=B * 1000 + Sq + Sk + D)
    scale = 1.0 / math.sqrt(D)
    o, lse = _run(case, scale, causal, window, use_sink)
    ro, rl = _oracle(case, scale, causal, window, use_sink)
    check_close("O", host64(o), ro, TOL_O)
    check_close("LSE", host64(lse), rl, TOL_LSE)


def test_prefill_fp32_window_and_gqa():
    need_gpu()
    say("case: fp32 B2 Sq90 Sk150 H6/2 D128 window (3,20)")
    case = synth.prefill_case(2, 90, 150, 6, 2, 128, dtype=synth.F32, seed=5)
    o, lse = _run(case, 0.1, True, (3, 20))
    ro, rl = _oracle(case, 0.1, True, (3, 20))
    check_close("O", host64(o), ro, TOL_F32)
    check_close("LSE", host64(lse), rl, TOL_F32)


def test_no_sink_equals_minus_inf_sink_bitwise():
    """sink == NULL and a vector of -inf take the same arithmetic path."""
    need_gpu()
    from softmax_learnable_sink_amd import binding
    case = synth.prefill_case(1, 200, 200, 8, 2, 64, seed=7)
    q, k, v = (dev_tensor(case[n], synth.BF16) for n in ("q", "k", "v"))
    o1, l1 = binding.attn_sink_fwd_prefill(q, k, v, None)
    o2, l2 = binding.attn_sink_fwd_prefill(q, k, v, torch.full((8,), -math.inf, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_prefill_deterministic():
    need_gpu()
    from softmax_learnable_sink_amd import binding
    case = synth.prefill_case(2, 320, 320, 16, 2, 64, seed=8)
    q, k, v = (dev_tensor(case[n], synth.BF16) for n in ("q", "k", "v"))
    sink = torch.from_numpy(case["sink"]).cuda()
    o1, l1 = binding.attn_sink_fwd_prefill(q, k, v, sink)
    o2, l2 = binding.attn_sink_fwd_prefill(q, k, v, sink)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_gqa_prefill_full_size_sampled_rows():
    """B4, S4096, 64/8 heads, D64, causal, bf16 -- sampled rows against the oracle."""
    need_gpu()
    from softmax_learnable_sink_amd import binding
    B, S, Hq, Hkv, D = 4, 4096, 64, 8, 64
    say("case: GQA prefill full size B4 S4096 H64/8 D64 causal")
    case = synth.prefill_case(B, S, S, Hq, Hkv, D, seed=0)
    q, k, v = (dev_tensor(case[n], synth.BF16) for n in ("q", "k", "v"))
    sink = torch.from_numpy(case["sink"]).cuda()
    o, lse = binding.attn_sink_fwd_prefill(q, k, v, sink, causal=True, softmax_scale=0.125)
    torch.cuda.synchronize()
    og, lg = host64(o), host64(lse)
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
    rng = np.random.default_rng(123)
    rows = [0, 1, 63, 64, 127, 128, 2047, 4094, 4095] + list(rng.integers(0, S, 23))
    worst_o = worst_l = 0.0
    for n, i in enumerate(rows):
        b = n % B
        h = int(rng.integers(0, Hq))
        kh = h // (Hq // Hkv)
        qi = vals(case["q"][b:b + 1, i:i + 1, h:h + 1], synth.BF16)
        ki = vals(case["k"][b:b + 1, :i + 1, kh:kh + 1], synth.BF16)
        vi = vals(case["v"][b:b + 1, :i + 1, kh:kh + 1], synth.BF16)
        ro, rl = oracle.prefill(qi, ki, vi, case["sink"][h:h + 1], 0.125, causal=True)
        worst_o = max(worst_o, float(np.max(np.abs(og[b, i, h] - ro[0, 0, 0]))))
        worst_l = max(worst_l, abs(lg[b, h, i] - rl[0, 0, 0]))
    say(f"  sampled {len(rows)} rows: O err {worst_o:.3e}, LSE err {worst_l:.3e}")
    assert worst_o <= TOL_O and worst_l <= TOL_LSE
