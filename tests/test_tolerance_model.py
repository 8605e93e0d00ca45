"""Where the dQ/dK/dV tolerance comes from (CPU only).

The backward feeds P and dS to bf16 matrix products and reads the forward's
bf16 output O for Di = <dO, O>; each of those roundings has relative error up
to 2^-9.  This test emulates an *ideal* bf16-operand backward -- every other
step exact in float64 -- on the oracle's own quantities and shows that:
  * even that ideal kernel misses a 1e-2 + 1e-2|ref| bound (so no bf16
    kernel can be held to it), and
  * it stays within 2e-2 (1 + |ref|), two thirds of the bound the GPU tests
    use, |gpu - ref| <= 3e-2 (1 + |ref|); the remaining third covers the
    kernel's fp32 accumulation order and the rounding inside the forward that
    produced O (the worst ideal ratio over the shapes below is 0.018).
"""

import math

import numpy as np
import pytest

import oracle
from softmax_learnable_sink_amd import synth


def _bf16(x):
    return synth.bf16_to_f32(synth.f32_to_bf16_bits(np.asarray(x, np.float32))).astype(np.float64)


def _ideal_bf16_backward(q, k, v, sink, dout, scale):
    """Causal backward with bf16-rounded P, dS and O; everything else float64."""
    o, lse = oracle.prefill(q, k, v, sink, scale, causal=True)
    ob = _bf16(o)
    B, S, Hq, D = q.shape
    g = Hq // k.shape[2]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    mask = np.tril(np.ones((S, S), dtype=bool))
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            s = scale * q[b, :, h] @ k[b, :, kh].T
            p = np.where(mask, np.exp(np.where(mask, s, 0.0) - lse[b, h][:, None]), 0.0)
            di = np.sum(dout[b, :, h] * ob[b, :, h], axis=-1)
            ds = p * (dout[b, :, h] @ v[b, :, kh].T - di[:, None])
            pb, dsb = _bf16(p), _bf16(ds)
            dv[b, :, kh] += pb.T @ dout[b, :, h]
            dk[b, :, kh] += scale * dsb.T @ q[b, :, h]
            dq[b, :, h] = scale * dsb @ k[b, :, kh]
    return dq, dk, dv


@pytest.mark.parametrize("S,Hq,Hkv,D", [(140, 8, 1, 128), (300, 16, 2, 64), (512, 8, 1, 64)])
def test_ideal_bf16_backward_error_sets_the_tolerance(S, Hq, Hkv, D):
    case = synth.prefill_case(1, S, S, Hq, Hkv, D, seed=S + S + D, dout=True)
    x = {n: synth.values(case[n], synth.BF16).astype(np.float64) for n in ("q", "k", "v", "dout")}
    scale = 1.0 / math.sqrt(D)
    ref = oracle.backward(x["q"], x["k"], x["v"], case["sink"], x["dout"], scale, True)[:3]
    emu = _ideal_bf16_backward(x["q"], x["k"], x["v"], case["sink"], x["dout"], scale)
    tight_violated = False
    for name, e, r in zip(("dQ", "dK", "dV"), emu, ref):
        err = np.abs(e - r)
        tight_violated |= bool(np.any(err > 1e-2 + 1e-2 * np.abs(r)))
        assert np.all(err <= 2e-2 * (1.0 + np.abs(r))), name
    if D == 128:
        assert tight_violated
