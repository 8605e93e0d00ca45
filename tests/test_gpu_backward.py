"""GPU parity of the backward (dQ, dK, dV, dSink) against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
from softmax_learnable_sink_amd import synth
from tests.gpu_util import (TOL_DSINK_REL, check_grad, dev_tensor, host64, need_gpu, say, vals)

pytestmark = pytest.mark.gpu


def _gpu_fwd_bwd(case, scale, causal, window, use_sink=True):
    from softmax_learnable_sink_amd import binding
    q, k, v, do = (dev_tensor(case[n], synth.BF16) for n in ("q", "k", "v", "dout"))
    sink = torch.from_numpy(case["sink"]).cuda() if use_sink else None
    o, lse = binding.attn_sink_fwd_prefill(q, k, v, sink, causal=causal, softmax_scale=scale,
                                           window=window)
    dq, dk, dv, ds = binding.attn_sink_bwd(q, k, v, o, do, lse, sink, causal=causal,
                                           softmax_scale=scale, window=window)
    torch.cuda.synchronize()
    return dq, dk, dv, ds


def _check_dsink(got, ref):
    rel = float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))
    say(f"  dSink: max-norm relative error {rel:.3e} (tol {TOL_DSINK_REL:.0e})")
    assert rel <= TOL_DSINK_REL


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,D,causal,window", [
    (2, 200, 200, 8, 2, 64, True, None),     # g=4, ragged, several tiles
    (1, 300, 300, 16, 2, 64, True, None),    # g=8 (the training head layout)
    (1, 150, 150, 4, 4, 64, True, None),     # MHA
    (1, 100, 100, 6, 3, 64, True, None),     # g=2
    (1, 90, 250, 8, 2, 64, True, None),      # Sq < Sk, bottom-right causal
    (1, 160, 130, 8, 2, 64, False, None),    # non-causal
    (1, 260, 260, 8, 2, 64, True, (40, 90)),  # first/last window
    (1, 140, 140, 8, 1, 128, True, None),    # D=128
])
@pytest.mark.parametrize("use_sink", [True, False])
def test_backward_matches_oracle(B, Sq, Sk, Hq, Hkv, D, causal, window, use_sink):
    need_gpu()
    say(f"case: bwd B{B} Sq{Sq} Sk{Sk} H{Hq}/{Hkv} D{D} causal={causal} window={window} sink={use_sink}")
    case = synth.prefill_case(B, Sq, Sk, Hq, Hkv, D, seed=Sq + Sk + D, dout=True)
    scale = 1.0 / math.sqrt(D)
    dq, dk, dv, ds = _gpu_fwd_bwd(case, scale, causal, window, use_sink)
    rdq, rdk, rdv, rds, _, _ = oracle.backward(
        vals(case["q"], synth.BF16), vals(case["k"], synth.BF16), vals(case["v"], synth.BF16),
        case["sink"] if use_sink else None, vals(case["dout"], synth.BF16), scale, causal, window)
    check_grad("dQ", host64(dq), rdq)
    check_grad("dK", host64(dk), rdk)
    check_grad("dV", host64(dv), rdv)
    if use_sink:
        _check_dsink(host64(ds), rds)
    else:
        assert ds is None


def test_backward_minus_inf_sink_entries_and_rows_before_the_context():
    """Sq > Sk under the causal mask (the first 30 rows see no key) with a sink vector
    whose heads 1 and 5 are -inf: those heads' dSink is exactly 0 (no NaN from the rows
    with LSE = -inf), everything matches the oracle, and an all -inf vector gives the
    gradients of sink = NULL bitwise."""
    need_gpu()
    say("case: bwd B1 Sq90 Sk60 H8/2 D64 causal, sink with -inf entries, seed 77")
    case = synth.prefill_case(1, 90, 60, 8, 2, 64, seed=77, dout=True)
    case["sink"][[1, 5]] = -np.inf
    dq, dk, dv, ds = _gpu_fwd_bwd(case, 0.125, True, None)
    rdq, rdk, rdv, rds, _, _ = oracle.backward(
        vals(case["q"], synth.BF16), vals(case["k"], synth.BF16), vals(case["v"], synth.BF16),
        case["sink"], vals(case["dout"], synth.BF16), 0.125, True)
    check_grad("dQ", host64(dq), rdq)
    check_grad("dK", host64(dk), rdk)
    check_grad("dV", host64(dv), rdv)
    dsg = host64(ds)
    assert np.all(np.isfinite(dsg))
    assert dsg[1] == 0.0 and dsg[5] == 0.0
    _check_dsink(dsg, rds)
    case["sink"][:] = -np.inf
    a = _gpu_fwd_bwd(case, 0.125, True, None)
    b = _gpu_fwd_bwd(case, 0.125, True, None, use_sink=False)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert torch.equal(a[3], torch.zeros_like(a[3]))


def test_backward_deterministic():
    need_gpu()
    case = synth.prefill_case(1, 256, 256, 8, 2, 64, seed=31, dout=True)
    a = _gpu_fwd_bwd(case, 0.125, True, None)
    b = _gpu_fwd_bwd(case, 0.125, True, None)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


def test_training_full_size_sampled():
    """B2, S8192, 64/8 heads, D64, causal: dQ on sampled rows, dK/dV on the last 64 keys
    (only the last rows see them, so the oracle's sub-problem with those rows is exact),
    dSink of two heads over both sequences."""
    need_gpu()
    say("case: training fwd+bwd full size B2 S8192 H64/8 D64 causal")
    B, S, Hq, Hkv, D = 2, 8192, 64, 8, 64
    scale = 0.125
    case = synth.prefill_case(B, S, S, Hq, Hkv, D, seed=0, dout=True)
    dq, dk, dv, ds = _gpu_fwd_bwd(case, scale, True, None)
    dq, dk, dv, ds = host64(dq), host64(dk), host64(dv), host64(ds)
    for x in (dq, dk, dv, ds):
        assert np.all(np.isfinite(x))
    g = Hq // Hkv
    # dK / dV of keys [S-64, S) for KV head 3 of sequence 1: rows [S-64, S) of its 8 heads
    b, kh, j0 = 1, 3, S - 64
    hs = slice(kh * g, (kh + 1) * g)
    q = vals(case["q"][b:b + 1, j0:, hs], synth.BF16)
    k = vals(case["k"][b:b + 1, :, kh:kh + 1], synth.BF16)
    v = vals(case["v"][b:b + 1, :, kh:kh + 1], synth.BF16)
    do = vals(case["dout"][b:b + 1, j0:, hs], synth.BF16)
    rdq, rdk, rdv, _, _, _ = oracle.backward(q, k, v, case["sink"][hs], do, scale, True)
    check_grad("dK[last 64 keys]", dk[b, j0:, kh], rdk[0, j0:, 0])
    check_grad("dV[last 64 keys]", dv[b, j0:, kh], rdv[0, j0:, 0])
    check_grad("dQ[last 64 rows]", dq[b, j0:, hs], rdq[0])
    # dQ of sampled single rows: row i's dQ only needs keys [0, i]
    rng = np.random.default_rng(5)
    for n, i in enumerate([0, 1, 63, 64, 4095] + list(rng.integers(0, S, 7))):
        b = n % B
        h = int(rng.integers(0, Hq))
        kh = h // g
        r = oracle.backward(vals(case["q"][b:b + 1, i:i + 1, h:h + 1], synth.BF16),
                            vals(case["k"][b:b + 1, :i + 1, kh:kh + 1], synth.BF16),
                            vals(case["v"][b:b + 1, :i + 1, kh:kh + 1], synth.BF16),
                            case["sink"][h:h + 1],
                            vals(case["dout"][b:b + 1, i:i + 1, h:h + 1], synth.BF16), scale, True)
        check_grad(f"dQ[b{b} row{i} h{h}]", dq[b, i, h], r[0][0, 0, 0])
    # dSink of heads 0 and 37: every row of both sequences; the bound is the
    # max-norm relative one over these two heads, normalised by the oracle alone
    # (every head at full size: tests/test_gpu_fullsize.py)
    ref = {}
    for h in (0, 37):
        kh = h // g
        r = oracle.backward(vals(case["q"][:, :, h:h + 1], synth.BF16),
                            vals(case["k"][:, :, kh:kh + 1], synth.BF16),
                            vals(case["v"][:, :, kh:kh + 1], synth.BF16),
                            case["sink"][h:h + 1], vals(case["dout"][:, :, h:h + 1], synth.BF16),
                            scale, True)
        ref[h] = r[3][0]
        say(f"  dSink[{h}] gpu {ds[h]:.6f} oracle {ref[h]:.6f} abs err {abs(ds[h] - ref[h]):.3e}")
    norm = max(abs(x) for x in ref.values())
    for h, x in ref.items():
        assert abs(ds[h] - x) <= TOL_DSINK_REL * norm
