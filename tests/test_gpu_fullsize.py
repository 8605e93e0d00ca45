"""Element-by-element GPU parity at the full workload sizes.

Every output element of the GQA prefill (B4 S4096, 64/8 heads, D64, causal),
of the training forward + backward (B2 S8192, 64/8 heads, D64, causal: O, LSE,
dQ, dK, dV and all 64 dSink values) and of the chunked-prefill workload (2
sequences x 4096 new tokens on 4096..12288 cached ones, 64/8 heads, page 16)
is compared with the fp64 oracle.  The oracle runs per (sequence, KV-head
group): a group's outputs depend on that sequence, its KV head and its query
heads only, so each sub-problem is the oracle's own definition on a slice of
the inputs, and dSink sums its per-sequence values over the sequences.
"""

import time

import numpy as np
import pytest
import torch

import oracle
from softmax_learnable_sink_amd import synth
from tests.gpu_util import (TOL_DSINK_REL, TOL_LSE, TOL_O, dev_tensor, grad_ratio, host64,
                            max_abs, need_gpu, oracle_map, say, vals)

pytestmark = [pytest.mark.gpu, pytest.mark.fullsize]


def _finite(*xs):
    for x in xs:
        assert np.all(np.isfinite(x)), "non-finite GPU output"


def test_gqa_prefill_full_size_every_element():
    need_gpu()
    from softmax_learnable_sink_amd import binding
    B, S, Hq, Hkv, D = 4, 4096, 64, 8, 64
    g = Hq // Hkv
    say("case: GQA prefill B4 S4096 H64/8 D64 causal bf16, every O and LSE element, seed 0")
    case = synth.prefill_case(B, S, S, Hq, Hkv, D, seed=0)
    q, k, v = (dev_tensor(case[n], synth.BF16) for n in ("q", "k", "v"))
    sink = torch.from_numpy(case["sink"]).cuda()
    o, lse = binding.attn_sink_fwd_prefill(q, k, v, sink, causal=True, softmax_scale=0.125)
    torch.cuda.synchronize()
    og, lg = host64(o), host64(lse)
    del q, k, v, o, lse
    _finite(og, lg)

    def job(bk):
        b, kh = bk
        hs = slice(kh * g, (kh + 1) * g)
        ro, rl = oracle.prefill(vals(case["q"][b:b + 1, :, hs], synth.BF16),
                                vals(case["k"][b:b + 1, :, kh:kh + 1], synth.BF16),
                                vals(case["v"][b:b + 1, :, kh:kh + 1], synth.BF16),
                                case["sink"][hs], 0.125, causal=True)
        return max_abs(og[b:b + 1, :, hs], ro), max_abs(lg[b:b + 1, hs], rl)

    t0 = time.time()
    errs = oracle_map(job, [(b, kh) for b in range(B) for kh in range(Hkv)])
    eo = max(e[0] for e in errs)
    el = max(e[1] for e in errs)
    say(f"  every element: O max err {eo:.3e} (tol {TOL_O:.0e}), LSE max err {el:.3e} "
        f"(tol {TOL_LSE:.0e}); oracle {time.time() - t0:.1f} s")
    assert eo <= TOL_O and el <= TOL_LSE


def test_training_full_size_every_element():
    need_gpu()
    from softmax_learnable_sink_amd import binding
    B, S, Hq, Hkv, D = 2, 8192, 64, 8, 64
    g = Hq // Hkv
    scale = 0.125
    say("case: training B2 S8192 H64/8 D64 causal bf16 fwd+bwd, every O, LSE, dQ, dK, dV "
        "element and all 64 dSink values, seed 0")
    case = synth.prefill_case(B, S, S, Hq, Hkv, D, seed=0, dout=True)
    q, k, v, do = (dev_tensor(case[n], synth.BF16) for n in ("q", "k", "v", "dout"))
    sink = torch.from_numpy(case["sink"]).cuda()
    o, lse = binding.attn_sink_fwd_prefill(q, k, v, sink, causal=True, softmax_scale=scale)
    dq, dk, dv, ds = binding.attn_sink_bwd(q, k, v, o, do, lse, sink, causal=True,
                                           softmax_scale=scale)
    torch.cuda.synchronize()
    og, lg, dqg, dkg, dvg, dsg = (host64(x) for x in (o, lse, dq, dk, dv, ds))
    del q, k, v, do, o, lse, dq, dk, dv, ds
    _finite(og, lg, dqg, dkg, dvg, dsg)

    def job(bk):
        b, kh = bk
        hs = slice(kh * g, (kh + 1) * g)
        rdq, rdk, rdv, rds, ro, rl = oracle.backward(
            vals(case["q"][b:b + 1, :, hs], synth.BF16),
            vals(case["k"][b:b + 1, :, kh:kh + 1], synth.BF16),
            vals(case["v"][b:b + 1, :, kh:kh + 1], synth.BF16), case["sink"][hs],
            vals(case["dout"][b:b + 1, :, hs], synth.BF16), scale, True)
        return dict(
            o=max_abs(og[b:b + 1, :, hs], ro), lse=max_abs(lg[b:b + 1, hs], rl),
            dq=grad_ratio(dqg[b:b + 1, :, hs], rdq),
            dk=grad_ratio(dkg[b:b + 1, :, kh:kh + 1], rdk),
            dv=grad_ratio(dvg[b:b + 1, :, kh:kh + 1], rdv),
            dq_abs=max_abs(dqg[b:b + 1, :, hs], rdq),
            dk_abs=max_abs(dkg[b:b + 1, :, kh:kh + 1], rdk),
            dv_abs=max_abs(dvg[b:b + 1, :, kh:kh + 1], rdv),
            kh=kh, rds=rds)

    t0 = time.time()
    res = oracle_map(job, [(b, kh) for b in range(B) for kh in range(Hkv)])
    ref_ds = np.zeros(Hq)
    for r in res:
        ref_ds[r["kh"] * g:(r["kh"] + 1) * g] += r["rds"]
    worst = {n: max(r[n] for r in res) for n in ("o", "lse", "dq", "dk", "dv", "dq_abs",
                                                 "dk_abs", "dv_abs")}
    ds_rel = float(np.max(np.abs(dsg - ref_ds)) / np.max(np.abs(ref_ds)))
    say(f"  forward: O max err {worst['o']:.3e}, LSE max err {worst['lse']:.3e}")
    for n in ("dq", "dk", "dv"):
        say(f"  {n}: max abs err {worst[n + '_abs']:.3e}, "
            f"max err/(3e-2(1+|ref|)) = {worst[n]:.3f}")
    say(f"  dSink: max|gpu-ref|/max|ref| = {ds_rel:.3e} over 64 heads (tol {TOL_DSINK_REL:.0e});"
        f" oracle {time.time() - t0:.1f} s")
    assert worst["o"] <= TOL_O and worst["lse"] <= TOL_LSE
    assert worst["dq"] <= 1.0 and worst["dk"] <= 1.0 and worst["dv"] <= 1.0
    assert ds_rel <= TOL_DSINK_REL


def test_chunked_prefill_workload_every_row():
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say("case: extend B2 nq4096 ctx~U[4096,12288] H64/8 D64 P16 sink, every O and LSE "
        "element, seed 0")
    Hq, Hkv = 64, 8
    g = Hq // Hkv
    case = synth.extend_case(2, Hq, Hkv, 64, 16, 4096, 4096, 4096, 12288, seed=0)
    o, lse = binding.attn_sink_fwd_extend_paged(
        dev_tensor(case["q"], synth.BF16), dev_tensor(case["k_cache"], synth.BF16),
        dev_tensor(case["v_cache"], synth.BF16), torch.from_numpy(case["block_table"]).cuda(),
        torch.from_numpy(case["cu_seqlens_q"]).cuda(), torch.from_numpy(case["seqlens"]).cuda(),
        case["max_seqlen_q"], torch.from_numpy(case["sink"]).cuda(), softmax_scale=0.125)
    torch.cuda.synchronize()
    og, lg = host64(o), host64(lse)
    del o, lse
    _finite(og, lg)

    def job(kh):
        hs = slice(kh * g, (kh + 1) * g)
        ro, rl = oracle.extend_paged(vals(case["q"][:, hs], synth.BF16), case["cu_seqlens_q"],
                                     vals(case["k_cache"][:, :, kh:kh + 1], synth.BF16),
                                     vals(case["v_cache"][:, :, kh:kh + 1], synth.BF16),
                                     case["block_table"], case["seqlens"], case["sink"][hs],
                                     0.125, None)
        return max_abs(og[:, hs], ro), max_abs(lg[hs], rl)

    t0 = time.time()
    errs = oracle_map(job, list(range(Hkv)))
    eo = max(e[0] for e in errs)
    el = max(e[1] for e in errs)
    say(f"  every element: O max err {eo:.3e}, LSE max err {el:.3e}; "
        f"oracle {time.time() - t0:.1f} s")
    assert eo <= TOL_O and el <= TOL_LSE
