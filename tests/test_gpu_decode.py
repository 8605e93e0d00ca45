"""GPU parity of paged decode, the window selection and the page gather."""

import math

import numpy as np
import pytest
import torch

import oracle
from softmax_learnable_sink_amd import synth
from tests.gpu_util import (TOL_LSE, TOL_O, check_close, dev_tensor, host64, need_gpu,
                            poison_unselected, say, vals)

pytestmark = pytest.mark.gpu


def _dev(case):
    return {
        "q": dev_tensor(case["q"], synth.BF16),
        "k": dev_tensor(case["k_cache"], synth.BF16),
        "v": dev_tensor(case["v_cache"], synth.BF16),
        "bt": torch.from_numpy(case["block_table"]).cuda(),
        "sl": torch.from_numpy(case["seqlens"]).cuda(),
        "sink": None if case["sink"] is None else torch.from_numpy(case["sink"]).cuda(),
    }


def _decode(d, scale, window, num_splits=0, sink="case"):
    from softmax_learnable_sink_amd import binding
    s = d["sink"] if sink == "case" else sink
    o, lse = binding.attn_sink_fwd_decode_paged(d["q"], d["k"], d["v"], d["bt"], d["sl"], s,
                                                softmax_scale=scale, window=window,
                                                num_splits=num_splits)
    torch.cuda.synchronize()
    return o, lse


def _oracle_decode(case, scale, window, batches=None):
    """Oracle decode, optionally on a subset of sequences (same per-sequence result)."""
    idx = list(range(len(case["seqlens"]))) if batches is None else list(batches)
    kf = case["k_cache"]
    vf = case["v_cache"]
    outs, lses = [], []
    for b in idx:
        slots = oracle.select_slots(case["block_table"][b:b + 1], case["seqlens"][b:b + 1],
                                    case["page_size"], window)[0]
        P = case["page_size"]
        ks = vals(kf[slots // P, slots % P], synth.BF16)[None]
        vs = vals(vf[slots // P, slots % P], synth.BF16)[None]
        q = vals(case["q"][b], synth.BF16)[None, None]
        o, l = oracle.prefill(q, ks, vs, case["sink"], scale, causal=False)
        outs.append(o[0, 0])
        lses.append(l[0, :, 0])
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("B,Hq,Hkv,D,P,lo,hi,window", [
    (4, 8, 2, 64, 16, 1, 700, None),        # g=4, short and ragged lengths
    (3, 16, 2, 128, 16, 100, 1500, None),   # D=128, g=8
    (5, 8, 8, 64, 1, 1, 300, None),         # MHA, page size 1
    (3, 64, 2, 64, 64, 10, 900, None),      # g=32: two head groups per KV head
    (2, 12, 4, 64, 8, 30, 400, None),       # g=3
    (4, 32, 8, 128, 16, 40, 500, (32, 96)),  # window, lengths around W1+W2
    (3, 8, 2, 64, 16, 120, 2600, (100, 700)),  # window, L > W1+W2 mostly
    (3, 8, 2, 64, 4, 1, 40, (0, 8)),        # pure sliding window, tiny
    (300, 8, 2, 64, 16, 1, 2500, None),     # > 256 sequences: chunk list built by a kernel
    (256, 8, 2, 64, 16, 1, 2500, (64, 512)),  # 256 sequences: chunks found by the scan
])
@pytest.mark.parametrize("use_sink", [True, False])
def test_decode_matches_oracle(B, Hq, Hkv, D, P, lo, hi, window, use_sink):
    need_gpu()
    say(f"case: decode B{B} H{Hq}/{Hkv} D{D} P{P} L[{lo},{hi}] window={window} sink={use_sink}")
    case = synth.decode_case(B, Hq, Hkv, D, P, lo, hi, seed=B + Hq + D + P + lo, sink=use_sink,
                             nan_poison=True)
    if window is not None:
        poison_unselected(case, window)
    scale = 1.0 / math.sqrt(D)
    d = _dev(case)
    ro, rl = _oracle_decode(case, scale, window)
    for ns in (0, 1, 3):
        o, lse = _decode(d, scale, window, ns)
        check_close(f"O (splits={ns})", host64(o), ro, TOL_O)
        check_close(f"LSE (splits={ns})", host64(lse), rl, TOL_LSE)


def test_decode_edge_lengths_window():
    """L = 1, W1+W2-1, W1+W2, W1+W2+1 and far beyond, page-unaligned window starts."""
    need_gpu()
    w = (16, 48)
    lengths = [1, 63, 64, 65, 66, 129, 1000, 1001]
    case = synth.decode_case(len(lengths), 8, 2, 64, 16, 1, 1001, seed=3, lengths=lengths,
                             nan_poison=True)
    poison_unselected(case, w)
    d = _dev(case)
    ro, rl = _oracle_decode(case, 0.125, w)
    o, lse = _decode(d, 0.125, w)
    check_close("O", host64(o), ro, TOL_O)
    check_close("LSE", host64(lse), rl, TOL_LSE)


def test_split_invariance_and_determinism():
    need_gpu()
    case = synth.decode_case(6, 16, 2, 64, 16, 500, 3000, seed=11)
    d = _dev(case)
    ro, _ = _oracle_decode(case, 0.125, None)
    outs = []
    for ns in (1, 2, 5, 64, 0):
        o, _ = _decode(d, 0.125, None, ns)
        check_close(f"O splits={ns}", host64(o), ro, TOL_O)
        o2, _ = _decode(d, 0.125, None, ns)
        assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "run-to-run difference"
        outs.append(host64(o))
    spread = max(float(np.max(np.abs(x - outs[0]))) for x in outs)
    say(f"  max spread across split counts: {spread:.3e}")


@pytest.mark.parametrize("B,Hq,Hkv,D,lo,hi,window", [
    (128, 8, 8, 64, 1, 2, None),           # 192 tokens: few ranges, each over many sequences
    (200, 8, 8, 64, 1, 300, None),         # ranges cross many sequence boundaries
    (128, 8, 8, 128, 1, 2100, None),       # D 128
    (129, 16, 8, 64, 100, 3000, (64, 512)),  # window, g 2
    (256, 8, 8, 64, 1000, 1300, None),     # 256 sequences (the largest scanned count)
])
def test_equal_ranges_match_oracle_and_one_split(B, Hq, Hkv, D, lo, hi, window):
    """The default work split for many KV-head units (equal token ranges per
    workgroup, crossing sequence boundaries) against the oracle, against one split
    per sequence, and run to run."""
    need_gpu()
    case = synth.decode_case(B, Hq, Hkv, D, 16, lo, hi, seed=21)
    d = _dev(case)
    scale = 1 / math.sqrt(D)
    ro, rl = _oracle_decode(case, scale, window)
    o, lse = _decode(d, scale, window)
    check_close("O", host64(o), ro, TOL_O)
    check_close("LSE", host64(lse), rl, TOL_LSE)
    o1, l1 = _decode(d, scale, window, 1)
    check_close("O vs one split", host64(o), host64(o1), TOL_O)
    check_close("LSE vs one split", host64(lse), host64(l1), TOL_LSE)
    o2, l2 = _decode(d, scale, window)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "run-to-run difference"
    assert torch.equal(lse, l2), "run-to-run difference (LSE)"


def test_paged_equals_identity_block_table_bitwise():
    """The physical page order does not change any bit of the result."""
    need_gpu()
    from softmax_learnable_sink_amd import binding
    B, Hq, Hkv, D, P = 3, 8, 2, 64, 16
    case = synth.decode_case(B, Hq, Hkv, D, P, 200, 900, seed=12)
    d = _dev(case)
    o1, l1 = _decode(d, 0.125, (32, 160))
    # rewrite the cache so that sequence b's pages are laid out contiguously
    bt = case["block_table"]
    npages = (case["seqlens"] + P - 1) // P
    order = np.concatenate([bt[b, :npages[b]] for b in range(B)])
    ident = np.full_like(bt, -1)
    pos = 0
    for b in range(B):
        ident[b, :npages[b]] = np.arange(pos, pos + npages[b])
        pos += npages[b]
    kc = dev_tensor(case["k_cache"][order], synth.BF16)
    vc = dev_tensor(case["v_cache"][order], synth.BF16)
    o2, l2 = binding.attn_sink_fwd_decode_paged(d["q"], kc, vc, torch.from_numpy(ident).cuda(),
                                                d["sl"], d["sink"], softmax_scale=0.125,
                                                window=(32, 160))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_decode_no_sink_equals_minus_inf_bitwise():
    need_gpu()
    case = synth.decode_case(4, 8, 2, 64, 16, 50, 800, seed=13)
    d = _dev(case)
    o1, l1 = _decode(d, 0.125, None, sink=None)
    o2, l2 = _decode(d, 0.125, None, sink=torch.full((8,), -math.inf, device="cuda"))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_decode_equals_last_row_of_gpu_prefill():
    """Decode of the newest token ~ last row of the GPU causal prefill over the same
    contiguous K/V (different kernels and orders: within the bf16 tolerance)."""
    need_gpu()
    from softmax_learnable_sink_amd import binding
    L, Hq, Hkv, D, P = 777, 8, 2, 64, 16
    case = synth.decode_case(1, Hq, Hkv, D, P, L, L, seed=14)
    d = _dev(case)
    o_dec, l_dec = _decode(d, 0.125, (64, 256))
    slots = oracle.select_slots(case["block_table"], case["seqlens"], P, None)[0]
    kseq = dev_tensor(case["k_cache"][slots // P, slots % P][None], synth.BF16)
    vseq = dev_tensor(case["v_cache"][slots // P, slots % P][None], synth.BF16)
    q = d["q"].view(1, 1, Hq, D)
    o_pf, l_pf = binding.attn_sink_fwd_prefill(q, kseq, vseq, d["sink"], causal=True,
                                               softmax_scale=0.125, window=(64, 256))
    torch.cuda.synchronize()
    check_close("O", host64(o_dec), host64(o_pf)[0, 0], TOL_O)
    check_close("LSE", host64(l_dec), host64(l_pf)[0, :, 0], TOL_LSE)


@pytest.mark.parametrize("P,window", [(16, (1024, 7168)), (16, None), (1, (3, 5)), (64, (10, 100))])
def test_select_slots_and_gather_bit_exact(P, window):
    need_gpu()
    from softmax_learnable_sink_amd import binding
    lengths = [1, 5, 9000, 8192, 8193, 20000] if P == 16 else [1, 7, 8, 9, 300, 1200]
    case = synth.decode_case(len(lengths), 4, 2, 64, P, 1, max(lengths), seed=15, lengths=lengths)
    bt = torch.from_numpy(case["block_table"]).cuda()
    sl = torch.from_numpy(case["seqlens"]).cuda()
    max_sel = max(len(oracle.select_tokens(L, window)) for L in lengths)
    slots, counts = binding.attn_sink_decode_select_slots(bt, sl, P, max_sel, window=window)
    torch.cuda.synchronize()
    ref = oracle.select_slots(case["block_table"], case["seqlens"], P, window)
    s_h, c_h = slots.cpu().numpy(), counts.cpu().numpy()
    for b in range(len(lengths)):
        assert c_h[b] == len(ref[b])
        assert np.array_equal(s_h[b, :len(ref[b])], ref[b])
        assert np.all(s_h[b, len(ref[b]):] == -1)
    kc, vc = dev_tensor(case["k_cache"], synth.BF16), dev_tensor(case["v_cache"], synth.BF16)
    ko, vo = binding.attn_sink_gather_kv(kc, vc, bt, sl, max_sel, window=window)
    torch.cuda.synchronize()
    rk, rv = oracle.gather_kv(case["k_cache"], case["v_cache"], case["block_table"],
                              case["seqlens"], P, window)
    ko_h = ko.view(torch.int16).cpu().numpy().view(np.uint16)
    vo_h = vo.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(len(lengths)):
        n = len(rk[b])
        assert np.array_equal(ko_h[b, :n], rk[b]) and np.array_equal(vo_h[b, :n], rv[b])
        assert np.all(ko_h[b, n:] == 0) and np.all(vo_h[b, n:] == 0)


def test_paged_decode_full_size():
    """B64, 64/8 heads, D64, P16, L ~ U[1024, 32768], random page permutation, sink N(0,1)."""
    need_gpu()
    say("case: paged decode full size B64 H64/8 D64 P16 L[1024,32768]")
    case = synth.decode_case(64, 64, 8, 64, 16, 1024, 32768, seed=0)
    d = _dev(case)
    o, lse = _decode(d, 0.125, None)
    ro, rl = _oracle_decode(case, 0.125, None)
    check_close("O", host64(o), ro, TOL_O)
    check_close("LSE", host64(lse), rl, TOL_LSE)


@pytest.mark.parametrize("B", [1, 32])
@pytest.mark.parametrize("use_sink", [False, True])
def test_window_decode_full_size(B, use_sink):
    """32/8 heads, D128, P16, window 1024+7168, L ~ U[16384, 65536]; unselected tokens
    hold NaN, so any read outside the selection shows up; selection checked bit-exact."""
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say(f"case: window decode full size B{B} sink={use_sink}")
    w = (1024, 7168)
    case = synth.decode_case(B, 32, 8, 128, 16, 16384, 65536, seed=0, sink=use_sink)
    poison_unselected(case, w)
    d = _dev(case)
    o, lse = _decode(d, 1.0 / math.sqrt(128), w)
    ro, rl = _oracle_decode(case, 1.0 / math.sqrt(128), w)
    check_close("O", host64(o), ro, TOL_O)
    check_close("LSE", host64(lse), rl, TOL_LSE)
    slots, counts = binding.attn_sink_decode_select_slots(d["bt"], d["sl"], 16, 8192, window=w)
    ref = oracle.select_slots(case["block_table"], case["seqlens"], 16, w)
    assert np.array_equal(slots.cpu().numpy(), np.stack(ref))
    assert np.all(counts.cpu().numpy() == 8192)
