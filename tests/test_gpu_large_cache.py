"""GPU parity of the paged kernels when a K/V cache array is larger than
4 GiB.  The kernels then read cache rows from 64-bit addresses (loads straight
into LDS for the chunked-prefill and index-list kernels, plain loads for the
decode) instead of 32-bit offsets from a buffer resource.  A small case's pages
are copied to the end of a cache of 4 GiB + a few pages, so every page the
kernels read lies past 4 GiB; the rest of the cache is never read and stays
uninitialised."""

import pytest
import torch

from softmax_learnable_sink_amd import synth
from tests import test_gpu_decode as tdec
from tests import test_gpu_extend as text
from tests import test_gpu_index as tidx
from tests.gpu_util import TOL_LSE, TOL_O, check_close, dev_tensor, host64, need_gpu, say

pytestmark = pytest.mark.gpu


def _embed(case):
    """(k, v, block table) with the case's pages at the end of caches of more
    than 4 GiB each."""
    npages, P, Hkv, D = case["k_cache"].shape
    page_bytes = P * Hkv * D * 2
    big = (4 << 30) // page_bytes + npages + 16
    base = big - npages
    assert base * page_bytes >= (4 << 30)
    k = torch.empty((big, P, Hkv, D), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((big, P, Hkv, D), dtype=torch.bfloat16, device="cuda")
    k[base:] = dev_tensor(case["k_cache"], synth.BF16)
    v[base:] = dev_tensor(case["v_cache"], synth.BF16)
    bt = torch.from_numpy(case["block_table"] + base).cuda()
    return k, v, bt


def test_extend_on_a_cache_past_4gib():
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say("case: extend B3 H8/2 D64 P16 q~U[1,150] ctx~U[0,300] sink, cache > 4 GiB, seed 7")
    case = synth.extend_case(3, 8, 2, 64, 16, 1, 150, 0, 300, seed=7, nan_poison=True)
    k, v, bt = _embed(case)
    o, lse = binding.attn_sink_fwd_extend_paged(
        dev_tensor(case["q"], synth.BF16), k, v, bt, torch.from_numpy(case["cu_seqlens_q"]).cuda(),
        torch.from_numpy(case["seqlens"]).cuda(), case["max_seqlen_q"],
        torch.from_numpy(case["sink"]).cuda(), softmax_scale=0.125)
    torch.cuda.synchronize()
    ro, rl = text._oracle(case, 0.125, None)
    check_close("O", host64(o), ro, TOL_O)
    check_close("LSE", host64(lse), rl, TOL_LSE)
    del k, v


def test_index_lists_on_a_cache_past_4gib():
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say("case: index B2 H16/2 D64 P1 q~U[60,200] ctx~U[100,2000] block 128 topk 256 "
        "shuffled padded, cache > 4 GiB, seed 9")
    case = synth.index_case(2, 16, 2, 64, 1, 60, 200, 100, 2000, 128, 256, seed=9, shuffle=True,
                            pad=20, nan_poison=True)
    k, v, bt = _embed(case)
    o, lse = binding.attn_sink_fwd_index_paged(
        dev_tensor(case["q"], synth.BF16), k, v, bt, tidx._i32(case["cu_seqlens_q"]),
        tidx._i32(case["seqlens"]), case["max_seqlen_q"], tidx._i32(case["kv_index"]),
        tidx._i32(case["cu_blocks"]), case["block_q"], torch.from_numpy(case["sink"]).cuda(),
        softmax_scale=0.125)
    torch.cuda.synchronize()
    ro, rl = tidx._oracle(case, 0.125)
    check_close("O", host64(o), ro, TOL_O)
    check_close("LSE", host64(lse), rl, TOL_LSE)
    del k, v


@pytest.mark.parametrize("window", [None, (64, 448)])
def test_decode_on_a_cache_past_4gib(window):
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say(f"case: decode B5 H16/4 D64 P16 L~U[1,3000] window {window} sink, cache > 4 GiB, seed 11")
    case = synth.decode_case(5, 16, 4, 64, 16, 1, 3000, seed=11)
    k, v, bt = _embed(case)
    o, lse = binding.attn_sink_fwd_decode_paged(
        dev_tensor(case["q"], synth.BF16), k, v, bt, torch.from_numpy(case["seqlens"]).cuda(),
        torch.from_numpy(case["sink"]).cuda(), softmax_scale=0.125, window=window)
    torch.cuda.synchronize()
    ro, rl = tdec._oracle_decode(case, 0.125, window)
    check_close("O", host64(o), ro, TOL_O)
    check_close("LSE", host64(lse), rl, TOL_LSE)
    del k, v


def test_index_rows_on_a_cache_past_4gib():
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say("case: index rows B3 H8/2 D64 P16 q~U[1,40] ctx~U[0,3000] topk 256, cache > 4 GiB, "
        "seed 13")
    case = synth.index_case(3, 8, 2, 64, 16, 1, 40, 0, 3000, 1, 256, seed=13, nan_poison=True)
    k, v, bt = _embed(case)
    o, lse = binding.attn_sink_fwd_index_rows_paged(
        dev_tensor(case["q"], synth.BF16), k, v, bt, tidx._i32(case["cu_seqlens_q"]),
        tidx._i32(case["seqlens"]), tidx._i32(case["kv_index"]),
        torch.from_numpy(case["sink"]).cuda(), softmax_scale=0.125)
    torch.cuda.synchronize()
    ro, rl = tidx._oracle_rows(case, 0.125)
    check_close("O", host64(o), ro, TOL_O)
    check_close("LSE", host64(lse), rl, TOL_LSE)
    del k, v


def test_varlen_forward_on_keys_past_4gib():
    """Packed K/V whose rows of the real sequences lie past 4 GiB: a first
    sequence with no queries owns the first 4 GiB of (never read) key rows."""
    need_gpu()
    import numpy as np

    import oracle
    from softmax_learnable_sink_amd import binding
    from tests.gpu_util import vals
    say("case: varlen forward B2 H8/2 D64 nq~U[1,300] causal sink behind a 4 GiB empty-query "
        "sequence, seed 11")
    case = synth.varlen_case(2, 8, 2, 64, 1, 300, None, None, seed=11)
    total_k, Hkv, D = case["k"].shape
    skip = (4 << 30) // (Hkv * D * 2) + 16  # rows of the query-less first sequence
    k = torch.empty((skip + total_k, Hkv, D), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((skip + total_k, Hkv, D), dtype=torch.bfloat16, device="cuda")
    k[skip:] = dev_tensor(case["k"], synth.BF16)
    v[skip:] = dev_tensor(case["v"], synth.BF16)
    cq = np.concatenate([[0], case["cu_seqlens_q"]]).astype(np.int32)
    ck = np.concatenate([[0], skip + case["cu_seqlens_k"]]).astype(np.int32)
    o, lse = binding.attn_sink_fwd_varlen(
        dev_tensor(case["q"], synth.BF16), k, v, tidx._i32(cq), tidx._i32(ck),
        case["max_seqlen_q"], torch.from_numpy(case["sink"]).cuda(), causal=True,
        softmax_scale=0.125)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_varlen(vals(case["q"], synth.BF16), case["cu_seqlens_q"],
                                   vals(case["k"], synth.BF16), vals(case["v"], synth.BF16),
                                   case["cu_seqlens_k"], case["sink"], 0.125, causal=True)
    check_close("O", host64(o), ro, TOL_O)
    check_close("LSE", host64(lse), rl, TOL_LSE)
    del k, v
