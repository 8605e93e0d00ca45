"""GPU parity of attention over per-query-block KV index lists against the fp64
oracle."""

import numpy as np
import pytest
import torch

import oracle
from softmax_learnable_sink_amd import synth
from tests.gpu_util import TOL_LSE, TOL_O, check_close, dev_tensor, host64, need_gpu, say, vals

pytestmark = pytest.mark.gpu


def _i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _run(case, scale, use_sink=True, kv_index=None):
    from softmax_learnable_sink_amd import binding
    sink = torch.from_numpy(case["sink"]).cuda() if use_sink else None
    kv_index = case["kv_index"] if kv_index is None else kv_index
    o, lse = binding.attn_sink_fwd_index_paged(
        dev_tensor(case["q"], synth.BF16), dev_tensor(case["k_cache"], synth.BF16),
        dev_tensor(case["v_cache"], synth.BF16), _i32(case["block_table"]),
        _i32(case["cu_seqlens_q"]), _i32(case["seqlens"]), case["max_seqlen_q"], _i32(kv_index),
        _i32(case["cu_blocks"]), case["block_q"], sink, softmax_scale=scale)
    torch.cuda.synchronize()
    return host64(o), host64(lse)


def _oracle(case, scale, use_sink=True, kv_index=None, heads=None):
    q = vals(case["q"], synth.BF16)
    kc, vc = vals(case["k_cache"], synth.BF16), vals(case["v_cache"], synth.BF16)
    sink = case["sink"] if use_sink else None
    if heads is not None:  # one KV head and its query heads
        hq, hk = heads
        q, kc, vc = q[:, hq], kc[:, :, hk], vc[:, :, hk]
        sink = None if sink is None else sink[hq]
    kv_index = case["kv_index"] if kv_index is None else kv_index
    return oracle.index_paged(q, case["cu_seqlens_q"], kc, vc, case["block_table"],
                              case["seqlens"], kv_index, case["cu_blocks"], case["block_q"], sink,
                              scale)


@pytest.mark.parametrize("B,Hq,Hkv,D,P,qlo,qhi,clo,chi,bq,topk,shuffle,pad", [
    (3, 8, 2, 64, 16, 1, 300, 0, 3000, 64, 512, False, 0),     # ragged, sorted lists
    (2, 16, 2, 64, 1, 60, 200, 100, 2000, 128, 256, True, 20),  # page 1, shuffled, padded, g=8
    (2, 8, 2, 128, 16, 1, 150, 0, 2500, 64, 300, False, 7),    # D=128, ragged last tile
    (2, 4, 1, 64, 64, 50, 130, 0, 100, 64, 2048, False, 0),    # lists = whole prefix, topk max
    (2, 32, 8, 64, 16, 100, 260, 500, 1500, 192, 640, True, 0),  # block 192, 8 KV heads
])
@pytest.mark.parametrize("use_sink", [True, False])
def test_index_matches_oracle(B, Hq, Hkv, D, P, qlo, qhi, clo, chi, bq, topk, shuffle, pad,
                              use_sink):
    need_gpu()
    say(f"case: index B{B} H{Hq}/{Hkv} D{D} P{P} q~U[{qlo},{qhi}] ctx~U[{clo},{chi}] "
        f"block {bq} topk {topk} shuffle {shuffle} pad {pad} sink {use_sink} seed 9")
    case = synth.index_case(B, Hq, Hkv, D, P, qlo, qhi, clo, chi, bq, topk, seed=9,
                            shuffle=shuffle, pad=pad, nan_poison=True)
    scale = D ** -0.5
    o, lse = _run(case, scale, use_sink)
    ro, rl = _oracle(case, scale, use_sink)
    check_close("O", o, ro, TOL_O)
    check_close("LSE", lse, rl, TOL_LSE)


def test_index_edge_rows():
    # an empty sequence, rows before the context, and a block whose list holds
    # only tokens after its rows (or outside [0, L))
    need_gpu()
    say("case: index edges q=[3,0,70,64] ctx=[5,9,0,100] block 64 topk 64")
    case = synth.index_case(4, 8, 2, 64, 16, 0, 0, 0, 0, 64, 64, seed=4, q_lens=[3, 0, 70, 64],
                            ctx_lens=[5, 9, 0, 100])
    case["seqlens"] = np.array([8, 9, 40, 164], dtype=np.int32)
    lists = case["kv_index"].copy()
    lists[-1] = -1
    lists[-1, :4] = [150, 163, 164, 10 ** 6]  # rows sit at 100..163
    o, lse = _run(case, 0.125, kv_index=lists)
    ro, rl = _oracle(case, 0.125, kv_index=lists)
    check_close("O", o, ro, TOL_O)
    check_close("LSE", lse, rl, TOL_LSE)


def test_index_full_lists_equal_extend_kernel_on_gpu_to_tolerance():
    # lists naming every cached token: the result is causal chunked prefill
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say("case: index full lists vs extend B2 H8/2 D64 P16 block 64")
    case = synth.index_case(2, 8, 2, 64, 16, 100, 200, 300, 600, 64, 1024, seed=8)
    L, nq = case["seqlens"], case["q_lens"]
    lists = np.full_like(case["kv_index"], -1)
    cb = case["cu_blocks"]
    for b in range(2):
        lists[cb[b]:cb[b + 1], :L[b]] = np.arange(L[b])
    o, lse = _run(case, 0.125, kv_index=lists)
    oe, le = binding.attn_sink_fwd_extend_paged(
        dev_tensor(case["q"], synth.BF16), dev_tensor(case["k_cache"], synth.BF16),
        dev_tensor(case["v_cache"], synth.BF16), _i32(case["block_table"]),
        _i32(case["cu_seqlens_q"]), _i32(L), case["max_seqlen_q"],
        torch.from_numpy(case["sink"]).cuda(), softmax_scale=0.125)
    torch.cuda.synchronize()
    check_close("O vs extend", o, host64(oe), TOL_O)
    check_close("LSE vs extend", lse, host64(le), TOL_LSE)


def test_index_workload_one_head_group():
    # the benchmark's index-list workload: 2 sequences x 4096 new tokens on 4096
    # cached ones, 64/8 heads, D 64, page 16, lists of 2048 per 128 queries;
    # every output of KV head 0's group against the oracle on that group alone
    need_gpu()
    say("case: index workload B2 nq4096 ctx4096 H64/8 D64 P16 block 128 topk 2048, group 0")
    case = synth.index_case(2, 64, 8, 64, 16, 4096, 4096, 4096, 4096, 128, 2048, seed=0)
    o, lse = _run(case, 0.125)
    ro, rl = _oracle(case, 0.125, heads=(slice(0, 8), slice(0, 1)))
    check_close("O", o[:, :8], ro, TOL_O)
    check_close("LSE", lse[:8], rl, TOL_LSE)
