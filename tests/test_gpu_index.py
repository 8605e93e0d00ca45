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
    q, kc, vc = case["q"], case["k_cache"], case["v_cache"]
    sink = case["sink"] if use_sink else None
    if heads is not None:  # one KV head and its query heads (sliced before the upcast)
        hq, hk = heads
        q, kc, vc = q[:, hq], kc[:, :, hk], vc[:, :, hk]
        sink = None if sink is None else sink[hq]
    q, kc, vc = vals(q, synth.BF16), vals(kc, synth.BF16), vals(vc, synth.BF16)
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


# ---------------------------------------------------------------------------
# Per-query lists (one list per packed query row)
# ---------------------------------------------------------------------------

def _run_rows(case, scale, use_sink=True, kv_index=None):
    from softmax_learnable_sink_amd import binding
    sink = torch.from_numpy(case["sink"]).cuda() if use_sink else None
    kv_index = case["kv_index"] if kv_index is None else kv_index
    o, lse = binding.attn_sink_fwd_index_rows_paged(
        dev_tensor(case["q"], synth.BF16), dev_tensor(case["k_cache"], synth.BF16),
        dev_tensor(case["v_cache"], synth.BF16), _i32(case["block_table"]),
        _i32(case["cu_seqlens_q"]), _i32(case["seqlens"]), _i32(kv_index), sink,
        softmax_scale=scale)
    torch.cuda.synchronize()
    return host64(o), host64(lse)


def _oracle_rows(case, scale, use_sink=True, kv_index=None, heads=None):
    c = dict(case)
    c["cu_blocks"] = case["cu_seqlens_q"]
    c["block_q"] = 1
    return _oracle(c, scale, use_sink, kv_index, heads)


@pytest.mark.parametrize("B,Hq,Hkv,D,P,qlo,qhi,clo,chi,topk,shuffle,pad", [
    (3, 8, 2, 64, 16, 1, 40, 0, 3000, 256, False, 0),       # g=4, ragged
    (2, 16, 2, 128, 1, 5, 30, 100, 2000, 128, True, 10),    # D=128, page 1, shuffled, padded
    (2, 12, 4, 64, 16, 1, 20, 0, 100, 3000, False, 0),      # g=3, lists longer than contexts
    (4, 32, 2, 64, 16, 1, 8, 500, 5000, 2048, True, 0),     # g=16
    (2, 40, 2, 64, 64, 1, 8, 200, 800, 512, False, 0),      # g=20: two head groups per KV head
])
@pytest.mark.parametrize("use_sink", [True, False])
def test_index_rows_match_oracle(B, Hq, Hkv, D, P, qlo, qhi, clo, chi, topk, shuffle, pad,
                                 use_sink):
    need_gpu()
    say(f"case: index rows B{B} H{Hq}/{Hkv} D{D} P{P} q~U[{qlo},{qhi}] ctx~U[{clo},{chi}] "
        f"topk {topk} shuffle {shuffle} pad {pad} sink {use_sink} seed 12")
    case = synth.index_case(B, Hq, Hkv, D, P, qlo, qhi, clo, chi, 1, topk, seed=12,
                            shuffle=shuffle, pad=pad, nan_poison=True)
    scale = D ** -0.5
    o, lse = _run_rows(case, scale, use_sink)
    ro, rl = _oracle_rows(case, scale, use_sink)
    check_close("O", o, ro, TOL_O)
    check_close("LSE", lse, rl, TOL_LSE)


def test_index_rows_edge_rows():
    # an empty sequence, rows before the context, lists with no visible token
    need_gpu()
    say("case: index rows edges q=[3,0,5,4] ctx=[5,9,0,100] topk 16")
    case = synth.index_case(4, 8, 2, 64, 16, 0, 0, 0, 0, 1, 16, seed=4, q_lens=[3, 0, 5, 4],
                            ctx_lens=[5, 9, 0, 100])
    case["seqlens"] = np.array([8, 9, 3, 104], dtype=np.int32)
    lists = case["kv_index"].copy()
    lists[-1] = -1
    lists[-1, :3] = [103, 104, 10 ** 6]  # the last row sits at 103
    lists[-2] = -1                       # the row before it lists nothing
    o, lse = _run_rows(case, 0.125, kv_index=lists)
    ro, rl = _oracle_rows(case, 0.125, kv_index=lists)
    check_close("O", o, ro, TOL_O)
    check_close("LSE", lse, rl, TOL_LSE)


def test_index_rows_with_block_lists_equal_the_block_kernel():
    # every row of a 64-row block carries its block's list: both entry points
    # compute the same attention
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say("case: index rows == index blocks, B2 H8/2 D64 P16 block 64 topk 512")
    case = synth.index_case(2, 8, 2, 64, 16, 64, 200, 300, 900, 64, 512, seed=14)
    cu, cb = case["cu_seqlens_q"], case["cu_blocks"]
    rows = np.concatenate([case["kv_index"][cb[b] + np.arange(cu[b + 1] - cu[b]) // 64]
                           for b in range(2)])
    o1, l1 = _run(case, 0.125)
    o2, l2 = _run_rows(case, 0.125, kv_index=rows)
    check_close("O rows vs blocks", o2, o1, TOL_O)
    check_close("LSE rows vs blocks", l2, l1, TOL_LSE)


def test_index_rows_decode_workload():
    # the benchmark's per-query workload: 64 sequences, one new token each on a
    # U[4096, 32768] context, lists of 2048 positions, 64/8 heads, D 64, page 16
    need_gpu()
    say("case: index rows decode workload B64 ctx~U[4096,32768] topk 2048 H64/8 D64 P16 seed 0")
    case = synth.index_case(64, 64, 8, 64, 16, 1, 1, 4096, 32768, 1, 2048, seed=0)
    o, lse = _run_rows(case, 0.125)
    # every row, KV head 0's group (the oracle on that group alone)
    ro, rl = _oracle_rows(case, 0.125, heads=(slice(0, 8), slice(0, 1)))
    check_close("O", o[:, :8], ro, TOL_O)
    check_close("LSE", lse[:8], rl, TOL_LSE)
