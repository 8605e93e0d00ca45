"""The forward entry points inside a captured HIP graph: the library launches kernels
only (no allocation, no memset, no host synchronisation), so a serving loop can
capture a decode or prefill step and replay it.  Each replay must reproduce the
eager result bit for bit, with eager work and synchronisations between replays."""

import math

import pytest
import torch

from softmax_learnable_sink_amd import synth
from tests.gpu_util import dev_tensor, need_gpu, say

pytestmark = pytest.mark.gpu


def _replay_and_compare(capture_fn, outputs, eager_fn, replays=3):
    # eager reference (also the warm-up before capture)
    ref = [t.clone() for t in eager_fn()]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture_fn()
    for r in range(replays):
        for t in outputs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outputs, ref):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want), \
                f"replay {r} differs from the eager result"
        eager_fn()  # eager work between replays
        torch.cuda.synchronize()
    say(f"  {replays} replays equal the eager result bitwise")


@pytest.mark.parametrize("B,Hq,Hkv,D,lo,hi,window", [
    (130, 16, 8, 64, 100, 2100, None),       # many KV-head units: equal token ranges
    (3, 32, 8, 128, 9000, 12000, (1024, 2048)),  # few: chunks, with the first/last window
])
def test_paged_decode_replays_in_a_graph(B, Hq, Hkv, D, lo, hi, window):
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say(f"case: graph decode B{B} H{Hq}/{Hkv} D{D} L~U[{lo},{hi}] window={window}")
    c = synth.decode_case(B, Hq, Hkv, D, 16, lo, hi, seed=5)
    q, kc, vc = (dev_tensor(c[n], synth.BF16) for n in ("q", "k_cache", "v_cache"))
    bt = torch.from_numpy(c["block_table"]).cuda()
    sl = torch.from_numpy(c["seqlens"]).cuda()
    sink = torch.from_numpy(c["sink"]).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = binding.lib().attn_sink_decode_workspace_bytes(B, Hq, Hkv, D, 16, bt.shape[1],
                                                         *binding._window(window), 0)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    scale = 1 / math.sqrt(D)

    def run(out, l, w):
        return binding.attn_sink_fwd_decode_paged(q, kc, vc, bt, sl, sink, softmax_scale=scale,
                                                  window=window, out=out, lse=l, workspace=w)

    o2, lse2, ws2 = torch.empty_like(o), torch.empty_like(lse), torch.empty_like(ws)
    _replay_and_compare(lambda: run(o, lse, ws), [o, lse], lambda: run(o2, lse2, ws2))


def test_prefill_replays_in_a_graph():
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say("case: graph prefill B2 S700 H16/2 D64 causal")
    c = synth.prefill_case(2, 700, 700, 16, 2, 64, seed=6)
    q, k, v = (dev_tensor(c[n], synth.BF16) for n in ("q", "k", "v"))
    sink = torch.from_numpy(c["sink"]).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((2, 16, 700), dtype=torch.float32, device=q.device)

    def run(out, l):
        return binding.attn_sink_fwd_prefill(q, k, v, sink, causal=True, softmax_scale=0.125,
                                             out=out, lse=l)

    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    _replay_and_compare(lambda: run(o, lse), [o, lse], lambda: run(o2, lse2))


def test_backward_replays_in_a_graph():
    """The training backward (preprocess, one launch of dK/dV and dQ, dSink reduction)."""
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say("case: graph backward B1 S600 H16/2 D64 causal")
    c = synth.prefill_case(1, 600, 600, 16, 2, 64, seed=7, dout=True)
    q, k, v, do = (dev_tensor(c[n], synth.BF16) for n in ("q", "k", "v", "dout"))
    sink = torch.from_numpy(c["sink"]).cuda()
    o, lse = binding.attn_sink_fwd_prefill(q, k, v, sink, causal=True, softmax_scale=0.125)
    need = binding.lib().attn_sink_bwd_workspace_bytes(1, 600, 600, 16, 2, 64)

    def buffers():
        return (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                torch.empty_like(sink), torch.empty(max(need, 16), dtype=torch.uint8,
                                                    device=q.device))

    def run(bufs):
        dq, dk, dv, ds, ws = bufs
        return binding.attn_sink_bwd(q, k, v, o, do, lse, sink, causal=True, softmax_scale=0.125,
                                     dq=dq, dk=dk, dv=dv, dsink=ds, workspace=ws)

    cap, eager = buffers(), buffers()
    _replay_and_compare(lambda: run(cap), list(cap[:4]), lambda: run(eager))


def test_chunked_prefill_replays_in_a_graph():
    """The extend kernel's tiles are gathered straight into LDS and its key order
    depends on the workgroups resident per XCD (queried on the first call)."""
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say("case: graph extend B3 H16/2 D64 P16 q~U[1,300] ctx~U[0,900] window (40,200)")
    c = synth.extend_case(3, 16, 2, 64, 16, 1, 300, 0, 900, seed=8)
    q, kc, vc = (dev_tensor(c[n], synth.BF16) for n in ("q", "k_cache", "v_cache"))
    bt = torch.from_numpy(c["block_table"]).cuda()
    cu = torch.from_numpy(c["cu_seqlens_q"]).cuda()
    sl = torch.from_numpy(c["seqlens"]).cuda()
    sink = torch.from_numpy(c["sink"]).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((16, q.shape[0]), dtype=torch.float32, device=q.device)

    def run(out, l):
        return binding.attn_sink_fwd_extend_paged(q, kc, vc, bt, cu, sl, c["max_seqlen_q"], sink,
                                                  softmax_scale=0.125, window=(40, 200),
                                                  out=out, lse=l)

    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    _replay_and_compare(lambda: run(o, lse), [o, lse], lambda: run(o2, lse2))


def test_index_lists_replay_in_a_graph():
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say("case: graph index B2 H16/2 D64 P16 q~U[60,200] ctx~U[100,2000] block 128 topk 256")
    c = synth.index_case(2, 16, 2, 64, 16, 60, 200, 100, 2000, 128, 256, seed=4, shuffle=True)
    q, kc, vc = (dev_tensor(c[n], synth.BF16) for n in ("q", "k_cache", "v_cache"))
    i32 = {n: torch.from_numpy(c[n].astype("int32")).cuda()
           for n in ("block_table", "cu_seqlens_q", "seqlens", "kv_index", "cu_blocks")}
    sink = torch.from_numpy(c["sink"]).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((16, q.shape[0]), dtype=torch.float32, device=q.device)

    def run(out, l):
        return binding.attn_sink_fwd_index_paged(
            q, kc, vc, i32["block_table"], i32["cu_seqlens_q"], i32["seqlens"], c["max_seqlen_q"],
            i32["kv_index"], i32["cu_blocks"], c["block_q"], sink, softmax_scale=0.125, out=out,
            lse=l)

    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    _replay_and_compare(lambda: run(o, lse), [o, lse], lambda: run(o2, lse2))


def test_packed_training_replays_in_a_graph():
    """The packed forward and backward (their grids are sized by the longest
    sequence; workgroups past a sequence's rows exit at once)."""
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say("case: graph varlen fwd+bwd B4 H16/2 D64 q~U[1,300] causal")
    c = synth.varlen_case(4, 16, 2, 64, 1, 300, seed=6, dout=True)
    q, k, v, do = (dev_tensor(c[n], synth.BF16) for n in ("q", "k", "v", "dout"))
    cq = torch.from_numpy(c["cu_seqlens_q"]).cuda()
    ck = torch.from_numpy(c["cu_seqlens_k"]).cuda()
    sink = torch.from_numpy(c["sink"]).cuda()
    mq, mk = c["max_seqlen_q"], c["max_seqlen_k"]
    tq = q.shape[0]
    o, lse = torch.empty_like(q), torch.empty((16, tq), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ds = torch.empty_like(sink)
    ws = torch.empty(binding.attn_sink_bwd_varlen_workspace_bytes(4, tq, mq, 16),
                     dtype=torch.uint8, device=q.device)

    def run(outs):
        o_, l_, dq_, dk_, dv_, ds_ = outs
        binding.attn_sink_fwd_varlen(q, k, v, cq, ck, mq, sink, causal=True, softmax_scale=0.125,
                                     out=o_, lse=l_)
        binding.attn_sink_bwd_varlen(q, k, v, o_, do, l_, cq, ck, mq, mk, sink, causal=True,
                                     softmax_scale=0.125, dq=dq_, dk=dk_, dv=dv_, dsink=ds_,
                                     workspace=ws)
        return outs

    mine = [o, lse, dq, dk, dv, ds]
    other = [torch.empty_like(t) for t in mine]
    _replay_and_compare(lambda: run(mine), mine, lambda: run(other))


def test_index_rows_replay_in_a_graph():
    """Per-row lists run the decode kernels in list mode (workspace given)."""
    need_gpu()
    from softmax_learnable_sink_amd import binding
    say("case: graph index rows B2 H16/2 D64 P16 q~U[5,40] ctx~U[100,900] topk 128 shuffled")
    c = synth.index_case(2, 16, 2, 64, 16, 5, 40, 100, 900, 1, 128, seed=7, shuffle=True)
    q, kc, vc = (dev_tensor(c[n], synth.BF16) for n in ("q", "k_cache", "v_cache"))
    i32 = {n: torch.from_numpy(c[n].astype("int32")).cuda()
           for n in ("block_table", "cu_seqlens_q", "seqlens", "kv_index")}
    sink = torch.from_numpy(c["sink"]).cuda()
    tq = q.shape[0]
    ws = torch.empty(max(binding.attn_sink_index_rows_workspace_bytes(tq, 16, 2, 64, 128), 16),
                     dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((16, tq), dtype=torch.float32, device=q.device)

    def run(out, l):
        return binding.attn_sink_fwd_index_rows_paged(
            q, kc, vc, i32["block_table"], i32["cu_seqlens_q"], i32["seqlens"], i32["kv_index"],
            sink, softmax_scale=0.125, out=out, lse=l, workspace=ws)

    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    _replay_and_compare(lambda: run(o, lse), [o, lse], lambda: run(o2, lse2))
