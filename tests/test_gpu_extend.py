"""GPU parity of the chunked-prefill (extend) path against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from softmax_learnable_sink_amd import synth
from tests.gpu_util import TOL_LSE, TOL_O, check_close, dev_tensor, host64, need_gpu, say, vals

pytestmark = pytest.mark.gpu


def _run(case, scale, window, use_sink=True):
    from softmax_learnable_sink_amd import binding
    sink = torch.from_numpy(case["sink"]).cuda() if use_sink else None
    o, lse = binding.attn_sink_fwd_extend_paged(
        dev_tensor(case["q"], synth.BF16), dev_tensor(case["k_cache"], synth.BF16),
        dev_tensor(case["v_cache"], synth.BF16), torch.from_numpy(case["block_table"]).cuda(),
        torch.from_numpy(case["cu_seqlens_q"]).cuda(), torch.from_numpy(case["seqlens"]).cuda(),
        case["max_seqlen_q"], sink, softmax_scale=scale, window=window)
    torch.cuda.synchronize()
    return host64(o), host64(lse)


def _oracle(case, scale, window, use_sink=True):
    return oracle.extend_paged(vals(case["q"], synth.BF16), case["cu_seqlens_q"],
                               vals(case["k_cache"], synth.BF16), vals(case["v_cache"], synth.BF16),
                               case["block_table"], case["seqlens"],
                               case["sink"] if use_sink else None, scale, window)


@pytest.mark.parametrize("B,Hq,Hkv,D,P,qlo,qhi,clo,chi,window", [
    (3, 8, 2, 64, 16, 1, 150, 0, 300, None),          # g=4, ragged tiles, page 16
    (2, 16, 2, 64, 1, 60, 200, 100, 400, None),       # g=8, page size 1
    (3, 6, 3, 64, 64, 1, 90, 0, 200, None),           # g=2, page 64
    (2, 3, 1, 64, 16, 20, 80, 0, 100, None),          # g=3: one head per wave
    (2, 8, 2, 128, 16, 1, 140, 0, 250, None),         # D=128
    (2, 8, 2, 64, 16, 100, 200, 300, 500, (40, 90)),  # first/last window
    (2, 8, 1, 128, 8, 50, 120, 200, 400, (16, 64)),   # window, D=128, g=8
    (2, 8, 2, 64, 256, 30, 200, 300, 1000, None),     # page 256: four tiles per page
    (2, 8, 1, 128, 128, 50, 150, 200, 700, (16, 64)),  # page 128, window, D=128
])
@pytest.mark.parametrize("use_sink", [True, False])
def test_extend_matches_oracle(B, Hq, Hkv, D, P, qlo, qhi, clo, chi, window, use_sink):
    need_gpu()
    say(f"case: extend B{B} H{Hq}/{Hkv} D{D} P{P} q~U[{qlo},{qhi}] ctx~U[{clo},{chi}] "
        f"window {window} sink {use_sink} seed 7")
    case = synth.extend_case(B, Hq, Hkv, D, P, qlo, qhi, clo, chi, seed=7, nan_poison=True)
    scale = D ** -0.5
    o, lse = _run(case, scale, window, use_sink)
    ro, rl = _oracle(case, scale, window, use_sink)
    check_close("O", o, ro, TOL_O)
    check_close("LSE", lse, rl, TOL_LSE)


def test_extend_empty_sequences_and_rows_before_the_context():
    need_gpu()
    say("case: extend edge rows (empty sequence, 70 rows on a 40-token context, single token)")
    case = synth.extend_case(4, 8, 2, 64, 16, 0, 0, 0, 0, seed=3, q_lens=[3, 0, 70, 1],
                             ctx_lens=[5, 9, 0, 0])
    case["seqlens"] = np.array([8, 9, 40, 1], dtype=np.int32)
    o, lse = _run(case, 0.125, None)
    ro, rl = _oracle(case, 0.125, None)
    check_close("O", o, ro, TOL_O)
    check_close("LSE", lse, rl, TOL_LSE)


def test_extend_chunked_prefill_workload_sampled_rows():
    # the chunked-prefill workload of the benchmark: 2 sequences x 4096 new
    # tokens on 4096..12288 cached ones, 64/8 heads, D 64, page 16, sink
    need_gpu()
    say("case: extend B2 nq4096 ctx~U[4096,12288] H64/8 D64 P16 sink, sampled rows, seed 0")
    case = synth.extend_case(2, 64, 8, 64, 16, 4096, 4096, 4096, 12288, seed=0)
    o, lse = _run(case, 0.125, None)
    kc, vc = vals(case["k_cache"], synth.BF16), vals(case["v_cache"], synth.BF16)
    q = vals(case["q"], synth.BF16)
    cu, L = case["cu_seqlens_q"], case["seqlens"]
    rng = np.random.default_rng(1)
    for b in range(2):
        nq = int(cu[b + 1] - cu[b])
        for i in [0, 1, 63, 64, nq - 1] + list(rng.integers(0, nq, 4)):
            p = int(L[b]) - nq + int(i)  # the row's position: it sees keys 0 .. p
            r = int(cu[b]) + int(i)
            ro, rl = oracle.extend_paged(q[r:r + 1], np.array([0, 1]), kc, vc,
                                         case["block_table"][b:b + 1], np.array([p + 1]),
                                         case["sink"], 0.125, None)
            check_close(f"O[b{b},i{i}]", o[r:r + 1], ro, TOL_O)
            check_close(f"LSE[b{b},i{i}]", lse[:, r:r + 1], rl, TOL_LSE)
