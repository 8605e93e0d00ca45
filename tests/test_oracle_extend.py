"""Pins of the oracle's chunked-prefill (extend) path against independent routes.

The extend oracle gathers a sequence's whole context from the paged cache and
applies the prefill definition at the new tokens' positions.  It is checked
against: the decode oracle (a different route, by token selection, for the
newest token), dense prefill on K/V the test writes into pages itself, and
properties that hold for any paging.
"""
import numpy as np
import pytest

import oracle
from softmax_learnable_sink_amd import synth


def _f64(case, name):
    return synth.values(case[name], case["dtype"])


def _extend(case, scale, window):
    return oracle.extend_paged(_f64(case, "q"), case["cu_seqlens_q"], _f64(case, "k_cache"),
                               _f64(case, "v_cache"), case["block_table"], case["seqlens"],
                               case["sink"], scale, window)


@pytest.mark.parametrize("window", [None, (4, 9)])
def test_newest_token_equals_decode(window):
    # one new token per sequence: the extend rule at position L-1 must select
    # exactly the decode path's tokens ([window] Code Review rule)
    B = 5
    c = synth.extend_case(B, 8, 2, 16, 4, 1, 1, 0, 40, dtype=synth.F32, seed=3,
                          ctx_lens=[0, 3, 12, 13, 40])
    o, lse = _extend(c, 0.3, window)
    od, ld = oracle.decode_paged(_f64(c, "q"), _f64(c, "k_cache"), _f64(c, "v_cache"),
                                 c["block_table"], c["seqlens"], c["sink"], 0.3, window)
    np.testing.assert_allclose(o, od, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ld.T, rtol=0, atol=1e-12)


def test_all_new_tokens_equal_dense_prefill():
    # every token of each sequence is new; K/V are written into random pages
    # here, token by token, and the result must equal dense prefill
    rng = np.random.default_rng(7)
    Hq, Hkv, D, P = 6, 2, 8, 4
    lens = [5, 1, 17, 9]
    qs = [rng.standard_normal((L, Hq, D)) for L in lens]
    ks = [rng.standard_normal((L, Hkv, D)) for L in lens]
    vs = [rng.standard_normal((L, Hkv, D)) for L in lens]
    npages = [(L + P - 1) // P for L in lens]
    perm = rng.permutation(sum(npages))
    kc = np.full((sum(npages), P, Hkv, D), np.nan)
    vc = np.full((sum(npages), P, Hkv, D), np.nan)
    bt = np.full((len(lens), max(npages)), -1, dtype=np.int32)
    pos = 0
    for b, L in enumerate(lens):
        bt[b, :npages[b]] = perm[pos:pos + npages[b]]
        pos += npages[b]
        for t in range(L):
            kc[bt[b, t // P], t % P] = ks[b][t]
            vc[bt[b, t // P], t % P] = vs[b][t]
    cu = np.concatenate([[0], np.cumsum(lens)])
    sink = rng.standard_normal(Hq)
    o, lse = oracle.extend_paged(np.concatenate(qs), cu, kc, vc, bt, np.array(lens), sink, 0.4,
                                 None)
    for b, L in enumerate(lens):
        ro, rl = oracle.prefill(qs[b][None], ks[b][None], vs[b][None], sink, 0.4, causal=True)
        np.testing.assert_allclose(o[cu[b]:cu[b + 1]], ro[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[:, cu[b]:cu[b + 1]], rl[0], rtol=0, atol=1e-12)


def test_result_does_not_depend_on_page_layout():
    c = synth.extend_case(3, 4, 2, 16, 4, 2, 9, 0, 30, dtype=synth.F32, seed=5)
    o1, l1 = _extend(c, 0.25, (3, 6))
    # move every page to a new physical place
    n = c["k_cache"].shape[0]
    perm = np.random.default_rng(11).permutation(n)
    inv = np.argsort(perm)
    c2 = dict(c)
    c2["k_cache"] = c["k_cache"][inv]
    c2["v_cache"] = c["v_cache"][inv]
    bt = c["block_table"].copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    c2["block_table"] = bt
    o2, l2 = _extend(c2, 0.25, (3, 6))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_empty_sequence_and_rows_before_the_context():
    # sequence 1 has no new token; sequence 2 claims more new tokens than its
    # context holds, so its first rows sit at negative positions and see no key
    c = synth.extend_case(3, 4, 2, 8, 4, 0, 0, 0, 0, dtype=synth.F32, seed=9,
                          q_lens=[3, 0, 4], ctx_lens=[2, 5, 0])
    c["seqlens"] = np.array([5, 5, 2], dtype=np.int32)
    o, lse = _extend(c, 0.5, None)
    sink = c["sink"].astype(np.float64)
    # rows 3, 4 (sequence 2, positions -2, -1): O = 0, LSE = sink
    np.testing.assert_array_equal(o[3:5], 0.0)
    np.testing.assert_allclose(lse[:, 3:5], np.repeat(sink[:, None], 2, axis=1), atol=0)
    # its last two rows see keys 0 and 0..1
    assert np.all(np.abs(o[5:]) > 0)
    assert o.shape == (7, 4, 8) and lse.shape == (4, 7)
