"""Pins of the oracle's index-list selection (CPU only).

index_paged attends, per block of query rows, to a list of token positions.
It is checked against the extend oracle (full lists; per-row window lists),
per-row brute force on the listed keys, and properties that hold for any list
(order, empty entries, page layout).
"""
import numpy as np
import pytest

import oracle
from softmax_learnable_sink_amd import synth


def _f64(c, name):
    return synth.values(c[name], c["dtype"])


def _index(c, kv_index, cu_blocks, block_q, scale=0.3):
    return oracle.index_paged(_f64(c, "q"), c["cu_seqlens_q"], _f64(c, "k_cache"),
                              _f64(c, "v_cache"), c["block_table"], c["seqlens"], kv_index,
                              cu_blocks, block_q, c["sink"], scale)


def _extend(c, window=None, scale=0.3):
    return oracle.extend_paged(_f64(c, "q"), c["cu_seqlens_q"], _f64(c, "k_cache"),
                               _f64(c, "v_cache"), c["block_table"], c["seqlens"], c["sink"],
                               scale, window)


def _case(seed=0, **kw):
    args = dict(B=3, Hq=6, Hkv=2, D=8, page_size=4, q_lo=1, q_hi=40, ctx_lo=0, ctx_hi=60,
                block_q=16, topk=32, dtype=synth.F32, seed=seed)
    args.update(kw)
    return synth.index_case(**args)


@pytest.mark.parametrize("block_q", [1, 7, 16])
def test_full_lists_equal_extend(block_q):
    # every block lists all L tokens (plus empty slots): causal extend
    c = _case(seed=1)
    L = c["seqlens"]
    nq = c["q_lens"]
    nblk = (nq + block_q - 1) // block_q
    cu_b = np.concatenate([[0], np.cumsum(nblk)]).astype(np.int32)
    lists = np.full((cu_b[-1], int(L.max()) + 5), -1, dtype=np.int32)
    for b in range(len(L)):
        lists[cu_b[b]:cu_b[b + 1], :L[b]] = np.arange(L[b])
    o, lse = _index(c, lists, cu_b, block_q)
    ro, rl = _extend(c)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [(2, 5), (0, 3), (6, 1)])
def test_per_row_window_lists_equal_windowed_extend(window):
    # block_q = 1 and row i lists the window selection of its own prefix
    c = _case(seed=2, ctx_hi=40)
    L, nq = c["seqlens"], c["q_lens"]
    cu_b = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    lists = np.full((cu_b[-1], int(L.max())), -1, dtype=np.int32)
    for b in range(len(L)):
        for i in range(nq[b]):
            p = L[b] - nq[b] + i
            sel = oracle.select_tokens(p + 1, window) if p >= 0 else []
            lists[cu_b[b] + i, :len(sel)] = sel
    o, lse = _index(c, lists, cu_b, 1)
    ro, rl = _extend(c, window)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_rows_match_brute_force_over_their_listed_keys():
    c = _case(seed=3, B=2, Hq=4, Hkv=2, D=3, q_lo=5, q_hi=12, ctx_lo=20, ctx_hi=40, block_q=4,
              topk=12, shuffle=True, pad=2)
    o, lse = _index(c, c["kv_index"], c["cu_blocks"], 4, scale=0.7)
    q = _f64(c, "q")
    ks, vs = oracle.gather_kv(_f64(c, "k_cache"), _f64(c, "v_cache"), c["block_table"],
                              c["seqlens"], 4, None)
    cu, cb = c["cu_seqlens_q"], c["cu_blocks"]
    for b in range(2):
        L, nq = int(c["seqlens"][b]), int(cu[b + 1] - cu[b])
        for i in range(nq):
            lst = c["kv_index"][cb[b] + i // 4]
            keep = [t for t in lst.tolist() if 0 <= t < L and t <= L - nq + i]
            ro, rl = oracle.prefill_bruteforce(q[None, cu[b] + i:cu[b] + i + 1],
                                               ks[b][None, keep], vs[b][None, keep], c["sink"],
                                               0.7, causal=False)
            np.testing.assert_allclose(o[cu[b] + i], ro[0, 0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[:, cu[b] + i], rl[0, :, 0], rtol=0, atol=1e-12)


def test_order_and_empty_entries_do_not_matter():
    c = _case(seed=4, topk=40, pad=8)
    o1, l1 = _index(c, c["kv_index"], c["cu_blocks"], 16)
    rng = np.random.default_rng(0)
    lists = c["kv_index"].copy()
    # shuffle each list, and overwrite empty slots with positions past L
    for r in range(len(lists)):
        lists[r] = rng.permutation(lists[r])
    lists[lists < 0] = 10 ** 6
    o2, l2 = _index(c, lists, c["cu_blocks"], 16)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_result_does_not_depend_on_page_layout():
    c = _case(seed=5)
    o1, l1 = _index(c, c["kv_index"], c["cu_blocks"], 16)
    n = c["k_cache"].shape[0]
    perm = np.random.default_rng(11).permutation(n)
    inv = np.argsort(perm)
    c2 = dict(c)
    c2["k_cache"] = c["k_cache"][inv]
    c2["v_cache"] = c["v_cache"][inv]
    bt = c["block_table"].copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    c2["block_table"] = bt
    o2, l2 = _index(c2, c["kv_index"], c["cu_blocks"], 16)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_rows_without_a_visible_listed_token():
    # the list holds only tokens after the block's rows: O = 0, LSE = sink
    c = _case(seed=6, B=1, q_lens=[8], ctx_lens=[20], block_q=8, topk=4)
    lists = np.array([[26, 27, -1, 40]], dtype=np.int32)  # rows sit at 20..27
    o, lse = _index(c, lists, np.array([0, 1], dtype=np.int32), 8)
    # rows at 20..25 see nothing; row 26 sees token 26, row 27 sees 26 and 27
    np.testing.assert_array_equal(o[:6], 0.0)
    np.testing.assert_array_equal(lse[:, :6], np.repeat(c["sink"][:, None], 6, axis=1))
    assert np.all(np.abs(o[6:]) > 0)
