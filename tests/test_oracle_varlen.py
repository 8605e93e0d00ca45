"""Pins of the oracle's packed variable-length forward and backward (CPU only).

The variable-length functions slice each sequence out of the packed tensors.
They are checked against routes that do not share that slicing: the batched
dense functions when every sequence has the same lengths, brute force per
sequence, central finite differences of the packed forward, and the
independence of one sequence's result from another sequence's data.
"""
import numpy as np
import pytest

import oracle


def _case(q_lens, k_lens, Hq=4, Hkv=2, D=3, seed=0, sink=True):
    rng = np.random.default_rng(seed)
    tq, tk = sum(q_lens), sum(k_lens)
    return dict(
        q=rng.standard_normal((tq, Hq, D)),
        k=rng.standard_normal((tk, Hkv, D)),
        v=rng.standard_normal((tk, Hkv, D)),
        dout=rng.standard_normal((tq, Hq, D)),
        sink=rng.standard_normal(Hq) if sink else None,
        cu_q=np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32),
        cu_k=np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int32),
    )


def _fwd(c, scale, causal, window):
    return oracle.prefill_varlen(c["q"], c["cu_q"], c["k"], c["v"], c["cu_k"], c["sink"], scale,
                                 causal, window)


def _bwd(c, scale, causal, window):
    return oracle.backward_varlen(c["q"], c["cu_q"], c["k"], c["v"], c["cu_k"], c["sink"],
                                  c["dout"], scale, causal, window)


@pytest.mark.parametrize("causal,window", [(True, None), (False, None), (True, (2, 3))])
def test_equal_lengths_equal_the_batched_functions(causal, window):
    # Sq != Sk so that query and key offsets differ
    B, Sq, Sk = 3, 5, 9
    c = _case([Sq] * B, [Sk] * B, seed=1)
    Hq, D = c["q"].shape[1:]
    Hkv = c["k"].shape[1]
    qb = c["q"].reshape(B, Sq, Hq, D)
    kb = c["k"].reshape(B, Sk, Hkv, D)
    vb = c["v"].reshape(B, Sk, Hkv, D)
    db = c["dout"].reshape(B, Sq, Hq, D)
    o, lse = _fwd(c, 0.7, causal, window)
    ro, rl = oracle.prefill(qb, kb, vb, c["sink"], 0.7, causal, window)
    np.testing.assert_array_equal(o, ro.reshape(B * Sq, Hq, D))
    np.testing.assert_array_equal(lse, rl.transpose(1, 0, 2).reshape(Hq, B * Sq))
    dq, dk, dv, ds, _, _ = _bwd(c, 0.7, causal, window)
    r = oracle.backward(qb, kb, vb, c["sink"], db, 0.7, causal, window)
    np.testing.assert_allclose(dq, r[0].reshape(dq.shape), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, r[1].reshape(dk.shape), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, r[2].reshape(dv.shape), rtol=0, atol=1e-13)
    np.testing.assert_allclose(ds, r[3], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal,window", [(True, None), (False, None), (True, (1, 2))])
def test_ragged_forward_matches_brute_force(causal, window):
    q_lens, k_lens = [3, 1, 6, 2], [5, 1, 6, 7]
    c = _case(q_lens, k_lens, seed=2)
    o, lse = _fwd(c, 0.6, causal, window)
    for b in range(len(q_lens)):
        a, e = c["cu_q"][b], c["cu_q"][b + 1]
        ka, ke = c["cu_k"][b], c["cu_k"][b + 1]
        ro, rl = oracle.prefill_bruteforce(c["q"][None, a:e], c["k"][None, ka:ke],
                                           c["v"][None, ka:ke], c["sink"], 0.6, causal, window)
        np.testing.assert_allclose(o[a:e], ro[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[:, a:e], rl[0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal,window", [(True, None), (False, None), (True, (1, 2))])
def test_backward_matches_finite_differences(causal, window):
    # ragged, with a sequence that has no query row and one whose first rows
    # sit before its first key (Sq > Sk)
    c = _case([2, 0, 3, 4], [3, 2, 4, 2], Hq=2, Hkv=1, D=3, seed=3)
    scale = 0.9
    dq, dk, dv, dsink, _, _ = _bwd(c, scale, causal, window)

    def loss():
        o, _ = _fwd(c, scale, causal, window)
        return float(np.sum(o * c["dout"]))

    for got, name in ((dq, "q"), (dk, "k"), (dv, "v"), (dsink, "sink")):
        x = c[name]
        ref = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + 1e-6
            fp = loss()
            x[idx] = old - 1e-6
            fm = loss()
            x[idx] = old
            ref[idx] = (fp - fm) / 2e-6
        assert np.max(np.abs(got - ref)) < 1e-8 * max(1.0, np.max(np.abs(ref))), name
    # keys of the sequence without queries get no gradient
    assert np.all(dk[3:5] == 0) and np.all(dv[3:5] == 0)


def test_sequences_do_not_see_each_other():
    q_lens, k_lens = [4, 3, 5], [6, 2, 5]
    c = _case(q_lens, k_lens, seed=4)
    o1, l1 = _fwd(c, 0.5, True, None)
    g1 = _bwd(c, 0.5, True, None)
    # replace every input of sequence 1
    c2 = {n: (x.copy() if isinstance(x, np.ndarray) else x) for n, x in c.items()}
    rng = np.random.default_rng(99)
    qa, qe = c["cu_q"][1], c["cu_q"][2]
    ka, ke = c["cu_k"][1], c["cu_k"][2]
    c2["q"][qa:qe] = rng.standard_normal(c2["q"][qa:qe].shape)
    c2["k"][ka:ke] = rng.standard_normal(c2["k"][ka:ke].shape)
    c2["v"][ka:ke] = rng.standard_normal(c2["v"][ka:ke].shape)
    c2["dout"][qa:qe] = rng.standard_normal(c2["dout"][qa:qe].shape)
    o2, l2 = _fwd(c2, 0.5, True, None)
    g2 = _bwd(c2, 0.5, True, None)
    keep_q = np.r_[0:qa, qe:len(c["q"])]
    keep_k = np.r_[0:ka, ke:len(c["k"])]
    np.testing.assert_array_equal(o1[keep_q], o2[keep_q])
    np.testing.assert_array_equal(l1[:, keep_q], l2[:, keep_q])
    np.testing.assert_array_equal(g1[0][keep_q], g2[0][keep_q])
    np.testing.assert_array_equal(g1[1][keep_k], g2[1][keep_k])
    np.testing.assert_array_equal(g1[2][keep_k], g2[2][keep_k])
    assert not np.array_equal(o1[qa:qe], o2[qa:qe])


@pytest.mark.parametrize("sink", [True, False])
def test_sequence_without_keys(sink):
    # sequence 1 has queries but no key: O = 0, LSE = sink (or -inf), no grads
    c = _case([2, 3, 1], [4, 0, 2], seed=5, sink=sink)
    for causal in (True, False):
        o, lse = _fwd(c, 0.5, causal, None)
        np.testing.assert_array_equal(o[2:5], 0.0)
        ref = (np.repeat(c["sink"][:, None], 3, axis=1) if sink
               else np.full((4, 3), -np.inf))
        np.testing.assert_array_equal(lse[:, 2:5], ref)
        dq, dk, dv, ds, _, _ = _bwd(c, 0.5, causal, None)
        np.testing.assert_array_equal(dq[2:5], 0.0)
        # its rows have Di = <dO, O> = 0, so dsink equals that of the batch
        # without the sequence
        c3 = dict(c)
        c3["q"] = np.delete(c["q"], np.s_[2:5], axis=0)
        c3["dout"] = np.delete(c["dout"], np.s_[2:5], axis=0)
        c3["cu_q"] = np.array([0, 2, 3], dtype=np.int32)
        c3["cu_k"] = np.array([0, 4, 6], dtype=np.int32)
        r3 = _bwd(c3, 0.5, causal, None)
        np.testing.assert_allclose(ds, r3[3], rtol=1e-13, atol=0)
        np.testing.assert_array_equal(dk, r3[1])
