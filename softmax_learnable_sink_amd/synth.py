"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke run.

This module holds no attention arithmetic.  It draws N(0,1) tensors with
``numpy.random.default_rng(seed)``, rounds them to bfloat16 (round to nearest
even) when the case is bf16, and builds paged KV caches with a seeded random
page permutation.  The same bits go to the GPU library and to the CPU oracle.

bf16 tensors are returned as ``uint16`` bit patterns; ``bf16_to_f32`` gives
their exact float values.  fp32 tensors are returned as ``float32``.

Draw order (fixed, so a seed names one input set):
  prefill:  q, k, v, [dout], sink
  decode:   q, sink, context lengths, page permutation, k pool, v pool
  varlen:   q, k, v, [dout], sink (packed; lengths from rng((seed, 3000)))
  index:    the extend case of the same seed, then index lists from rng((seed, 4000))
Each N(0,1) tensor is drawn in blocks of 2^22 elements; block i of the n-th
tensor of a case comes from numpy.random.default_rng((seed, n, i)), so large
pools can be drawn by several threads with a result that does not depend on
the thread count.  The small integer draws (lengths, permutation) come from
numpy.random.default_rng((seed, 1000)).
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_BLOCK = 1 << 22

BF16 = "bf16"
F32 = "f32"


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest even) and return the bits."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    lsb = u >> 16
    lsb &= 1
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= 16
    return u.astype(np.uint16)


def bf16_to_f32(bits):
    """Exact float32 values of bfloat16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def values(x, dtype):
    """Exact float32 values of a synth tensor of the given dtype."""
    return bf16_to_f32(x) if dtype == BF16 else np.asarray(x, dtype=np.float32)


class _Draws:
    """Numbered N(0,1) tensors of one case (see the module docstring)."""

    def __init__(self, seed):
        self.seed = int(seed)
        self.n = 0

    def normal(self, shape, dtype):
        tid = self.n
        self.n += 1
        size = int(np.prod(shape))
        out = np.empty(size, dtype=np.uint16 if dtype == BF16 else np.float32)
        nblk = (size + _BLOCK - 1) // _BLOCK

        def fill(i):
            lo, hi = i * _BLOCK, min(size, (i + 1) * _BLOCK)
            x = np.random.default_rng((self.seed, tid, i)).standard_normal(hi - lo, dtype=np.float32)
            out[lo:hi] = f32_to_bf16_bits(x) if dtype == BF16 else x

        if nblk > 1:
            workers = min(16, len(os.sched_getaffinity(0)), nblk)
            with ThreadPoolExecutor(workers) as ex:
                list(ex.map(fill, range(nblk)))
        elif nblk == 1:
            fill(0)
        return out.reshape(shape)

    def sink(self, Hq):
        return self.normal((Hq,), F32)


def prefill_case(B, Sq, Sk, Hq, Hkv, D, dtype=BF16, seed=0, sink=True, dout=False):
    """Q [B,Sq,Hq,D], K/V [B,Sk,Hkv,D], optional dO [B,Sq,Hq,D], sink [Hq] fp32."""
    dr = _Draws(seed)
    case = {
        "dtype": dtype,
        "q": dr.normal((B, Sq, Hq, D), dtype),
        "k": dr.normal((B, Sk, Hkv, D), dtype),
        "v": dr.normal((B, Sk, Hkv, D), dtype),
    }
    if dout:
        case["dout"] = dr.normal((B, Sq, Hq, D), dtype)
    case["sink"] = dr.sink(Hq) if sink else None
    return case


def packed_lengths(total, lo, hi, seed=0):
    """Sequence lengths ~ U[lo, hi] drawn until they add up to `total` tokens;
    the last one is cut to fit (so it may be shorter than lo)."""
    rng = np.random.default_rng((int(seed), 3001))
    out, left = [], int(total)
    while left > 0:
        n = min(int(rng.integers(lo, hi, endpoint=True)), left)
        out.append(n)
        left -= n
    return np.asarray(out, dtype=np.int32)


def varlen_case(B, Hq, Hkv, D, q_lo=1, q_hi=1, k_lo=None, k_hi=None, dtype=BF16, seed=0,
                sink=True, dout=False, q_lens=None, k_lens=None):
    """Packed variable-length inputs: q [total_q,Hq,D], k/v [total_k,Hkv,D], optional
    dO [total_q,Hq,D], sink [Hq], cu_seqlens_q / cu_seqlens_k [B+1] int32.

    Sequence b has nq_b ~ U[q_lo, q_hi] queries (or `q_lens`) and nk_b keys:
    `k_lens` if given, else nk_b = nq_b when k_lo is None (self-attention),
    else U[k_lo, k_hi].
    """
    rng = np.random.default_rng((int(seed), 3000))
    if q_lens is None:
        q_lens = rng.integers(q_lo, q_hi, size=B, endpoint=True)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    if k_lens is None:
        k_lens = q_lens if k_lo is None else rng.integers(k_lo, k_hi, size=B, endpoint=True)
    k_lens = np.asarray(k_lens, dtype=np.int32)
    assert len(q_lens) == B and len(k_lens) == B
    cu_q = np.zeros(B + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(q_lens)
    cu_k = np.zeros(B + 1, dtype=np.int32)
    cu_k[1:] = np.cumsum(k_lens)
    dr = _Draws(seed)
    case = {
        "dtype": dtype,
        "q": dr.normal((int(cu_q[-1]), Hq, D), dtype),
        "k": dr.normal((int(cu_k[-1]), Hkv, D), dtype),
        "v": dr.normal((int(cu_k[-1]), Hkv, D), dtype),
    }
    if dout:
        case["dout"] = dr.normal((int(cu_q[-1]), Hq, D), dtype)
    case["sink"] = dr.sink(Hq) if sink else None
    case.update({"cu_seqlens_q": cu_q, "cu_seqlens_k": cu_k, "q_lens": q_lens, "k_lens": k_lens,
                 "max_seqlen_q": int(q_lens.max()) if B else 0,
                 "max_seqlen_k": int(k_lens.max()) if B else 0})
    return case


def decode_case(B, Hq, Hkv, D, page_size, len_lo, len_hi, dtype=BF16, seed=0,
                sink=True, max_len=None, lengths=None, nan_poison=False):
    """Paged decode inputs.

    Context lengths L_b ~ integers U[len_lo, len_hi] (inclusive), or `lengths`.
    Sequence b owns ceil(L_b / P) pages; a seeded random permutation of all
    page ids is handed out in order (b, page).  block_table is int32
    [B, ceil(max_len / P)] padded with -1.  Pools are [num_pages, P, Hkv, D].
    With nan_poison, the slots past L_b in each sequence's last page hold NaN.
    """
    dr = _Draws(seed)
    rng = np.random.default_rng((int(seed), 1000))
    case = {"dtype": dtype, "q": dr.normal((B, Hq, D), dtype)}
    case["sink"] = dr.sink(Hq) if sink else None
    if lengths is None:
        lengths = rng.integers(len_lo, len_hi, size=B, endpoint=True)
    lengths = np.asarray(lengths, dtype=np.int32)
    max_len = int(max_len if max_len is not None else max(len_hi, int(lengths.max())))
    npages = (lengths.astype(np.int64) + page_size - 1) // page_size
    total = int(npages.sum())
    perm = rng.permutation(total).astype(np.int32)
    max_pages = (max_len + page_size - 1) // page_size
    bt = np.full((B, max_pages), -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        n = int(npages[b])
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    shape = (total, page_size, Hkv, D)
    kc = dr.normal(shape, dtype)
    vc = dr.normal(shape, dtype)
    if nan_poison:
        nan = f32_to_bf16_bits(np.float32(np.nan)) if dtype == BF16 else np.float32(np.nan)
        for b in range(B):
            L = int(lengths[b])
            last = L - 1
            page = bt[b, last // page_size]
            off = last % page_size + 1
            kc[page, off:] = nan
            vc[page, off:] = nan
    case.update({"k_cache": kc, "v_cache": vc, "block_table": bt, "seqlens": lengths,
                 "page_size": page_size, "num_pages": total, "max_len": max_len})
    return case



def extend_case(B, Hq, Hkv, D, page_size, q_lo, q_hi, ctx_lo, ctx_hi, dtype=BF16, seed=0,
                sink=True, q_lens=None, ctx_lens=None, nan_poison=False):
    """Chunked-prefill inputs: packed new queries against a paged cache.

    Sequence b has nq_b ~ U[q_lo, q_hi] new tokens (or `q_lens`) on top of
    c_b ~ U[ctx_lo, ctx_hi] cached tokens (or `ctx_lens`); its context length
    is L_b = c_b + nq_b and its cache holds all L_b tokens.  q is packed
    [total_q, Hq, D] with cu_seqlens_q [B+1]; pages are handed out (and, with
    nan_poison, the slots past L_b poisoned) as in decode_case.
    """
    rng = np.random.default_rng((int(seed), 2000))
    if q_lens is None:
        q_lens = rng.integers(q_lo, q_hi, size=B, endpoint=True)
    if ctx_lens is None:
        ctx_lens = rng.integers(ctx_lo, ctx_hi, size=B, endpoint=True)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    L = np.asarray(ctx_lens, dtype=np.int32) + q_lens
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    case = decode_case(B, Hq, Hkv, D, page_size, 0, 0, dtype=dtype, seed=seed, sink=sink,
                       lengths=np.maximum(L, 1), nan_poison=nan_poison)
    dr = _Draws(seed)
    dr.n = 100  # a tensor number of its own: the packed queries
    case["q"] = dr.normal((int(cu[-1]), Hq, D), dtype)
    case.update({"cu_seqlens_q": cu, "seqlens": L, "q_lens": q_lens,
                 "max_seqlen_q": int(q_lens.max()) if B else 0})
    return case


def index_case(B, Hq, Hkv, D, page_size, q_lo, q_hi, ctx_lo, ctx_hi, block_q, topk, dtype=BF16,
               seed=0, sink=True, q_lens=None, ctx_lens=None, n_first=64, n_local=512,
               shuffle=False, pad=0, nan_poison=False):
    """Chunked-prefill inputs (as extend_case) plus one KV index list per block of
    block_q query rows of each sequence: kv_index [num_blocks, topk] int32 and
    cu_blocks [B+1] (sequence b's lists are rows cu_blocks[b] ..).

    For a block whose last row sits at position p1: if p1 + 1 <= topk - pad the
    list is every token 0..p1; otherwise it is the first n_first tokens, the
    n_local tokens ending at p1 (at most (topk - pad) / 8 and / 2 of them), and
    a uniform sample of the tokens between them, topk - pad entries in all.  Lists are ascending (or shuffled) and end
    in `pad` (or more) entries of -1.
    """
    case = extend_case(B, Hq, Hkv, D, page_size, q_lo, q_hi, ctx_lo, ctx_hi, dtype=dtype,
                       seed=seed, sink=sink, q_lens=q_lens, ctx_lens=ctx_lens,
                       nan_poison=nan_poison)
    rng = np.random.default_rng((int(seed), 4000))
    k_sel = topk - pad
    nq = case["q_lens"].astype(np.int64)
    L = case["seqlens"].astype(np.int64)
    nblk = (nq + block_q - 1) // block_q
    cu_b = np.zeros(B + 1, dtype=np.int32)
    cu_b[1:] = np.cumsum(nblk)
    lists = np.full((int(cu_b[-1]), topk), -1, dtype=np.int32)
    for b in range(B):
        for j in range(int(nblk[b])):
            p1 = int(L[b] - nq[b] + min(nq[b], (j + 1) * block_q) - 1)
            if p1 + 1 <= k_sel:
                sel = np.arange(max(p1 + 1, 0))
            else:
                nf, nl = min(n_first, k_sel // 8), min(n_local, k_sel // 2)
                first = np.arange(nf)
                local = np.arange(p1 + 1 - nl, p1 + 1)
                mid = np.arange(nf, p1 + 1 - nl)
                sel = np.concatenate([first, rng.choice(mid, k_sel - nf - nl, replace=False),
                                      local])
                sel.sort()
            if shuffle:
                sel = rng.permutation(sel)
            lists[cu_b[b] + j, :len(sel)] = sel
    case.update({"kv_index": lists, "cu_blocks": cu_b, "block_q": block_q, "topk": topk})
    return case
