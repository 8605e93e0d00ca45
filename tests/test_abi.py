"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments on the host before any HIP call
(fake, never-dereferenced addresses are used for the pointer arguments)."""

import ctypes
import os
import re

import pytest

from softmax_learnable_sink_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_sink.h")

P = ctypes.c_void_p(0x10000)   # 16-byte aligned fake address, never dereferenced
P_ODD = ctypes.c_void_p(0x10002)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from softmax_learnable_sink_amd import build
        build.build()
    return binding.lib()


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(attn_sink_\w+)\s*\(", text,
                                 re.M)))


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for n in ("attn_sink_fwd_prefill", "attn_sink_fwd_decode_paged", "attn_sink_bwd",
              "attn_sink_fwd_extend_paged", "attn_sink_fwd_varlen", "attn_sink_bwd_varlen",
              "attn_sink_bwd_varlen_workspace_bytes", "attn_sink_fwd_index_paged",
              "attn_sink_fwd_index_rows_paged", "attn_sink_index_rows_workspace_bytes",
              "attn_sink_decode_workspace_bytes", "attn_sink_bwd_workspace_bytes",
              "attn_sink_decode_select_slots", "attn_sink_gather_kv", "attn_sink_last_error",
              "attn_sink_abi_version", "attn_sink_fwd_decode_paged_noalloc"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), f"{name} not exported"


def test_abi_version(lib):
    text = open(HEADER).read()
    v = int(re.search(r"#define ATTN_SINK_ABI_VERSION (\d+)", text).group(1))
    assert binding.abi_version() == v


def _prefill(lib, **kw):
    a = dict(q=P, k=P, v=P, sink=None, o=P, lse=None, B=1, Sq=8, Sk=8, Hq=4, Hkv=2, D=64,
             scale=0.125, causal=1, w1=-1, w2=-1, dtype=binding.BF16)
    a.update(kw)
    return lib.attn_sink_fwd_prefill(a["q"], a["k"], a["v"], a["sink"], a["o"], a["lse"], a["B"],
                                     a["Sq"], a["Sk"], a["Hq"], a["Hkv"], a["D"], a["scale"],
                                     a["causal"], a["w1"], a["w2"], a["dtype"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q=None), binding.ERR_INVALID_ARG, "must not be NULL"),
    (dict(o=None), binding.ERR_INVALID_ARG, "must not be NULL"),
    (dict(B=0), binding.ERR_INVALID_ARG, "B >= 1"),
    (dict(Sq=0), binding.ERR_INVALID_ARG, "Sq >= 1"),
    (dict(Hq=6, Hkv=4), binding.ERR_INVALID_ARG, "multiple of Hkv"),
    (dict(D=96), binding.ERR_UNSUPPORTED, "64 or 128"),
    (dict(scale=0.0), binding.ERR_INVALID_ARG, "softmax_scale"),
    (dict(scale=float("nan")), binding.ERR_INVALID_ARG, "softmax_scale"),
    (dict(w1=4, w2=0), binding.ERR_INVALID_ARG, "window"),
    (dict(w1=-2, w2=5), binding.ERR_INVALID_ARG, "window"),
    (dict(w1=4, w2=8, causal=0), binding.ERR_UNSUPPORTED, "causal"),
    (dict(causal=2), binding.ERR_INVALID_ARG, "causal"),
    (dict(dtype=7), binding.ERR_UNSUPPORTED, "dtype"),
    (dict(q=P_ODD), binding.ERR_INVALID_ARG, "aligned"),
    (dict(B=70000, Sq=1, Sk=1), binding.ERR_UNSUPPORTED, "B must be <="),
    (dict(Sk=1 << 22, Hkv=8, Hq=8, D=128), binding.ERR_UNSUPPORTED, "4 GiB"),
])
def test_prefill_rejects(lib, kw, status, msg):
    assert _prefill(lib, **kw) == status
    assert msg in binding.last_error()


def _decode(lib, **kw):
    a = dict(B=2, Hq=8, Hkv=2, D=64, P=16, maxp=4, npages=8, scale=0.125, w1=-1, w2=-1, ns=0,
             ws=P, wsb=1 << 20, dtype=binding.BF16, q=P, bt=P, sl=P)
    a.update(kw)
    return lib.attn_sink_fwd_decode_paged(a["q"], P, P, a["bt"], a["sl"], None, P, None, a["B"],
                                          a["Hq"], a["Hkv"], a["D"], a["P"], a["maxp"],
                                          a["npages"], a["scale"], a["w1"], a["w2"], a["ns"],
                                          a["ws"], a["wsb"], a["dtype"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(P=12), binding.ERR_UNSUPPORTED, "power of two"),
    (dict(P=512), binding.ERR_UNSUPPORTED, "power of two"),
    (dict(D=32), binding.ERR_UNSUPPORTED, "64 or 128"),
    (dict(Hq=9), binding.ERR_INVALID_ARG, "multiple of Hkv"),
    (dict(maxp=0), binding.ERR_INVALID_ARG, "max_pages_per_seq"),
    (dict(npages=0), binding.ERR_INVALID_ARG, "num_pages"),
    (dict(ns=-1), binding.ERR_INVALID_ARG, "num_splits"),
    (dict(ws=None), binding.ERR_WORKSPACE, "workspace"),
    (dict(wsb=16), binding.ERR_WORKSPACE, "too small"),
    (dict(bt=None), binding.ERR_INVALID_ARG, "must not be NULL"),
    (dict(sl=None), binding.ERR_INVALID_ARG, "must not be NULL"),
    (dict(dtype=binding.F32), binding.ERR_UNSUPPORTED, "bf16"),
    (dict(w1=3, w2=-1), binding.ERR_INVALID_ARG, "window"),
    (dict(B=70000, wsb=1 << 40), binding.ERR_UNSUPPORTED, "must each be <="),
])
def test_decode_rejects(lib, kw, status, msg):
    assert _decode(lib, **kw) == status
    assert msg in binding.last_error()


def _decode_noalloc(lib, **kw):
    a = dict(B=2, Hq=8, Hkv=2, D=64, P=16, maxp=4, npages=8, scale=0.125, w1=-1, w2=-1, ns=0,
             dtype=binding.BF16, q=P, bt=P, sl=P, o=P)
    a.update(kw)
    return lib.attn_sink_fwd_decode_paged_noalloc(
        a["q"], P, P, a["bt"], a["sl"], None, a["o"], None, a["B"], a["Hq"], a["Hkv"], a["D"],
        a["P"], a["maxp"], a["npages"], a["scale"], a["w1"], a["w2"], a["ns"], a["dtype"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(P=12), binding.ERR_UNSUPPORTED, "power of two"),
    (dict(D=32), binding.ERR_UNSUPPORTED, "64 or 128"),
    (dict(Hq=9), binding.ERR_INVALID_ARG, "multiple of Hkv"),
    (dict(npages=0), binding.ERR_INVALID_ARG, "num_pages"),
    (dict(ns=-1), binding.ERR_INVALID_ARG, "num_splits"),
    (dict(o=None), binding.ERR_INVALID_ARG, "must not be NULL"),
    (dict(q=P_ODD), binding.ERR_INVALID_ARG, "16-byte aligned"),
    (dict(dtype=binding.F32), binding.ERR_UNSUPPORTED, "bf16"),
    (dict(w1=3, w2=-1), binding.ERR_INVALID_ARG, "window"),
    (dict(scale=float("nan")), binding.ERR_INVALID_ARG, "softmax_scale"),
    # equal token ranges over 256 sequences at D 128 need 64 * 1280 * 130 * 4 B > 32 MiB
    (dict(B=256, Hq=64, Hkv=8, D=128, maxp=2048, npages=1 << 16), binding.ERR_UNSUPPORTED,
     "scratch"),
])
def test_decode_noalloc_rejects(lib, kw, status, msg):
    assert _decode_noalloc(lib, **kw) == status
    assert msg in binding.last_error()


def test_decode_noalloc_scratch_limit(lib):
    text = open(HEADER).read()
    m = re.search(r"#define ATTN_SINK_DECODE_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.DECODE_SCRATCH_BYTES
    # the benchmark's decode workloads fit the scratch
    assert 0 < binding.attn_sink_decode_workspace_bytes(64, 64, 8, 64, 16, 2048) <= \
        binding.DECODE_SCRATCH_BYTES
    assert 0 < binding.attn_sink_decode_workspace_bytes(32, 32, 8, 128, 16, 4096, (1024, 7168)) <= \
        binding.DECODE_SCRATCH_BYTES
    assert binding.attn_sink_decode_workspace_bytes(256, 64, 8, 128, 16, 2048) > \
        binding.DECODE_SCRATCH_BYTES


def test_decode_workspace_query(lib):
    # 64 sequences of up to 2048 pages of 16 tokens, 64/8 heads, D 64
    # default (num_splits 0, at most 256 sequences): equal token ranges per workgroup,
    # fp32 partials [Hq, 1024 + B, D + 2], then the sequences' starts [B + 1]
    n = binding.attn_sink_decode_workspace_bytes(64, 64, 8, 64, 16, 2048)
    assert n == 64 * (1024 + 64) * 66 * 4 + 65 * 4
    # an explicit split count: fp32 partials [B, Hq, splits, D + 2], then the chunk list
    # [B * splits] and its length
    splits = 16
    n = binding.attn_sink_decode_workspace_bytes(64, 64, 8, 64, 16, 2048, None, splits)
    assert n == 64 * 64 * splits * 66 * 4 + (64 * splits + 1) * 4
    # with chunks the window caps the selected length, so the workspace shrinks
    assert binding.attn_sink_decode_workspace_bytes(300, 64, 8, 64, 16, 2048, (1024, 7168)) < \
        binding.attn_sink_decode_workspace_bytes(300, 64, 8, 64, 16, 2048)
    # more requested splits never need less workspace
    a = binding.attn_sink_decode_workspace_bytes(4, 8, 2, 64, 16, 64, None, 2)
    b = binding.attn_sink_decode_workspace_bytes(4, 8, 2, 64, 16, 64, None, 8)
    assert 0 < a < b
    # little work (1 sequence, 32/8 heads, D 128, the 1024 + 7168 window: 8 units x 4
    # chunks of 2048): 128-token chunks instead of equal ranges
    n = binding.attn_sink_decode_workspace_bytes(1, 32, 8, 128, 16, 4096, (1024, 7168))
    assert n == 32 * 64 * 130 * 4 + (64 + 1) * 4
    # more than 256 sequences: 2048-token chunks
    n = binding.attn_sink_decode_workspace_bytes(300, 8, 2, 64, 16, 256)
    assert n == 300 * 8 * 2 * 66 * 4 + (300 * 2 + 1) * 4
    assert binding.attn_sink_decode_workspace_bytes(4, 8, 2, 96, 16, 64) == 0


def _extend(lib, **kw):
    a = dict(B=2, tq=10, mq=6, Hq=8, Hkv=2, D=64, P=16, maxp=4, npages=8, scale=0.125, w1=-1,
             w2=-1, dtype=binding.BF16, q=P, cu=P, sl=P, bt=P)
    a.update(kw)
    return lib.attn_sink_fwd_extend_paged(a["q"], P, P, a["bt"], a["cu"], a["sl"], None, P, None,
                                          a["B"], a["tq"], a["mq"], a["Hq"], a["Hkv"], a["D"],
                                          a["P"], a["maxp"], a["npages"], a["scale"], a["w1"],
                                          a["w2"], a["dtype"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dtype=binding.F32), binding.ERR_UNSUPPORTED, "bf16"),
    (dict(B=0), binding.ERR_INVALID_ARG, "B >= 1"),
    (dict(tq=-1), binding.ERR_INVALID_ARG, "total_q >= 0"),
    (dict(D=96), binding.ERR_UNSUPPORTED, "64 or 128"),
    (dict(Hq=9), binding.ERR_INVALID_ARG, "multiple of Hkv"),
    (dict(P=24), binding.ERR_UNSUPPORTED, "power of two"),
    (dict(npages=0), binding.ERR_INVALID_ARG, "num_pages"),
    (dict(cu=None), binding.ERR_INVALID_ARG, "must not be NULL"),
    (dict(q=P_ODD), binding.ERR_INVALID_ARG, "aligned"),
    (dict(w1=3, w2=0), binding.ERR_INVALID_ARG, "window"),
    (dict(scale=-1.0), binding.ERR_INVALID_ARG, "softmax_scale"),
])
def test_extend_rejects(lib, kw, status, msg):
    assert _extend(lib, **kw) == status
    assert msg in binding.last_error()


def test_extend_with_no_rows_is_a_no_op(lib):
    # no new query anywhere: accepted, and nothing is launched (no GPU needed)
    assert _extend(lib, tq=0, mq=0) == binding.OK


def _bwd(lib, **kw):
    a = dict(sink=None, dsink=None, B=1, Sq=8, Sk=8, Hq=4, Hkv=2, D=64, scale=0.125, causal=1,
             w1=-1, w2=-1, ws=P, wsb=1 << 20, dtype=binding.BF16, lse=P, dq=P)
    a.update(kw)
    return lib.attn_sink_bwd(P, P, P, P, P, a["lse"], a["sink"], a["dq"], P, P, a["dsink"], a["B"],
                             a["Sq"], a["Sk"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["causal"],
                             a["w1"], a["w2"], a["ws"], a["wsb"], a["dtype"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(sink=P), binding.ERR_INVALID_ARG, "dsink"),
    (dict(lse=None), binding.ERR_INVALID_ARG, "must not be NULL"),
    (dict(dq=None), binding.ERR_INVALID_ARG, "must not be NULL"),
    (dict(dtype=binding.F32), binding.ERR_UNSUPPORTED, "bf16"),
    (dict(wsb=4), binding.ERR_WORKSPACE, "too small"),
    (dict(ws=None), binding.ERR_WORKSPACE, "workspace"),
    (dict(Sk=0), binding.ERR_INVALID_ARG, "Sk >= 1"),
    (dict(D=256), binding.ERR_UNSUPPORTED, "64 or 128"),
    (dict(w1=2, w2=3, causal=0), binding.ERR_UNSUPPORTED, "causal"),
    (dict(B=70000, Sq=1, Sk=1, wsb=1 << 40), binding.ERR_UNSUPPORTED, "must each be <="),
    (dict(Sq=1 << 22, Hq=8, Hkv=8, D=128, wsb=1 << 40), binding.ERR_UNSUPPORTED, "4 GiB"),
])
def test_bwd_rejects(lib, kw, status, msg):
    assert _bwd(lib, **kw) == status
    assert msg in binding.last_error()


def test_bwd_workspace_query(lib):
    B, S, Hq = 2, 8192, 64
    n = binding.attn_sink_bwd_workspace_bytes(B, S, S, Hq, 8, 64)
    assert n == 4 * (2 * B * Hq * S + B * Hq * (S // 64))  # -Di, LSE log2 e, dSink partials
    assert binding.attn_sink_bwd_workspace_bytes(B, S, S, Hq, 7, 64) == 0


def _index(lib, **kw):
    a = dict(B=2, tq=10, mq=6, Hq=8, Hkv=2, D=64, P=16, maxp=4, npages=8, bq=64, topk=256,
             scale=0.125, dtype=binding.BF16, q=P, idx=P, cb=P)
    a.update(kw)
    return lib.attn_sink_fwd_index_paged(a["q"], P, P, P, P, P, a["idx"], a["cb"], None, P, None,
                                         a["B"], a["tq"], a["mq"], a["Hq"], a["Hkv"], a["D"],
                                         a["P"], a["maxp"], a["npages"], a["bq"], a["topk"],
                                         a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dtype=binding.F32), binding.ERR_UNSUPPORTED, "bf16"),
    (dict(B=0), binding.ERR_INVALID_ARG, "B >= 1"),
    (dict(Hq=6, Hkv=3), binding.ERR_UNSUPPORTED, "multiple of 4"),
    (dict(bq=96), binding.ERR_UNSUPPORTED, "multiple of 64"),
    (dict(bq=0), binding.ERR_UNSUPPORTED, "multiple of 64"),
    (dict(topk=0), binding.ERR_UNSUPPORTED, "topk"),
    (dict(topk=4096), binding.ERR_UNSUPPORTED, "topk"),
    (dict(D=96), binding.ERR_UNSUPPORTED, "64 or 128"),
    (dict(P=12), binding.ERR_UNSUPPORTED, "power of two"),
    (dict(idx=None), binding.ERR_INVALID_ARG, "must not be NULL"),
    (dict(cb=None), binding.ERR_INVALID_ARG, "must not be NULL"),
    (dict(q=P_ODD), binding.ERR_INVALID_ARG, "aligned"),
    (dict(scale=0.0), binding.ERR_INVALID_ARG, "softmax_scale"),
])
def test_index_rejects(lib, kw, status, msg):
    assert _index(lib, **kw) == status
    assert msg in binding.last_error()


def test_index_with_no_rows_is_a_no_op(lib):
    assert _index(lib, tq=0, mq=0) == binding.OK


def _index_rows(lib, **kw):
    a = dict(B=2, tq=10, Hq=8, Hkv=2, D=64, P=16, maxp=4, npages=8, topk=256, scale=0.125,
             dtype=binding.BF16, q=P, idx=P, ws=P, wsb=1 << 30)
    a.update(kw)
    return lib.attn_sink_fwd_index_rows_paged(a["q"], P, P, P, P, P, a["idx"], None, P, None,
                                              a["B"], a["tq"], a["Hq"], a["Hkv"], a["D"],
                                              a["P"], a["maxp"], a["npages"], a["topk"],
                                              a["scale"], a["ws"], a["wsb"], a["dtype"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dtype=binding.F32), binding.ERR_UNSUPPORTED, "bf16"),
    (dict(B=0), binding.ERR_INVALID_ARG, "B >= 1"),
    (dict(topk=0), binding.ERR_INVALID_ARG, "topk"),
    (dict(Hq=9), binding.ERR_INVALID_ARG, "multiple of Hkv"),
    (dict(P=12), binding.ERR_UNSUPPORTED, "power of two"),
    (dict(idx=None), binding.ERR_INVALID_ARG, "must not be NULL"),
    (dict(q=P_ODD), binding.ERR_INVALID_ARG, "aligned"),
    (dict(ws=None), binding.ERR_WORKSPACE, "workspace"),
    (dict(wsb=4), binding.ERR_WORKSPACE, "too small"),
])
def test_index_rows_rejects(lib, kw, status, msg):
    assert _index_rows(lib, **kw) == status
    assert msg in binding.last_error()


def test_index_rows_workspace_query(lib):
    # partials [rows, Hq, splits, D + 2] fp32 and the row -> sequence map
    n = binding.attn_sink_index_rows_workspace_bytes(64, 64, 8, 64, 2048)
    assert n == 64 * 64 * 1 * 66 * 4 + 64 * 4 or n > 64 * 64 * 66 * 4
    assert binding.attn_sink_index_rows_workspace_bytes(64, 64, 7, 64, 2048) == 0
    assert _index_rows(lib, tq=0) == binding.OK


def _fwd_varlen(lib, **kw):
    a = dict(B=2, tq=10, tk=12, mq=6, Hq=8, Hkv=2, D=64, scale=0.125, causal=1, w1=-1, w2=-1,
             dtype=binding.BF16, q=P, k=P, cq=P, ck=P)
    a.update(kw)
    return lib.attn_sink_fwd_varlen(a["q"], a["k"], a["k"], a["cq"], a["ck"], None, P, None,
                                    a["B"], a["tq"], a["tk"], a["mq"], a["Hq"], a["Hkv"], a["D"],
                                    a["scale"], a["causal"], a["w1"], a["w2"], a["dtype"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dtype=binding.F32), binding.ERR_UNSUPPORTED, "bf16"),
    (dict(B=0), binding.ERR_INVALID_ARG, "B >= 1"),
    (dict(tk=-1), binding.ERR_INVALID_ARG, "total_k >= 0"),
    (dict(D=96), binding.ERR_UNSUPPORTED, "64 or 128"),
    (dict(Hq=9), binding.ERR_INVALID_ARG, "multiple of Hkv"),
    (dict(ck=None), binding.ERR_INVALID_ARG, "must not be NULL"),
    (dict(k=None), binding.ERR_INVALID_ARG, "must not be NULL"),
    (dict(q=P_ODD), binding.ERR_INVALID_ARG, "aligned"),
    (dict(causal=2), binding.ERR_INVALID_ARG, "causal"),
    (dict(w1=1, w2=4, causal=0), binding.ERR_UNSUPPORTED, "causal"),
    (dict(tq=1 << 28, Hq=16, Hkv=2), binding.ERR_UNSUPPORTED, "32-bit"),
])
def test_fwd_varlen_rejects(lib, kw, status, msg):
    assert _fwd_varlen(lib, **kw) == status
    assert msg in binding.last_error()


def test_fwd_varlen_with_no_rows_is_a_no_op(lib):
    assert _fwd_varlen(lib, tq=0, mq=0) == binding.OK
    # no key at all: k and v may be NULL
    assert _fwd_varlen(lib, tq=0, mq=0, tk=0, k=None) == binding.OK


def _bwd_varlen(lib, **kw):
    a = dict(sink=None, dsink=None, B=2, tq=10, tk=12, mq=6, mk=8, Hq=4, Hkv=2, D=64, scale=0.125,
             causal=1, w1=-1, w2=-1, ws=P, wsb=1 << 20, dtype=binding.BF16, lse=P, dq=P, cq=P)
    a.update(kw)
    return lib.attn_sink_bwd_varlen(P, P, P, P, P, a["lse"], a["sink"], a["cq"], P, a["dq"], P, P,
                                    a["dsink"], a["B"], a["tq"], a["tk"], a["mq"], a["mk"],
                                    a["Hq"], a["Hkv"], a["D"], a["scale"], a["causal"], a["w1"],
                                    a["w2"], a["ws"], a["wsb"], a["dtype"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(sink=P), binding.ERR_INVALID_ARG, "dsink"),
    (dict(lse=None), binding.ERR_INVALID_ARG, "must not be NULL"),
    (dict(cq=None), binding.ERR_INVALID_ARG, "must not be NULL"),
    (dict(dtype=binding.F32), binding.ERR_UNSUPPORTED, "bf16"),
    (dict(wsb=4), binding.ERR_WORKSPACE, "too small"),
    (dict(ws=None), binding.ERR_WORKSPACE, "workspace"),
    (dict(mk=-1), binding.ERR_INVALID_ARG, ">= 0"),
    (dict(D=256), binding.ERR_UNSUPPORTED, "64 or 128"),
    (dict(w1=2, w2=3, causal=0), binding.ERR_UNSUPPORTED, "causal"),
    (dict(B=70000, wsb=1 << 40), binding.ERR_UNSUPPORTED, "must each be <="),
    (dict(mq=1 << 22, Hq=8, Hkv=8, D=128, wsb=1 << 40), binding.ERR_UNSUPPORTED, "4 GiB"),
])
def test_bwd_varlen_rejects(lib, kw, status, msg):
    assert _bwd_varlen(lib, **kw) == status
    assert msg in binding.last_error()


def test_bwd_varlen_workspace_query(lib):
    B, tq, mq, Hq = 3, 5000, 4096, 16
    n = binding.attn_sink_bwd_varlen_workspace_bytes(B, tq, mq, Hq)
    assert n == 4 * (2 * Hq * tq + B * Hq * (mq // 64))
    assert binding.attn_sink_bwd_varlen_workspace_bytes(0, tq, mq, Hq) == 0


def test_select_and_gather_reject(lib):
    r = lib.attn_sink_decode_select_slots(P, P, 1, 4, 3, -1, -1, P, P, 8, None)
    assert r == binding.ERR_UNSUPPORTED and "power of two" in binding.last_error()
    r = lib.attn_sink_decode_select_slots(None, P, 1, 4, 4, -1, -1, P, P, 8, None)
    assert r == binding.ERR_INVALID_ARG
    r = lib.attn_sink_gather_kv(P, P, P, P, 1, 2, 64, 16, 4, 5, 0, P, P, 8, binding.BF16, None)
    assert r == binding.ERR_INVALID_ARG and "window" in binding.last_error()


def test_binding_refuses_cpu_tensors(lib):
    import torch
    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        binding.attn_sink_fwd_prefill(q, q, q)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()


def test_launch_size_limits(lib):
    """Problems whose grid would exceed 32-bit work-item counts (or 65535 in y/z) are
    rejected on the host with ERR_UNSUPPORTED before any HIP call."""
    big = "too large for one launch"
    # prefill: 25165824 one-head groups -> as many 256-thread workgroups
    h = 25165824
    assert _prefill(lib, Sq=1, Sk=1, Hq=h, Hkv=h) == binding.ERR_UNSUPPORTED
    assert big in binding.last_error()
    # fp32 prefill: the head count is a grid's y extent
    assert _prefill(lib, Hq=70000, Hkv=70000, Sq=1, Sk=1, dtype=binding.F32) == \
        binding.ERR_UNSUPPORTED
    assert big in binding.last_error()
    # paged decode: 60000 sequences x ~60000 explicit splits
    assert _decode(lib, B=60000, maxp=(1 << 26), ns=60000, wsb=1 << 62) == binding.ERR_UNSUPPORTED
    assert big in binding.last_error()
    assert _decode_noalloc(lib, B=60000, maxp=(1 << 26), ns=60000) == binding.ERR_UNSUPPORTED
    assert big in binding.last_error()
    # backward: the head count is the preprocess grid's y extent
    assert _bwd(lib, Hq=70000, Hkv=70000, Sq=1, Sk=1) == binding.ERR_UNSUPPORTED
    assert big in binding.last_error()
    assert _bwd_varlen(lib, Hq=70000, Hkv=70000) == binding.ERR_UNSUPPORTED
    assert big in binding.last_error()
    # test exports: 2^24 selected rows x 256 threads, 2^24 sequences x 256 threads
    r = lib.attn_sink_gather_kv(P, P, P, P, 1, 2, 64, 16, 4, -1, -1, P, P, 1 << 24, binding.BF16,
                                None)
    assert r == binding.ERR_UNSUPPORTED and big in binding.last_error()
    r = lib.attn_sink_decode_select_slots(P, P, 1 << 24, 4, 16, -1, -1, P, P, 8, None)
    assert r == binding.ERR_UNSUPPORTED and big in binding.last_error()
    # extend: 16 sequences x 64 one-head groups x 2^24 / 256 row tiles = 2^26 workgroups
    assert _extend(lib, B=16, tq=1 << 24, mq=1 << 24, Hq=64, Hkv=64) == binding.ERR_UNSUPPORTED
    assert big in binding.last_error()
