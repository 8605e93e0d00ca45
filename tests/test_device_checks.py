"""Device-side preconditions (seqlens_k, block-table entries, cumulative offsets).

CPU: the release library reports that it has no device checks; the debug
library (libattn_sink_debug.so) carries the check kernels; and the checks'
predicates -- the same host/device functions the check kernels run -- are
exercised with invalid inputs through the host-side checker.  Invalid inputs
never go to a GPU: the GPU test of the debug library (tests/test_gpu_debug_checks.py)
uses valid inputs only.
"""

import ctypes
import subprocess

import numpy as np
import pytest

from softmax_learnable_sink_amd import binding

SEQ, PAGE, CU = binding.CHECK_SEQLEN, binding.CHECK_PAGE, binding.CHECK_CU_SEQLENS


@pytest.fixture(scope="module")
def libs():
    if not __import__("os").path.exists(binding.DEBUG_LIB_PATH):
        from softmax_learnable_sink_amd import build
        build.build()
    return binding.lib(), binding.debug_lib()


def test_release_library_has_no_device_checks(libs):
    rel, _ = libs
    flags = ctypes.c_uint(7)
    assert rel.attn_sink_device_check_flags(ctypes.byref(flags), 0, None) == \
        binding.ERR_UNSUPPORTED
    assert flags.value == 0 and "without device checks" in binding.last_error()


def test_debug_library_carries_the_check_kernels(libs):
    def syms(path):
        return subprocess.run(["nm", "-C", path], capture_output=True, text=True).stdout
    assert "check_paged_kernel" in syms(binding.DEBUG_LIB_PATH)
    assert "check_cu_kernel" in syms(binding.DEBUG_LIB_PATH)
    assert "check_paged_kernel" not in syms(binding.LIB_PATH)


def _table(B=3, max_pages=8, num_pages=32, seed=0):
    rng = np.random.default_rng(seed)
    return rng.permutation(num_pages)[:B * max_pages].reshape(B, max_pages).astype(np.int32)


def chk(bt, sl, **kw):
    kw.setdefault("page_size", 16)
    kw.setdefault("num_pages", 32)
    return binding.attn_sink_check_paged_inputs(bt, sl, **kw)


def test_valid_inputs_pass(libs):
    bt = _table()
    sl = np.array([5, 128, 40])
    assert chk(bt, sl) == 0
    assert chk(bt, sl, decode=False) == 0
    assert chk(bt, sl, window=(16, 32)) == 0
    cu = np.array([0, 3, 3, 10])
    assert chk(bt, sl, decode=False, cu_seqlens_q=cu, total_q=10, max_seqlen_q=7) == 0


def test_sequence_lengths(libs):
    bt = _table()
    # decode needs L >= 1 (the current token); extend allows an empty context
    assert chk(bt, np.array([0, 128, 40])) == SEQ
    assert chk(bt, np.array([0, 128, 40]), decode=False) == 0
    # longer than max_pages * page_size = 128
    assert chk(bt, np.array([5, 129, 40])) == SEQ
    assert chk(bt, np.array([5, 129, 40]), decode=False) == SEQ
    assert chk(bt, np.array([-3, 5, 5]), decode=False) == SEQ


def test_block_table_entries(libs):
    sl = np.array([5, 128, 40])
    for bad in (-1, 32, 1 << 30):
        bt = _table()
        bt[2, 1] = bad  # page 1 holds tokens 16..31 of the 40-token sequence
        assert chk(bt, sl) == PAGE
        assert chk(bt, sl, decode=False) == PAGE
    # entries past a sequence's last page are never read
    bt = _table()
    bt[0, 5] = -1
    assert chk(bt, sl) == 0 and chk(bt, sl, decode=False) == 0
    # window (16, 32) on L = 128: the decode reads pages 0, 6 and 7 only; the
    # extend and index-list paths read every page of [0, L)
    bt = _table()
    bt[1, 3] = -5
    assert chk(bt, sl, window=(16, 32)) == 0
    assert chk(bt, sl, window=(16, 32), decode=False) == PAGE
    bt[1, 6] = 99
    assert chk(bt, sl, window=(16, 32)) == PAGE


def test_cumulative_offsets(libs):
    bt = _table()
    sl = np.array([5, 128, 40])
    kw = dict(decode=False, total_q=10, max_seqlen_q=7)
    assert chk(bt, sl, cu_seqlens_q=np.array([1, 3, 3, 10]), **kw) == CU   # cu[0] != 0
    assert chk(bt, sl, cu_seqlens_q=np.array([0, 5, 3, 10]), **kw) == CU   # decreasing
    assert chk(bt, sl, cu_seqlens_q=np.array([0, 3, 3, 9]), **kw) == CU    # cu[B] != total
    assert chk(bt, sl, cu_seqlens_q=np.array([0, 1, 1, 10]), **kw) == CU   # 9 > max 7
    # several violations at once
    bt[0, 0] = -1
    assert chk(bt, np.array([5, 200, 40]), cu_seqlens_q=np.array([0, 5, 3, 10]), **kw) == \
        SEQ | PAGE | CU
