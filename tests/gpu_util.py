"""Shared helpers of the GPU parity tests: synth arrays -> device tensors,
device tensors -> exact float64 NumPy values, and the tolerance checks."""

import os
import sys

import numpy as np
import pytest
import torch

from softmax_learnable_sink_amd import synth

# Tolerances (against the fp64 oracle): fp32 1e-5 max-abs; bf16 1e-2 max-abs
# on O, 1e-3 on LSE, 2e-2 relative (max-norm over heads) on dSink; dQ/dK/dV
# elementwise |gpu - ref| <= 3e-2 (1 + |ref|), the bound derived from the
# bf16 operand roundings in tests/test_tolerance_model.py.
TOL_F32 = 1e-5
TOL_O = 1e-2
TOL_LSE = 1e-3
TOL_DSINK_REL = 2e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from softmax_learnable_sink_amd import binding
    binding.lib()  # a missing library fails loudly


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tensor(x, dtype):
    """Synth array (uint16 bf16 bits or float32) -> contiguous CUDA tensor."""
    if dtype == synth.BF16:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to("cuda")


def host64(t):
    """Device tensor -> float64 NumPy array of its exact values."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def vals(x, dtype):
    return synth.values(x, dtype).astype(np.float64)


def max_abs(a, b):
    if a.size == 0:
        return 0.0
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.max(d))


def check_close(name, got, ref, tol):
    err = max_abs(got, ref)
    say(f"  {name}: max_abs_err={err:.3e} (tol {tol:.1e})")
    assert np.all(np.isfinite(got) | np.isinf(ref)), f"{name}: non-finite output"
    assert err <= tol, f"{name}: max abs error {err:.3e} > {tol:.1e}"


TOL_GRAD = 3e-2


def check_grad(name, got, ref):
    bound = TOL_GRAD * (1.0 + np.abs(ref))
    ratio = float(np.max(np.abs(got - ref) / bound)) if got.size else 0.0
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    say(f"  {name}: max_abs_err={err:.3e}, max err/(3e-2(1+|ref|)) = {ratio:.3f}")
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    assert ratio <= 1.0, f"{name}: error above 3e-2 (1 + |ref|)"


def poison_unselected(case, window):
    """Write NaN into every cached token that the window leaves out, so that a
    kernel reading outside the selection produces NaN."""
    import oracle
    P = case["page_size"]
    nan = synth.f32_to_bf16_bits(np.float32(np.nan)) if case["dtype"] == synth.BF16 else np.nan
    for b, L in enumerate(case["seqlens"].tolist()):
        keep = np.zeros(L, dtype=bool)
        keep[oracle.select_tokens(L, window)] = True
        t = np.nonzero(~keep)[0]
        pages = case["block_table"][b, t // P]
        case["k_cache"][pages, t % P] = nan
        case["v_cache"][pages, t % P] = nan
    return case


def env_flag(name):
    return os.environ.get(name, "") not in ("", "0")


def oracle_map(fn, items):
    """Run fn over items on a thread pool, one BLAS thread each: the oracle's
    elementwise NumPy work releases the GIL, so independent (sequence,
    KV-head group) sub-problems of a full-size workload run side by side.
    Results come back in the order of items."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    workers = max(1, min(16, len(os.sched_getaffinity(0)), len(items)))
    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(workers) as ex:
            return list(ex.map(fn, items))


def grad_ratio(got, ref):
    """max |got - ref| / (3e-2 (1 + |ref|)) -- at most 1 within the bound."""
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / (TOL_GRAD * (1.0 + np.abs(ref)))))
