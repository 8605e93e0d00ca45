"""fp64 CPU oracle for sink attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, headers, helpers or constants) and imports
nothing from it; inputs come from the caller as NumPy arrays.
"""

from .sink_attention import (  # noqa: F401
    NEG_INF,
    visible,
    prefill,
    prefill_bruteforce,
    select_tokens,
    select_slots,
    gather_kv,
    decode_paged,
    extend_paged,
    backward,
    prefill_varlen,
    backward_varlen,
    index_paged,
)
