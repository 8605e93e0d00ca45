"""CPU check of the generated code of the kernels that load their K/V (or
Q/dO) tiles straight into LDS: every load is requested tiles ahead, and the
kernel waits for a tile only before the barrier that starts its step.  The
compiler adds a wait of its own for any load still in flight before an LDS
read it cannot tell apart from that load's destination (one LDS variable per
buffer, read addresses a few steps from it); such a wait would hold every
step on the next tile's loads.  The test compiles the sources to gfx950
assembly and checks that no LDS read in these kernels directly follows a
wait on the vector-memory counter."""

import re

import pytest

from softmax_learnable_sink_amd import build

KERNELS = {
    "prefill.hip": ["prefill_bf16_kernel", "extend_kernel", "index_kernel"],
    "backward.hip": ["bwd_main_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"],
}


def _functions(asm):
    """kernel symbol -> list of instruction lines (mnemonic first)."""
    out, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur = m.group(1)
            out[cur] = []
            continue
        t = line.strip()
        if cur is None or not t or t.startswith((".", ";")) or t.endswith(":"):
            continue
        out[cur].append(t)
        if t == "s_endpgm":
            cur = None
    return out


@pytest.fixture(scope="module", params=sorted(KERNELS))
def asm(request, tmp_path_factory):
    try:
        build.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    out = tmp_path_factory.mktemp("asm") / (request.param + ".s")
    build.device_asm(request.param, str(out))
    return request.param, out.read_text()


def test_no_compiler_wait_on_tiles_in_flight(asm):
    source, text = asm
    funcs = _functions(text)
    checked = 0
    for name in KERNELS[source]:
        syms = [s for s in funcs if name in s]
        assert syms, f"{name} not found in {source}"
        for sym in syms:
            insts = funcs[sym]
            assert any(re.match(r"buffer_load_dword\S* .* lds", i) or
                       i.startswith("global_load_lds") for i in insts), \
                f"{sym}: no tile loads into LDS"
            # (a wait on every counter is the kernels' own, before the first
            # tile's request)
            bad = [(a, b) for a, b in zip(insts, insts[1:])
                   if a.startswith("s_waitcnt") and "vmcnt" in a and b.startswith("ds_read")
                   and a != "s_waitcnt vmcnt(0) expcnt(0) lgkmcnt(0)"]
            assert not bad, f"{sym}: LDS reads held on loads in flight: {bad[:3]}"
            # the steps' own waits sit right before their barriers
            step_waits = [a for a, b in zip(insts, insts[1:])
                          if a.startswith("s_waitcnt") and "vmcnt" in a and b == "s_barrier"]
            assert step_waits, f"{sym}: no wait before a step barrier"
            checked += 1
    assert checked >= len(KERNELS[source])
