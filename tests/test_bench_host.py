"""Host logic of bench.py (no GPU): kernel-name shortening, labelling each dispatch of
a profiled run with the bench part that launched it, the counter summaries, the
work counts, and the --gpus contract."""

import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("raw,short", [
    ("_ZN9attn_sink12_GLOBAL__N_119prefill_bf16_kernelILi64ELi2EEEvPKDF16bS3_S3_PKfPDF16bPfiiii",
     "prefill_bf16_kernel<64,2>"),
    ("_ZN9attn_sink12_GLOBAL__N_121decode_partial_kernelILi128ELi4ELi2EEEvPKDF16bS3_S3_PKiS5_",
     "decode_partial_kernel<128,4,2>"),
    ("_ZN9attn_sink12_GLOBAL__N_115bwd_main_kernelILi64EEEvPKDF16bS3_S3_S3_PKfS5_PDF16bS6_",
     "bwd_main_kernel<64>"),
    ("void attn_sink::(anonymous namespace)::decode_combine_kernel<64, 2>(float const*, int)",
     "decode_combine_kernel<64,2>"),
    ("bwd_dsink_reduce_kernel(float const*, float*, int, int, int)", "bwd_dsink_reduce_kernel"),
    ("__amd_rocclr_copyBuffer", "__amd_rocclr_copyBuffer"),
])
def test_kernel_name_shortening(raw, short):
    assert bench._short(raw) == short


def test_dispatches_are_labelled_by_part_in_step_order():
    parts = ["prefill", "decode", "train"]
    one_step = (["prefill_bf16_kernel<64,2>", "reduce_kernel",
                 "decode_partial_kernel<64,4,2>", "decode_combine_kernel<64,2>"]
                + ["prefill_bf16_kernel<64,2>", "bwd_preprocess_kernel<64>", "bwd_main_kernel<64>",
                   "bwd_dsink_reduce_kernel"])
    names = ["__amd_rocclr_copyBuffer"] + one_step * 2
    labels = bench._label(names, parts)
    want_step = ["prefill", None, "decode", "decode"] + ["train"] * 4
    assert labels == [None] + want_step * 2


def test_a_dispatch_out_of_order_is_an_error():
    with pytest.raises(SystemExit):
        bench._label(["decode_partial_kernel<64,4,2>"], ["prefill", "decode"])


def _write_trace(path, rows):
    """rows in submission order; written shuffled by start time like a trace
    whose kernels overlap at their ends."""
    cols = ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X",
            "Grid_Size_Y", "Grid_Size_Z"]
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        for i, (name, t0, t1, g) in enumerate(rows):
            w.writerow([i + 1, name, t0, t1, g, 1, 1])


def test_kernel_stats_per_part(tmp_path, capsys):
    p = tmp_path / "trace.csv"
    # two steps of prefill (same kernel, same grid as the training forward) + train
    step = [("prefill_bf16_kernel<64,2>", 1000), ("prefill_bf16_kernel<64,2>", 3000),
            ("bwd_preprocess_kernel<64>", 10), ("bwd_main_kernel<64>", 9000),
            ("bwd_dsink_reduce_kernel", 5)]
    rows, t = [], 0
    for _ in range(2):
        for name, dur in step:
            rows.append((name, t, t + dur, 4096))
            t += dur + 1
    # the dSink reduction's start stamped before the start of the main kernel
    # submitted ahead of it: labels follow the submission order
    name, t0, t1, g = rows[4]
    rows[4] = (name, rows[3][1] - 5, rows[3][1], g)
    _write_trace(p, rows)
    bench.kernel_stats(str(p), ["prefill", "train"])
    out = capsys.readouterr().out.splitlines()
    pre = [ln for ln in out if ln.startswith("prefill ")]
    trn = [ln for ln in out if ln.startswith("train ") and "prefill_bf16" in ln]
    assert len(pre) == 1 and len(trn) == 1
    assert pre[0].split()[3] == "2" and float(pre[0].split()[4]) == pytest.approx(1.0)
    assert float(trn[0].split()[4]) == pytest.approx(3.0)


def test_sq_summary_formula(tmp_path, capsys):
    p = tmp_path / "counters.csv"
    vals = {"SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 500.0, "GRBM_GUI_ACTIVE": 8 * 1000.0,
            "SQ_INSTS_MFMA": 10.0, "SQ_INSTS_VALU": 120.0, "SQ_WAIT_INST_ANY": 30.0,
            "SQ_WAVE_CYCLES": 100.0}
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        for c, v in vals.items():
            w.writerow([1, "prefill_bf16_kernel<64,2>", 4096, c, v])
    vals.update({"SQ_ACTIVE_INST_VALU": 1024 * 100.0, "SQ_ACTIVE_INST_LDS": 1024 * 50.0,
                 "SQ_WAIT_INST_LDS": 10.0, "SQ_LDS_BANK_CONFLICT": 256 * 20.0})
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        for c, v in vals.items():
            w.writerow([1, "prefill_bf16_kernel<64,2>", 4096, c, v])
    bench.sq_stats(str(p), ["prefill"])
    lines = capsys.readouterr().out.splitlines()
    head = lines[0].split()
    row = dict(zip(head[3:], [ln for ln in lines if ln.startswith("prefill ")][0].split()[3:]))
    assert float(row["mfma_busy"]) == pytest.approx(0.5)   # 500 of 1000 cycles per SIMD
    assert float(row["valu_act"]) == pytest.approx(0.4)    # 4 * 100 of 1000 (4-cycle ticks)
    assert float(row["valu/mfma"]) == pytest.approx(12.0)  # VALU instructions per MFMA
    assert float(row["wait"]) == pytest.approx(0.3)        # wait fraction
    assert float(row["lds_act"]) == pytest.approx(0.2)
    assert float(row["lds_wait"]) == pytest.approx(0.1)
    assert float(row["bank_conf"]) == pytest.approx(0.02)  # 20 of 1000 cycles per CU


def test_causal_pair_count():
    # bottom-right causal: Sq = Sk = S gives S(S+1)/2 pairs per head
    assert bench.causal_pairs(4, 64, 4096, 4096) == 4 * 64 * 4096 * 4097 // 2
    # Sq < Sk: row i sees Sk - Sq + i + 1 keys
    assert bench.causal_pairs(1, 1, 2, 5) == 4 + 5


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
