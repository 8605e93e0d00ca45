"""Benchmark of the sink-attention hot path on one MI355X.

One step runs every entry point once over its synthetic workload:
  prefill   B4, S4096, 64 query / 8 KV heads, D64, causal, bf16, sink      (value)
  decode    B64, 64/8 heads, D64, page 16, L ~ U[1024, 32768], sink
  window32  B32, 32/8 heads, D128, page 16, L ~ U[16384, 65536], window 1024+7168, sink
  window1   the same with B1 (latency bound, reported only)
  extend    chunked prefill: B2 x 4096 new tokens on 4096..12288 cached ones, 64/8 heads,
            D64, page 16, sink (packed queries against the paged cache)
  train     B2, S8192, 64/8 heads, D64, causal: forward + backward with dSink
  varlen    packed training: 16384 tokens in sequences of U[512, 4096] tokens (the last
            one cut to fit), 64/8 heads, D64, causal: forward + backward with dSink
  index     index-list selection: B2 x 4096 new tokens on 4096 cached ones, 64/8 heads, D64,
            page 16, one list of 2048 positions per 128 queries (first 64, last 512, uniform
            middle), sink
Each entry point is bracketed by HIP events on the stream it is launched on
(the HBM-bound decode parts are preceded, outside their events, by a 512 MiB
read that leaves the caches holding clean lines); every rate is taken from the
median step of its part, with the minimum and the mean reported beside it;
`value` is the prefill throughput in TFLOP/s of algorithmic work (4*D flops per
visible (query, key) pair), `decode_gbps` the paged decode's algorithmic HBM
bytes (K and V rows of the attended tokens + Q + O + block table) per second.
A bounded sample of the fp64 CPU oracle is timed on the host for comparison.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--parts a,b] [--no-cpu-baseline]
Profile summaries (after rocprofv3 runs of this script):
       python bench.py --kernel-stats-from run_kernel_trace.csv [--parts ...]
       python bench.py --sq-from run_counter_collection.csv --parts ...
       python bench.py --traffic-from FETCH.csv WRITE.csv --copy-probe-mib 1024
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill attention TFLOP/s + paged-decode HBM GB/s (% of MI355X roofline)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PARTS = ("prefill", "decode", "window32", "window1", "extend", "train", "varlen", "index")
HBM_PARTS = ("decode", "window32", "window1")


def causal_pairs(B, Hq, Sq, Sk):
    """Visible (query, key) pairs of a bottom-right causal attention."""
    off = Sk - Sq
    per_head = sum(max(0, min(Sk, off + i + 1)) for i in range(Sq))
    return B * Hq * per_head


KERNEL_SOURCES = {  # sources each measured kernel is compiled from
    "prefill": ("prefill.hip", "common.h", "launch.h"),
    "decode": ("decode.hip", "common.h", "launch.h"),
}


def kernel_source_hash(which):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "softmax_learnable_sink_amd", "csrc")
    for name in KERNEL_SOURCES[which]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


TRAFFIC_KERNELS = {  # key in hbm_traffic.json -> (kernel-name substring, source set)
    "prefill_bf16_kernel": ("prefill_bf16_kernelILi64ELi2", "prefill"),
    "decode_partial_kernel": ("decode_partial_kernelILi64", "decode"),
    "decode_combine_kernel": ("decode_combine_kernelILi64", "decode"),
    "decode_partial_kernel_d128": ("decode_partial_kernelILi128", "decode"),
    "extend_kernel": ("extend_kernelILi64ELi2", "prefill"),
    "index_kernel": ("index_kernelILi64ELi2", "prefill"),
}


def write_traffic(fetch_csv, write_csv, probe_mib):
    """profiles/hbm_traffic.json from two rocprofv3 counter runs (FETCH_SIZE,
    then WRITE_SIZE, both in KiB per dispatch) of `bench.py --copy-probe-mib N`.
    Each counter is scaled by bytes / counter of the plain N MiB device copy in
    the same run, so the figures are HBM bytes per launch."""
    import csv
    probe = probe_mib << 20

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    out = {"source_hash": {k: kernel_source_hash(k) for k in KERNEL_SOURCES},
           "probe_bytes": probe, "bytes_per_launch": {}, "raw_kib_per_launch": {}}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = per_kernel(path, counter)
        copies = [v for k, vs in vals.items() if "copyBuffer" in k for v in vs]
        ref = max(copies)  # the probe copy is the largest copy of the run
        out[counter.lower() + "_scale"] = probe / (ref * 1024.0)
        for key, (sub, _) in TRAFFIC_KERNELS.items():
            vs = [v for k, v_ in vals.items() if sub in k for v in v_]
            if vs:
                kib = sum(vs) / len(vs)
                out["raw_kib_per_launch"].setdefault(key, {})[counter] = kib
                b = kib * 1024.0 * out[counter.lower() + "_scale"]
                out["bytes_per_launch"][key] = out["bytes_per_launch"].get(key, 0) + b
    for key in out["bytes_per_launch"]:
        out["bytes_per_launch"][key] = int(out["bytes_per_launch"][key])
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def _grid(row):
    if "Grid_Size" in row and row["Grid_Size"]:
        return int(row["Grid_Size"])
    g = 1
    for ax in ("X", "Y", "Z"):
        g *= int(row.get("Grid_Size_" + ax) or 1)
    return g


def _short(name):
    """kernel<template args> from a profiler's kernel name (mangled or not)."""
    import re
    m = re.search(r"GLOBAL__N_1(\d+)", name) or re.search(r"attn_sink(\d+)", name)
    if m:
        n = int(m.group(1))
        rest = name[m.end():]
        base, rest = rest[:n], rest[n:]
        args = re.match(r"I((?:L[a-z]+\d+E)+)E", rest)
        if args:
            base += "<" + ",".join(re.findall(r"L[a-z]+(\d+)E", args.group(1))) + ">"
        return base
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    return name.replace("attn_sink::", "").split("(")[0].replace(" ", "")


# Library kernels each bench part launches, in launch order (one stream).
PART_KERNELS = {
    "prefill": ("prefill_bf16_kernel",),
    "decode": ("decode_partial_kernel", "decode_combine_kernel"),
    "window32": ("decode_partial_kernel", "decode_combine_kernel"),
    "window1": ("decode_partial_kernel", "decode_combine_kernel"),
    "extend": ("extend_kernel",),
    "train": ("prefill_bf16_kernel", "bwd_preprocess_kernel", "bwd_main_kernel",
              "bwd_dsink_reduce_kernel"),
    "varlen": ("extend_kernel", "bwd_preprocess_kernel", "bwd_main_kernel",
               "bwd_dsink_reduce_kernel"),
    "index": ("index_kernel",),
}


def _label(names, parts):
    """The bench part of each dispatch (None for kernels not of this library):
    the parts run in order every step, each launching PART_KERNELS[part]."""
    ours = {k for p in parts for k in PART_KERNELS[p]}
    seq = [k for p in parts for k in PART_KERNELS[p]]
    owner = [p for p in parts for _ in PART_KERNELS[p]]
    out, i = [], 0
    for n in names:
        base = n.split("<")[0]
        if base not in ours:
            out.append(None)
            continue
        if base != seq[i % len(seq)]:
            raise SystemExit(f"dispatch {n} does not follow the part order {parts}")
        out.append(owner[i % len(seq)])
        i += 1
    return out


def kernel_stats(trace_csv, parts):
    """Per (bench part, kernel) launch count and duration from the
    kernel_trace.csv of a `rocprofv3 --kernel-trace` run of this script with
    these parts."""
    import csv
    # submission order (a kernel's start timestamp can precede the end of the
    # one submitted before it)
    with open(trace_csv) as f:
        recs = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
    names = [_short(r["Kernel_Name"]) for r in recs]
    rows = {}
    for r, n, p in zip(recs, names, _label(names, parts)):
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        rows.setdefault((p or "-", n, _grid(r)), []).append(us)
    total = sum(sum(v) for v in rows.values())
    print(f"{'part':9s} {'kernel':34s} {'grid':>9s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} "
          f"{'max_us':>9s} {'share%':>7s}")
    order = {p: i for i, p in enumerate(parts)}
    for (p, k, g), v in sorted(rows.items(), key=lambda kv: (order.get(kv[0][0], 99), kv[0][1])):
        print(f"{p:9s} {k:34s} {g:9d} {len(v):6d} {sum(v) / len(v):9.1f} {min(v):9.1f} "
              f"{max(v):9.1f} {100 * sum(v) / total:7.2f}")


def sq_stats(counter_csv, parts, xcds=8, simds=1024, cus=256):
    """Per (bench part, kernel), from the counter_collection.csv of a rocprofv3 SQ
    counter run (the last launch of each is reported; a metric is shown when its
    counters were collected):
      mfma_busy   SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs * SIMDs)
      valu_act    4 * SQ_ACTIVE_INST_VALU / (same): the SQ's cycle counters tick
                  once per 4 cycles
      valu/mfma   SQ_INSTS_VALU / SQ_INSTS_MFMA (SQ_INSTS_VALU counts the MFMA issues)
      wait        SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES
      lds_act     4 * SQ_ACTIVE_INST_LDS / (GRBM_GUI_ACTIVE / XCDs * SIMDs)
      lds_wait    SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES
      bank_conf   SQ_LDS_BANK_CONFLICT / (GRBM_GUI_ACTIVE / XCDs * CUs)"""
    import csv
    disp = {}
    with open(counter_csv) as f:
        for r in csv.DictReader(f):
            d = disp.setdefault(int(r["Dispatch_Id"]),
                                {"name": _short(r["Kernel_Name"]), "grid": _grid(r)})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ids = sorted(disp)
    labels = _label([disp[i]["name"] for i in ids], parts)
    last = {}
    for i, p in zip(ids, labels):
        if p:
            last[(p, disp[i]["name"])] = disp[i]

    def metrics(d):
        gui = d.get("GRBM_GUI_ACTIVE", 0.0)
        simd_cyc = gui / xcds * simds
        out = {}
        if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in d:
            out["mfma_busy"] = d["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cyc
        if gui and "SQ_ACTIVE_INST_VALU" in d:
            out["valu_act"] = 4 * d["SQ_ACTIVE_INST_VALU"] / simd_cyc
        if d.get("SQ_INSTS_MFMA") and "SQ_INSTS_VALU" in d:
            out["valu/mfma"] = d["SQ_INSTS_VALU"] / d["SQ_INSTS_MFMA"]
        wave = max(1.0, d.get("SQ_WAVE_CYCLES", 0.0))
        if "SQ_WAIT_INST_ANY" in d:
            out["wait"] = d["SQ_WAIT_INST_ANY"] / wave
        if gui and "SQ_ACTIVE_INST_LDS" in d:
            out["lds_act"] = 4 * d["SQ_ACTIVE_INST_LDS"] / simd_cyc
        if "SQ_WAIT_INST_LDS" in d:
            out["lds_wait"] = d["SQ_WAIT_INST_LDS"] / wave
        if gui and "SQ_LDS_BANK_CONFLICT" in d:
            out["bank_conf"] = d["SQ_LDS_BANK_CONFLICT"] / (gui / xcds * cus)
        return out
    cols = []
    for d in last.values():
        for k in metrics(d):
            if k not in cols:
                cols.append(k)
    print(f"{'part':9s} {'kernel':34s} {'grid':>9s} " + " ".join(f"{c:>9s}" for c in cols))
    for (p, k), d in last.items():
        m = metrics(d)
        print(f"{p:9s} {k:34s} {d['grid']:9d} " +
              " ".join(f"{m[c]:9.3f}" if c in m else f"{'-':>9s}" for c in cols))


def load_traffic():
    """HBM bytes per launch from the committed counter summary, for each kernel
    whose sources are unchanged since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return {}
    taken = data.get("source_hash", {})
    return {key: b for key, b in data.get("bytes_per_launch", {}).items()
            if key in TRAFFIC_KERNELS
            and taken.get(TRAFFIC_KERNELS[key][1]) == kernel_source_hash(TRAFFIC_KERNELS[key][1])}


class Workloads:
    def __init__(self, parts, dev):
        import numpy as np
        import torch
        from softmax_learnable_sink_amd import synth

        def dt(x):
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

        def i32(x):
            return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)

        self.parts = parts
        self.info = {}
        if "prefill" in parts:
            B, S, Hq, Hkv, D = 4, 4096, 64, 8, 64
            c = synth.prefill_case(B, S, S, Hq, Hkv, D, seed=0)
            self.pf = dict(q=dt(c["q"]), k=dt(c["k"]), v=dt(c["v"]),
                           sink=torch.from_numpy(c["sink"]).to(dev))
            self.pf["o"] = torch.empty_like(self.pf["q"])
            self.pf["lse"] = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
            pairs = causal_pairs(B, Hq, S, S)
            # Q, K, V in and O out (bf16), LSE out (fp32), sink in
            io = 2 * (2 * B * S * Hq * D + 2 * B * S * Hkv * D) + 4 * B * Hq * S + 4 * Hq
            self.info["prefill"] = dict(flops=4 * D * pairs, pairs=pairs, bytes=io,
                                        shape=f"B{B} S{S} H{Hq}/{Hkv} D{D} causal bf16")
            self.pf_case = c
        for name, spec in (("decode", (64, 64, 8, 64, 1024, 32768, None)),
                           ("window32", (32, 32, 8, 128, 16384, 65536, (1024, 7168))),
                           ("window1", (1, 32, 8, 128, 16384, 65536, (1024, 7168)))):
            if name not in parts:
                continue
            B, Hq, Hkv, D, lo, hi, w = spec
            c = synth.decode_case(B, Hq, Hkv, D, 16, lo, hi, seed=0)
            d = dict(q=dt(c["q"]), k=dt(c["k_cache"]), v=dt(c["v_cache"]), bt=i32(c["block_table"]),
                     sl=i32(c["seqlens"]), sink=torch.from_numpy(c["sink"]).to(dev), window=w)
            d["o"] = torch.empty_like(d["q"])
            d["lse"] = torch.empty((B, Hq), dtype=torch.float32, device=dev)
            from softmax_learnable_sink_amd import binding
            nbytes = binding.attn_sink_decode_workspace_bytes(B, Hq, Hkv, D, 16, c["block_table"].shape[1], w)
            d["ws"] = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            L = c["seqlens"].astype(np.int64)
            sel = np.minimum(L, sum(w)) if w else L
            kv_bytes = int(sel.sum()) * Hkv * D * 2 * 2
            # pages holding selected tokens: one int32 block-table entry each
            pages = 0
            for Lb in L.tolist():
                if w and Lb > sum(w):
                    toks = np.concatenate([np.arange(w[0]), np.arange(Lb - w[1], Lb)])
                    pages += len(np.unique(toks // 16))
                else:
                    pages += (Lb + 15) // 16
            # q in, o out (bf16), lse out (fp32), seqlens, sink, block-table entries
            io_bytes = 2 * B * Hq * D * 2 + 4 * B * Hq + 4 * B + 4 * Hq + 4 * pages
            self.info[name] = dict(bytes=kv_bytes + io_bytes, kv_bytes=kv_bytes,
                                   flops=4 * D * Hq * int(sel.sum()),
                                   shape=f"B{B} H{Hq}/{Hkv} D{D} P16 L~U[{lo},{hi}]"
                                         + (f" window {w[0]}+{w[1]}" if w else ""))
            setattr(self, name, d)
            if name == "decode":
                self.dec_case = c
        if "extend" in parts:
            B, Hq, Hkv, D = 2, 64, 8, 64
            c = synth.extend_case(B, Hq, Hkv, D, 16, 4096, 4096, 4096, 12288, seed=0)
            e = dict(q=dt(c["q"]), k=dt(c["k_cache"]), v=dt(c["v_cache"]),
                     bt=i32(c["block_table"]), cu=i32(c["cu_seqlens_q"]), sl=i32(c["seqlens"]),
                     sink=torch.from_numpy(c["sink"]).to(dev), max_sq=c["max_seqlen_q"])
            e["o"] = torch.empty_like(e["q"])
            e["lse"] = torch.empty((Hq, e["q"].shape[0]), dtype=torch.float32, device=dev)
            nq = np.diff(c["cu_seqlens_q"]).astype(np.int64)
            L = c["seqlens"].astype(np.int64)
            pairs = int(Hq * (nq * (L - nq) + nq * (nq + 1) // 2).sum())
            tq = int(nq.sum())
            # Q in, O out (bf16), LSE out, K and V of every context token, one
            # block-table entry per page, cu_seqlens, seqlens, sink
            io = (2 * 2 * tq * Hq * D + 4 * Hq * tq + int(L.sum()) * Hkv * D * 2 * 2
                  + 4 * int(((L + 15) // 16).sum()) + 4 * (2 * B + 1) + 4 * Hq)
            self.info["extend"] = dict(flops=4 * D * pairs, pairs=pairs, bytes=io,
                                       shape=f"B{B} nq{int(nq[0])} L~U[8192,16384] H{Hq}/{Hkv} "
                                             f"D{D} P16 causal bf16")
            self.ext = e
        if "train" in parts:
            B, S, Hq, Hkv, D = 2, 8192, 64, 8, 64
            c = synth.prefill_case(B, S, S, Hq, Hkv, D, seed=0, dout=True)
            t = dict(q=dt(c["q"]), k=dt(c["k"]), v=dt(c["v"]), do=dt(c["dout"]),
                     sink=torch.from_numpy(c["sink"]).to(dev))
            t["o"] = torch.empty_like(t["q"])
            t["lse"] = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
            t["dq"] = torch.empty_like(t["q"])
            t["dk"] = torch.empty_like(t["k"])
            t["dv"] = torch.empty_like(t["v"])
            t["dsink"] = torch.empty_like(t["sink"])
            from softmax_learnable_sink_amd import binding
            t["ws"] = torch.empty(binding.attn_sink_bwd_workspace_bytes(B, S, S, Hq, Hkv, D),
                                  dtype=torch.uint8, device=dev)
            pairs = causal_pairs(B, Hq, S, S)
            self.info["train"] = dict(flops=14 * D * pairs, fwd_flops=4 * D * pairs,
                                      bwd_flops=10 * D * pairs, pairs=pairs,
                                      shape=f"B{B} S{S} H{Hq}/{Hkv} D{D} causal bf16 fwd+bwd")
            self.tr = t
        if "varlen" in parts:
            Hq, Hkv, D = 64, 8, 64
            lens = synth.packed_lengths(16384, 512, 4096, seed=0)
            B = len(lens)
            c = synth.varlen_case(B, Hq, Hkv, D, seed=0, dout=True, q_lens=lens)
            t = dict(q=dt(c["q"]), k=dt(c["k"]), v=dt(c["v"]), do=dt(c["dout"]),
                     sink=torch.from_numpy(c["sink"]).to(dev), cq=i32(c["cu_seqlens_q"]),
                     ck=i32(c["cu_seqlens_k"]), mq=c["max_seqlen_q"], mk=c["max_seqlen_k"])
            tq = t["q"].shape[0]
            t["o"] = torch.empty_like(t["q"])
            t["lse"] = torch.empty((Hq, tq), dtype=torch.float32, device=dev)
            t["dq"] = torch.empty_like(t["q"])
            t["dk"] = torch.empty_like(t["k"])
            t["dv"] = torch.empty_like(t["v"])
            t["dsink"] = torch.empty_like(t["sink"])
            from softmax_learnable_sink_amd import binding
            t["ws"] = torch.empty(binding.attn_sink_bwd_varlen_workspace_bytes(B, tq, t["mq"], Hq),
                                  dtype=torch.uint8, device=dev)
            L = lens.astype(np.int64)
            pairs = int(Hq * (L * (L + 1) // 2).sum())
            self.info["varlen"] = dict(flops=14 * D * pairs, fwd_flops=4 * D * pairs,
                                       bwd_flops=10 * D * pairs, pairs=pairs,
                                       shape=f"packed {tq} tokens in {B} sequences "
                                             f"(U[512,4096]) H{Hq}/{Hkv} D{D} causal bf16 fwd+bwd")
            self.vl = t
        if "index" in parts:
            B, Hq, Hkv, D, bq, topk = 2, 64, 8, 64, 128, 2048
            c = synth.index_case(B, Hq, Hkv, D, 16, 4096, 4096, 4096, 4096, bq, topk, seed=0)
            e = dict(q=dt(c["q"]), k=dt(c["k_cache"]), v=dt(c["v_cache"]),
                     bt=i32(c["block_table"]), cu=i32(c["cu_seqlens_q"]), sl=i32(c["seqlens"]),
                     idx=i32(c["kv_index"]), cb=i32(c["cu_blocks"]),
                     sink=torch.from_numpy(c["sink"]).to(dev), max_sq=c["max_seqlen_q"], bq=bq)
            e["o"] = torch.empty_like(e["q"])
            e["lse"] = torch.empty((Hq, e["q"].shape[0]), dtype=torch.float32, device=dev)
            # visible (row, listed token) pairs: tokens of the row's list at or before it
            pairs = 0
            for b in range(B):
                nq, L = int(c["q_lens"][b]), int(c["seqlens"][b])
                for j in range(int(c["cu_blocks"][b + 1] - c["cu_blocks"][b])):
                    lst = c["kv_index"][c["cu_blocks"][b] + j]
                    lst = np.sort(lst[(lst >= 0) & (lst < L)])
                    pos = L - nq + np.arange(j * bq, min(nq, (j + 1) * bq))
                    pairs += int(np.searchsorted(lst, pos, side="right").sum())
            pairs *= Hq
            # Q in, O out (bf16), LSE out, K and V of every distinct listed token of a
            # sequence, the lists, one block-table entry per page touched, small arrays
            kv_rows, pages = 0, 0
            for b in range(B):
                lst = c["kv_index"][c["cu_blocks"][b]:c["cu_blocks"][b + 1]]
                toks = np.unique(lst[(lst >= 0) & (lst < int(c["seqlens"][b]))])
                kv_rows += len(toks)
                pages += len(np.unique(toks // 16))
            tq = int(c["q_lens"].sum())
            io = (2 * 2 * tq * Hq * D + 4 * Hq * tq + kv_rows * Hkv * D * 2 * 2
                  + c["kv_index"].size * 4 + 4 * pages + 4 * (3 * B + 2) + 4 * Hq)
            self.info["index"] = dict(flops=4 * D * pairs, pairs=pairs, bytes=io,
                                      shape=f"B{B} nq4096 L8192 H{Hq}/{Hkv} D{D} P16 "
                                            f"list {topk} per {bq} queries causal bf16")
            self.ix = e

    def run(self, name):
        from softmax_learnable_sink_amd import binding
        if name == "prefill":
            p = self.pf
            binding.attn_sink_fwd_prefill(p["q"], p["k"], p["v"], p["sink"], causal=True,
                                          softmax_scale=0.125, out=p["o"], lse=p["lse"])
        elif name in ("decode", "window32", "window1"):
            d = getattr(self, name)
            D = d["q"].shape[-1]
            binding.attn_sink_fwd_decode_paged(d["q"], d["k"], d["v"], d["bt"], d["sl"], d["sink"],
                                               softmax_scale=1 / math.sqrt(D), window=d["window"],
                                               out=d["o"], lse=d["lse"], workspace=d["ws"])
        elif name == "extend":
            e = self.ext
            binding.attn_sink_fwd_extend_paged(e["q"], e["k"], e["v"], e["bt"], e["cu"], e["sl"],
                                               e["max_sq"], e["sink"], softmax_scale=0.125,
                                               out=e["o"], lse=e["lse"])
        elif name == "index":
            e = self.ix
            binding.attn_sink_fwd_index_paged(e["q"], e["k"], e["v"], e["bt"], e["cu"], e["sl"],
                                              e["max_sq"], e["idx"], e["cb"], e["bq"], e["sink"],
                                              softmax_scale=0.125, out=e["o"], lse=e["lse"])
        elif name == "train":
            t = self.tr
            binding.attn_sink_fwd_prefill(t["q"], t["k"], t["v"], t["sink"], causal=True,
                                          softmax_scale=0.125, out=t["o"], lse=t["lse"])
            binding.attn_sink_bwd(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], t["sink"],
                                  causal=True, softmax_scale=0.125, dq=t["dq"], dk=t["dk"],
                                  dv=t["dv"], dsink=t["dsink"], workspace=t["ws"])
        elif name == "varlen":
            t = self.vl
            binding.attn_sink_fwd_varlen(t["q"], t["k"], t["v"], t["cq"], t["ck"], t["mq"], t["sink"],
                                         causal=True, softmax_scale=0.125, out=t["o"], lse=t["lse"])
            binding.attn_sink_bwd_varlen(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], t["cq"],
                                         t["ck"], t["mq"], t["mk"], t["sink"], causal=True,
                                         softmax_scale=0.125, dq=t["dq"], dk=t["dk"], dv=t["dv"],
                                         dsink=t["dsink"], workspace=t["ws"])


def host_info():
    """CPU model (/proc/cpuinfo), BLAS library and thread count NumPy runs with."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            i = libs[0]
            blas = f"{i.get('internal_api', '?')} {i.get('version', '?')}"
            threads = int(i.get("num_threads", threads))
    except Exception:  # noqa: BLE001
        pass
    return model, blas, threads


def cpu_baseline(wl, budget_s=10.0, train_budget_s=10.0):
    """The fp64 oracle (as it stands) on bounded samples: the prefill workload's
    first (batch, head) pairs, in order, that fit the time budget, all 4096 query
    rows each; and, for the training workload (B2 S8192 64/8 heads D64 causal),
    the forward + backward of its first (batch, head) pairs in order, all 8192
    rows each, within its own budget."""
    import numpy as np
    import oracle
    from softmax_learnable_sink_amd import synth
    model, blas, cores = host_info()
    c = wl.pf_case
    B, S, Hq, Hkv, D = 4, 4096, 64, 8, 64
    g = Hq // Hkv
    t_total, n = 0.0, 0
    while t_total < budget_s and n < B * Hq:
        b, h = divmod(n, Hq)
        q = synth.bf16_to_f32(c["q"][b:b + 1, :, h:h + 1]).astype(np.float64)
        k = synth.bf16_to_f32(c["k"][b:b + 1, :, h // g:h // g + 1]).astype(np.float64)
        v = synth.bf16_to_f32(c["v"][b:b + 1, :, h // g:h // g + 1]).astype(np.float64)
        t0 = time.perf_counter()
        oracle.prefill(q, k, v, c["sink"][h:h + 1], 0.125, causal=True)
        t_total += time.perf_counter() - t0
        n += 1
    flops = 4 * D * causal_pairs(1, n, S, S)
    out = {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
           "kind": "oracle",
           "sample": f"prefill S4096 D64 causal, the first {n} of 256 (batch, head) pairs "
                     f"in (batch, head) order, all rows; {t_total:.1f} s of oracle time",
           "cpu_model": model, "blas": blas}
    # training fwd + bwd (14 D flops per visible pair), the workload's own inputs
    S = 8192
    ct = synth.prefill_case(2, S, S, Hq, Hkv, D, seed=0, dout=True)
    t_total, n = 0.0, 0
    while t_total < train_budget_s and n < 2 * Hq:
        b, h = divmod(n, Hq)
        sl = (slice(b, b + 1), slice(None))
        q = synth.bf16_to_f32(ct["q"][sl + (slice(h, h + 1),)]).astype(np.float64)
        do = synth.bf16_to_f32(ct["dout"][sl + (slice(h, h + 1),)]).astype(np.float64)
        k = synth.bf16_to_f32(ct["k"][sl + (slice(h // g, h // g + 1),)]).astype(np.float64)
        v = synth.bf16_to_f32(ct["v"][sl + (slice(h // g, h // g + 1),)]).astype(np.float64)
        t0 = time.perf_counter()
        oracle.backward(q, k, v, ct["sink"][h:h + 1], do, 0.125, True)
        t_total += time.perf_counter() - t0
        n += 1
    flops = 14 * D * causal_pairs(1, n, S, S)
    out["train"] = {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s",
                    "sample": f"training fwd+bwd S8192 D64 causal (14 D flops per pair), the "
                              f"first {n} of 128 (batch, head) pairs in order, all rows; "
                              f"{t_total:.1f} s of oracle time"}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--parts", default=",".join(PARTS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/hbm_traffic.json from the counter_collection.csv of a "
                         "FETCH_SIZE and a WRITE_SIZE rocprofv3 run made with --copy-probe-mib, "
                         "then exit")
    ap.add_argument("--kernel-stats-from", metavar="TRACE_CSV",
                    help="print per-kernel launch times from the kernel_trace.csv of a "
                         "rocprofv3 --kernel-trace run, then exit")
    ap.add_argument("--sq-from", metavar="COUNTER_CSV",
                    help="print MFMA utilisation per kernel from the counter_collection.csv of "
                         "a rocprofv3 SQ counter run, then exit")
    args = ap.parse_args()
    if args.kernel_stats_from:
        kernel_stats(args.kernel_stats_from, [p for p in args.parts.split(",") if p])
        return
    if args.sq_from:
        sq_stats(args.sq_from, [p for p in args.parts.split(",") if p])
        return
    if args.traffic_from:
        write_traffic(args.traffic_from[0], args.traffic_from[1], args.copy_probe_mib or 1024)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the sink-attention path has no multi-GPU code)", file=sys.stderr)
        sys.exit(2)
    parts = [p for p in args.parts.split(",") if p]
    for p in parts:
        if p not in PARTS:
            sys.exit(f"unknown part {p}")

    import torch
    from softmax_learnable_sink_amd import binding
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    binding.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"# building workloads: {parts}", file=sys.stderr, flush=True)
    wl = Workloads(parts, dev)
    torch.cuda.synchronize()

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    events = {p: [] for p in parts}
    # Before each HBM-bound part, a 512 MiB read (outside the part's events) leaves
    # the L2 and the 256 MB Infinity Cache holding clean lines: otherwise the decode
    # pays for writing back the dirty output of the part before it (the prefill's
    # 128 MiB of O), which is that part's traffic, not its own.
    flush = (torch.zeros(128 << 20, dtype=torch.float32, device=dev)
             if any(p in HBM_PARTS for p in parts) else None)

    def step(record):
        for p in parts:
            if p in HBM_PARTS:
                flush.sum()
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            wl.run(p)
            if record:
                e1.record(stream)
                events[p].append((e0, e1))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    print(f"# warmup done, timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = {p: sorted(a.elapsed_time(b) for a, b in events[p]) for p in parts}
    # rates from the median step of each part; min and mean reported beside it
    ms = {p: (t[len(t) // 2] if len(t) % 2 else 0.5 * (t[len(t) // 2 - 1] + t[len(t) // 2]))
          for p, t in times.items()}

    traffic = load_traffic()
    out = {"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / max(1, args.steps), 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": "sink attention hot path: " + "; ".join(
               f"{p} {wl.info[p]['shape']}" for p in parts)}}
    parts_out = {}
    for p in parts:
        info = wl.info[p]
        rec = {"ms": round(ms[p], 5), "ms_min": round(times[p][0], 5),
               "ms_mean": round(sum(times[p]) / len(times[p]), 5), "shape": info["shape"]}
        if "bytes" in info:
            gbps = info["bytes"] / (ms[p] * 1e-3) / 1e9
            rec.update(gbps=round(gbps, 2), hbm_frac=round(gbps / PEAK_HBM_GBPS, 4),
                       algorithmic_bytes=info["bytes"])
        if p in ("prefill", "extend", "train", "varlen", "index"):
            tf = info["flops"] / (ms[p] * 1e-3) / 1e12
            rec.update(tflops=round(tf, 2), mfma_frac=round(tf / PEAK_BF16_TFLOPS, 4),
                       algorithmic_flops=info["flops"])
        parts_out[p] = rec
    out["parts"] = parts_out
    if "prefill" in parts:
        pf = parts_out["prefill"]
        out["value"] = pf["tflops"]
        tb = traffic.get("prefill_bf16_kernel")
        out["roofline"] = {"bound": "mfma", "achieved": pf["tflops"], "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": pf["mfma_frac"],
                           "traffic": tb, "kernel": "prefill_bf16_kernel<64,2>",
                           "algorithmic_bytes": wl.info["prefill"]["bytes"]}
    if "decode" in parts:
        dc = parts_out["decode"]
        out["decode_gbps"] = dc["gbps"]
        out["decode_roofline"] = {"bound": "hbm", "achieved": dc["gbps"], "peak": PEAK_HBM_GBPS,
                                  "unit": "GB/s", "frac": dc["hbm_frac"],
                                  "traffic": traffic.get("decode_partial_kernel"),
                                  "kernel": "decode_partial_kernel<64> + decode_combine_kernel<64>"}
    if out["value"] is None:
        first = parts_out[parts[0]]
        out["value"] = first.get("tflops", first.get("gbps"))
        out["unit"] = "TFLOP/s" if "tflops" in first else "GB/s"
    if not args.no_cpu_baseline and "prefill" in parts:
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
