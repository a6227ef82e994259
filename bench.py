"""Benchmark of the exact tiled attention hot path on one MI355X.

A step is one pass of the whole hot path over the long-sequence causal workload
(B=1, H=16, N=16384, bf16, causal, at d=64 and at d=128): for each head dimension
the forward (O, lse) and the backward (the dQ kernel, whose prologue is the D =
rowsum(dO o O) pre-pass, then the dK/dV kernel) through the C ABI, on inputs already
resident in device memory. The K timed steps run bare (the metric); K more steps with the
library's per-kernel events armed (fa_time_next_call) give each kernel's and each phase's
time, and their step time is reported as instrumented_ms_per_step.

FLOP convention: forward 4*B*H*N^2*d, halved for causal; backward 2.5x the forward
(five products per score tile instead of two). value = FLOP per step / time per step.
The backward's dK/dV kernel performs four of the five products (2.0x the forward); its
dQ kernel the fifth, plus a recomputation of two that the convention does not count.

Packed variable-length sequences and the sliding-window mask are timed outside the step
on their own workloads and reported under "varlen" (FLOP counted exactly over the allowed
query-key pairs: 4 d per pair forward, 2.5x that backward).

Dropout (p = 0.1) on the step's workloads is timed outside the step and reported under
"dropout", by the same FLOP convention (the generator's work is not counted).

The short-sequence workloads (BERT-shaped N=512 with key padding, GPT-2-shaped N=1024
causal) are timed outside the step as forward + backward pairs, eagerly and as a replayed
HIP graph, under "short_n".

The key/value-cache forward (a few queries against a long cache, HBM-bound) is timed
outside the step on its decode workloads and reported under "kvcache_decode": algorithmic
bytes = every valid cached key and value read once plus Q and O, divided by the time of the
whole call (key-split kernel and merge).

Every named workload (single-head fp32, BERT-shaped with key padding, GPT-2-shaped causal,
the long causal pair, block-sparse 64K) is also reported under "configs", forward and
backward separately: ms, TFLOP/s and fraction of peak by the headline convention (plus the
allowed-pair convention for key padding; kept blocks for the block mask) and HBM GB/s of
the compulsory bytes. "clock" samples the engine clock (rocm-smi) while the step runs.

Prints ONE JSON line (the metric line). `--report FILE` additionally times every
workload (forward and backward separately) and writes a per-workload JSON;
`--decode-only` times only the decode workloads (for profiling them).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3    # MI355X dense fp32 (the fp32 forward's MFMA rate)
PEAK_CLOCK_MHZ = 2400.0    # the engine clock that peak assumes
DROPOUT_P, DROPOUT_SEED = 0.1, 1234  # the dropout report's probability and seed
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd+bwd TFLOP/s (bf16, causal) and % of MI355X bf16 MFMA peak"
STEP_WORKLOADS = ("long_causal_d64", "long_causal_d128")
SHORT_WORKLOADS = ("bert_padded", "gpt2_causal")
# Algorithmic FLOP of each timed kernel, as a multiple of the forward FLOP: the forward's two
# products; four of the backward's five (dV, dP, dK and the recomputed S count as S, dP, dV,
# dK of the convention) in the dK/dV kernel; the fifth (dQ) in the dQ kernel, which also
# recomputes S and dP (executed: 1.5x) without the convention counting them.
KERNEL_FLOP_FACTOR = {"fwd": 1.0, "bwd_dkdv": 2.0, "bwd_dq": 0.5}
KERNEL_EXECUTED_FACTOR = {"fwd": 1.0, "bwd_dkdv": 2.0, "bwd_dq": 1.5}
CALIBRATION_BYTES = 256 << 20


# Minimum GPU time of every warm-up: the engine clock falls while the GPU idles (for instance
# while the next workload's inputs are generated on the host) and takes milliseconds to climb
# back, so a fixed few warm-up calls can leave the first timed calls at a low clock.
MIN_WARMUP_S = 0.2


def warm_up(fn, calls: int, min_s: float = MIN_WARMUP_S) -> None:
    """Runs `fn` at least `calls` times and until `min_s` seconds have passed, then syncs."""
    import torch
    t_end = time.perf_counter() + min_s
    n = 0
    while n < calls or time.perf_counter() < t_end:
        fn()
        n += 1
        if n >= calls:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def attn_flops(w, kept_fraction=None) -> float:
    """Forward FLOP of a workload under the convention above."""
    f = 4.0 * w.B * w.H * w.N * w.N * w.d
    if w.causal:
        f /= 2
    if kept_fraction is not None:
        f *= kept_fraction
    return f


class Runner:
    """Device-resident inputs, outputs and workspace for one workload."""

    def __init__(self, fa, w, dev):
        import torch
        from exact_tiled_attention_32_amd import workloads
        self.fa, self.w = fa, w
        x = workloads.generate(w)
        self.q, self.k, self.v = (x[n].to(dev) for n in ("q", "k", "v"))
        self.do = x["do"].to(dev) if x["do"] is not None else None
        self.kv = None if x["kv_len"] is None else x["kv_len"].to(dev)
        self.mask = None if x["block_mask"] is None else x["block_mask"].to(dev)
        self.scale = x["scale"]
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:3], dtype=torch.float32, device=dev)
        if w.backward:
            self.dq, self.dk, self.dv = (torch.empty_like(self.q) for _ in range(3))
            self.ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
        self.kept = None
        if self.mask is not None:
            self.kept = float(x["block_mask"].double().mean())

    @property
    def bwd_kernels(self):
        """The backward call's kernels in launch order (the timer's event order)."""
        return (["bwd_order"] if self.mask is not None else []) + ["bwd_dq", "bwd_dkdv"]

    def fwd(self):
        if self.mask is not None:
            self.fa.fa_fwd_blocksparse(self.q, self.k, self.v, self.scale, self.mask, self.w.mask_block,
                                       self.w.causal, self.kv, o=self.o, lse=self.lse)
        else:
            self.fa.fa_fwd(self.q, self.k, self.v, self.scale, self.w.causal, self.kv, o=self.o, lse=self.lse)

    def bwd(self):
        self.fa.fa_bwd(self.q, self.k, self.v, self.o, self.do, self.lse, self.scale, self.w.causal, self.kv,
                       self.mask, self.w.mask_block, dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.ws)


class KernelClock:
    """HIP events recorded by the library before a call's first kernel and after each of
    its kernels (fa_time_next_call), on the call's own stream."""

    def __init__(self):
        self.samples = {}

    @staticmethod
    def new_events(n):
        import torch
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        # torch creates the HIP event at its first record; the library then re-records it
        # around the kernel launches on the same stream
        for e in evs:
            e.record()
        return evs

    def arm(self, fa, name, events):
        """Has the library time the kernels of its next call with `events` (made beforehand
        by new_events, so that no event is created inside a timed region)."""
        self.samples.setdefault(name, []).append(events)
        fa.fa_time_next_call(events)

    def kernel_ms(self, name, i):
        """Mean duration of the i-th kernel of the calls armed under `name`."""
        ev = self.samples.get(name, [])
        return sum(e[i].elapsed_time(e[i + 1]) for e in ev) / len(ev) if ev else float("nan")

    def call_ms(self, name):
        """Mean time from before the first to after the last bracketed kernel."""
        ev = self.samples.get(name, [])
        return sum(e[0].elapsed_time(e[-1]) for e in ev) / len(ev) if ev else float("nan")

    def call_ms_median(self, name):
        """Median over the calls of the time from before the first to after the last
        bracketed kernel."""
        ev = self.samples.get(name, [])
        if not ev:
            return float("nan")
        t = sorted(e[0].elapsed_time(e[-1]) for e in ev)
        m = len(t) // 2
        return t[m] if len(t) % 2 else 0.5 * (t[m - 1] + t[m])


KERNEL_NAMES = {  # demangled kernel -> short name used by the bench and the traffic file
    # (template arguments: tile width, dropout flag, head dimension in memory; for the
    # forward also its K/V buffer count, two on these long workloads; for dK/dV the query
    # halves, 1 for the dense 4-wave layout, and the query-block override, 0 for none)
    "fwd_bf16_kernel<64, false, 64, 2>": "fwd_d64", "fwd_bf16_kernel<128, false, 128, 2>": "fwd_d128",
    "bwd_dkdv_kernel<64, false, 64, 1, 0>": "bwd_dkdv_d64", "bwd_dkdv_kernel<128, false, 128, 1, 0>": "bwd_dkdv_d128",
    "bwd_dq_kernel<64, false, 64>": "bwd_dq_d64", "bwd_dq_kernel<128, false, 128>": "bwd_dq_d128",
    "kvc_split_kernel<64>": "kvc_split_d64", "kvc_split_kernel<128>": "kvc_split_d128",
    "kvc_merge_kernel<64>": "kvc_merge_d64", "kvc_merge_kernel<128>": "kvc_merge_d128",
}


def summarize_pmc(fetch_csv: str, write_csv: str, out_path: str) -> dict:
    """HBM bytes per dispatch from two rocprofv3 --pmc runs of `bench.py --pmc-pass`
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by the factor that makes
    the 256 MiB calibration copy read and write exactly its size."""
    import csv

    def load(path, counter):
        per = {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            key = (int(row["Dispatch_Id"]), row["Kernel_Name"])
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"]) * 1024.0
        return per

    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")

    def calib(per):
        # the calibration copy is the last device copy before the first library kernel
        # (the uploads of the inputs come before it)
        items = sorted(per.items())
        first = next((i for i, ((d, n), v) in enumerate(items) if "fa::" in n), len(items))
        vals = [v for (d, n), v in items[:first] if "copyBuffer" in n]
        if not vals:
            raise RuntimeError("calibration copy not found in the counter file")
        return CALIBRATION_BYTES / vals[-1]

    ff, fw = calib(fetch), calib(write)

    def short(name):
        for k, v in KERNEL_NAMES.items():
            if k in name:
                return v
        return None

    def by_kernel(per, factor):
        out = {}
        for (d, n), v in sorted(per.items()):
            s = short(n)
            if s:
                out.setdefault(s, []).append(v * factor)
        return {k: sum(v) / len(v) for k, v in out.items()}

    fb, wb = by_kernel(fetch, ff), by_kernel(write, fw)
    digest = kernel_source_digest()
    res = {"calibration": {"copy_bytes": CALIBRATION_BYTES, "fetch_factor": ff, "write_factor": fw},
           "kernels": {k: {"fetch_bytes": fb[k], "write_bytes": wb.get(k, 0.0),
                           "bytes_per_launch": fb[k] + wb.get(k, 0.0), "source_digest": digest} for k in fb}}
    with open(out_path, "w") as f:
        json.dump(res, f, indent=1)
    return res


COUNTER_SETS = {  # one rocprofv3 --pmc pass each (at most 8 SQ, 4 TCC and 2 GRBM counters)
    "sq": "SQ_BUSY_CU_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT "
          "SQ_LDS_IDX_ACTIVE SQ_WAVE_CYCLES GRBM_GUI_ACTIVE",
    "valu": "SQ_BUSY_CU_CYCLES SQ_ACTIVE_INST_VALU SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_SALU SQ_ACTIVE_INST_LDS",
    "fetch": "FETCH_SIZE",
    "write": "WRITE_SIZE",
}


def counter_sequence(workloads):
    """(workload, kernel) of every library dispatch of `--counter-pass`, in launch order."""
    seq = []
    for _ in range(2):
        for name, w in workloads.WORKLOADS.items():
            seq.append((name, "fwd_f32_kernel<64>" if w.dtype == "f32" else f"fwd_bf16_kernel<{w.d}>"))
            if w.backward:
                if w.sparse:
                    seq.append((name, "bwd_order_kernel"))
                seq += [(name, f"bwd_dq_kernel<{w.d}>"), (name, f"bwd_dkdv_kernel<{w.d}>")]
        for name, w in workloads.VARLEN_WORKLOADS.items():
            seq += [(name, f"fwd_bf16_kernel<{w.d}>"), (name, f"bwd_dq_kernel<{w.d}>"),
                    (name, f"bwd_dkdv_kernel<{w.d}>")]
        for name in STEP_WORKLOADS:
            d = workloads.WORKLOADS[name].d
            seq += [(name + "_dropout", f"fwd_bf16_kernel<{d}>"), (name + "_dropout", f"bwd_dq_kernel<{d}>"),
                    (name + "_dropout", f"bwd_dkdv_kernel<{d}>")]
        for name, w in workloads.DECODE_WORKLOADS.items():
            seq += [(name, f"kvc_split_kernel<{w.d}>"), (name, f"kvc_merge_kernel<{w.d}>")]
    return seq


def counter_pass(fa, dev):
    """For rocprofv3: the calibration copy, then every workload's forward and backward and
    every decode call, twice (the second round is the one summarised)."""
    import torch
    from exact_tiled_attention_32_amd import workloads
    runners = [Runner(fa, w, dev) for w in workloads.WORKLOADS.values()]
    dec = []
    for w in workloads.DECODE_WORKLOADS.values():
        x = workloads.generate_decode(w)
        q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
        kv = None if x["kv_len"] is None else x["kv_len"].to(dev)
        ws = torch.empty(fa.fa_fwd_kvcache_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d), dtype=torch.uint8,
                         device=dev)
        dec.append((w, q, k, v, kv, x["scale"], ws))
    var = []
    for w in workloads.VARLEN_WORKLOADS.values():
        x = workloads.generate_varlen(w)
        t = {n: x[n].to(dev) for n in ("q", "k", "v", "do", "cu_seqlens")}
        var.append((w, x, t))
    src = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    for _ in range(2):
        for r in runners:
            r.fwd()
            if r.w.backward:
                r.bwd()
            torch.cuda.synchronize()
        for w, x, t in var:
            kw = dict(causal=w.causal, window_left=w.window_left, window_right=w.window_right)
            o, lse = fa.fa_fwd_varlen(t["q"], t["k"], t["v"], t["cu_seqlens"], x["max_seqlen"], x["scale"], **kw)
            fa.fa_bwd_varlen(t["q"], t["k"], t["v"], o, t["do"], lse, t["cu_seqlens"], x["max_seqlen"], x["scale"],
                             **kw)
            torch.cuda.synchronize()
        for r in runners:
            if r.w.name in STEP_WORKLOADS:
                o, lse = fa.fa_fwd_dropout(r.q, r.k, r.v, r.scale, DROPOUT_P, DROPOUT_SEED, True)
                fa.fa_bwd_dropout(r.q, r.k, r.v, o, r.do, lse, r.scale, DROPOUT_P, DROPOUT_SEED, True)
                torch.cuda.synchronize()
        for w, q, k, v, kv, scale, ws in dec:
            fa.fa_fwd_kvcache(q, k, v, scale, w.causal, kv, workspace=ws)
            torch.cuda.synchronize()
    print("counter pass done", flush=True)


def summarize_counters(sq_csv, fetch_csv, write_csv, trace_csv, valu_csv=None) -> str:
    """Markdown table per (workload, kernel) of the second round of `--counter-pass`:
    duration (kernel trace), HBM bytes and GB/s (FETCH_SIZE, WRITE_SIZE scaled by the
    calibration copy), MFMA busy and LDS bank conflicts (SQ counters), and with a VALU
    counter file the VALU-active cycles and VALU instructions per MFMA."""
    import csv
    from exact_tiled_attention_32_amd import workloads

    def ours(name):
        return "fa::" in name or "copyBuffer" in name

    def load(path):
        per = {}
        for row in csv.DictReader(open(path)):
            if not ours(row["Kernel_Name"]):
                continue
            d = per.setdefault(int(row["Dispatch_Id"]), {"name": row["Kernel_Name"]})
            d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
        return [per[k] for k in sorted(per)]

    def calib(rows, counter):
        # the calibration copy is the last device copy before the first library kernel
        # (the uploads of the inputs come before it)
        first = next(i for i, r in enumerate(rows) if "fa::" in r["name"])
        c = [r for r in rows[:first] if "copyBuffer" in r["name"]]
        return CALIBRATION_BYTES / (c[-1][counter] * 1024.0)

    sq, fe, wr = load(sq_csv), load(fetch_csv), load(write_csv)
    va = load(valu_csv) if valu_csv else None
    ff, fw = calib(fe, "FETCH_SIZE"), calib(wr, "WRITE_SIZE")
    trace = []
    for row in csv.DictReader(open(trace_csv)):
        if "fa::" in row["Kernel_Name"]:
            trace.append((int(row["Dispatch_Id"]), row["Kernel_Name"],
                          (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-3))
    trace.sort()
    seq = counter_sequence(workloads)
    strip = lambda rows: [r for r in rows if "copyBuffer" not in r["name"]]
    sq, fe, wr = strip(sq), strip(fe), strip(wr)
    checks = [("sq", sq), ("fetch", fe), ("write", wr), ("trace", trace)]
    if va is not None:
        va = strip(va)
        checks.append(("valu", va))
    for what, rows in checks:
        if len(rows) != len(seq):
            raise RuntimeError(f"{what}: {len(rows)} library dispatches, expected {len(seq)}")
    half = len(seq) // 2
    lines = ["| workload | kernel | µs | FETCH MB | WRITE MB | HBM GB/s | MFMA busy | VALU pipe | VALU insts / MFMA "
             "| LDS bank-conflict cycles / LDS active cycles | MFMA insts | LDS insts |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for i in range(half, len(seq)):
        wname, kname = seq[i]
        name = trace[i][1]
        if kname.split("<")[0] not in name:
            raise RuntimeError(f"dispatch {i}: expected {kname}, found {name}")
        us = trace[i][2]
        fb, wb = fe[i]["FETCH_SIZE"] * 1024.0 * ff, wr[i]["WRITE_SIZE"] * 1024.0 * fw
        c = sq[i]
        # SQ_VALU_MFMA_BUSY_CYCLES and SQ_BUSY_CU_CYCLES are both summed over the CUs; the
        # MFMA counter adds the nominal issue cycles of each MFMA instruction (32 for a
        # 32x32x16 bf16 one) over the CU's four SIMDs. Active MHz: GRBM_GUI_ACTIVE summed
        # over the 8 XCDs, per microsecond of the kernel.
        mfma = c["SQ_VALU_MFMA_BUSY_CYCLES"] / max(4.0 * c["SQ_BUSY_CU_CYCLES"], 1.0)
        bank = c["SQ_LDS_BANK_CONFLICT"] / max(c["SQ_LDS_IDX_ACTIVE"], 1.0)
        if va is not None:
            v = va[i]
            # VALU pipe: non-MFMA VALU instructions (SQ_INSTS_VALU counts MFMAs too) x 4 cycles
            # each (a wave64 instruction on a 16-lane SIMD) over the SIMD cycles (4 x
            # SQ_BUSY_CU_CYCLES, as for MFMA busy); transcendentals take longer, so this is a
            # lower bound of the pipe's occupancy
            valu = (f"{100 * 4.0 * (v['SQ_INSTS_VALU'] - v['SQ_INSTS_MFMA']) / max(4.0 * v['SQ_BUSY_CU_CYCLES'], 1.0):.1f}"
                    f" %")
            vpm = f"{(v['SQ_INSTS_VALU'] - v['SQ_INSTS_MFMA']) / max(v['SQ_INSTS_MFMA'], 1.0):.2f}"
        else:
            valu = vpm = "—"
        lines.append(f"| {wname} | {kname} | {us:.1f} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | "
                     f"{(fb + wb) / us / 1e3:.0f} | {100 * mfma:.1f} % | {valu} | {vpm} | {100 * bank:.2f} % | "
                     f"{c['SQ_INSTS_MFMA']:.3g} | {c['SQ_INSTS_LDS']:.3g} |")
    return "\n".join(lines)


STALL_COUNTERS_A = ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_ANY",
                    "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES")
STALL_COUNTERS_B = ("SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_SCA",
                    "SQ_ACTIVE_INST_MISC", "SQ_INST_LEVEL_LDS", "SQ_INSTS_LDS", "SQ_ACTIVE_INST_VMEM")


def summarize_stalls(a_csv, b_csv) -> str:
    """Markdown table per (workload, kernel) of the second round of `--counter-pass`, from two
    counter files taken with STALL_COUNTERS_A and STALL_COUNTERS_B: where the waves' cycles go
    (issuing an instruction, waiting for a wait count or the barrier, or holding an instruction
    that does not issue), the share of MFMA-busy cycles in which a vector instruction issued
    as well, and the cycles spent on vector, LDS and scalar instructions. Every share is of
    SQ_WAVE_CYCLES of the same run (the SQ_WAIT_* and SQ_ACTIVE_INST_* counters are in the
    same units)."""
    import csv
    from exact_tiled_attention_32_amd import workloads

    def load(path):
        per = {}
        for row in csv.DictReader(open(path)):
            if "fa::" not in row["Kernel_Name"]:
                continue
            d = per.setdefault(int(row["Dispatch_Id"]), {"name": row["Kernel_Name"]})
            d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
        return [per[k] for k in sorted(per)]

    A, B = load(a_csv), load(b_csv)
    seq = counter_sequence(workloads)
    for what, rows, names in (("A", A, STALL_COUNTERS_A), ("B", B, STALL_COUNTERS_B)):
        if len(rows) != len(seq):
            raise RuntimeError(f"{what}: {len(rows)} library dispatches, expected {len(seq)}")
        missing = [n for n in names if any(n not in r for r in rows)]
        if missing:
            raise RuntimeError(f"{what}: counters missing: {missing}")
    pct = lambda x: f"{100 * x:.1f} %"
    lines = ["| workload | kernel | MFMA busy | issuing | waiting (wait count, barrier) | ready, not issued "
             "| LDS issue wait | vector co-issue / MFMA busy | vector | LDS | scalar |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for i in range(len(seq) // 2, len(seq)):
        wname, kname = seq[i]
        a, b = A[i], B[i]
        if kname.split("<")[0] not in a["name"] or kname.split("<")[0] not in b["name"]:
            raise RuntimeError(f"dispatch {i}: expected {kname}, found {a['name']} / {b['name']}")
        wa, wb = max(a["SQ_WAVE_CYCLES"], 1.0), max(b["SQ_WAVE_CYCLES"], 1.0)
        mfma = a["SQ_VALU_MFMA_BUSY_CYCLES"] / max(4.0 * a["SQ_BUSY_CU_CYCLES"], 1.0)
        coex = a["SQ_VALU_MFMA_COEXEC_CYCLES"] / max(a["SQ_VALU_MFMA_BUSY_CYCLES"], 1.0)
        lines.append(f"| {wname} | {kname} | {pct(mfma)} | {pct(a['SQ_ACTIVE_INST_ANY'] / wa)} | "
                     f"{pct(a['SQ_WAIT_ANY'] / wa)} | {pct(a['SQ_WAIT_INST_ANY'] / wa)} | "
                     f"{pct(a['SQ_WAIT_INST_LDS'] / wa)} | {pct(coex)} | {pct(b['SQ_ACTIVE_INST_VALU'] / wb)} | "
                     f"{pct(b['SQ_ACTIVE_INST_LDS'] / wb)} | {pct(b['SQ_ACTIVE_INST_SCA'] / wb)} |")
    return "\n".join(lines)


def kernel_source_digest() -> str:
    """Digest of the step kernels' code: comments and whitespace are left out, so that
    only a change of the code itself invalidates counter data taken on it."""
    import re
    h = hashlib.sha256()
    for f in ("fa_device.h", "fa_bwd.hip", "fa_fwd.hip", "fa_launch.h"):
        with open(os.path.join(ROOT, "exact_tiled_attention_32_amd", "csrc", f)) as fh:
            code = fh.read()
        code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    entry = t.get("kernels", {}).get(kernel)
    if not entry or entry.get("source_digest") != kernel_source_digest():
        return None
    return entry.get("bytes_per_launch")


def cpu_info() -> dict:
    """The host the oracle runs on: CPU model, core counts, BLAS library and NumPy version."""
    import platform

    import numpy as np
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    blas = []
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas.append({"library": i.get("internal_api"), "version": i.get("version"),
                             "threads": i.get("num_threads")})
    except Exception:  # noqa: BLE001
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cores": affinity, "blas": blas,
            "numpy": np.__version__}


def _oracle_case(w):
    """fp64 copies of head (0, 0) of a workload's seeded inputs, plus its mask arguments."""
    import numpy as np
    from exact_tiled_attention_32_amd import workloads
    x = workloads.generate(w)
    head = {n: x[n][0:1, 0:1].float().numpy().astype(np.float64) for n in ("q", "k", "v")}
    head["do"] = None if x["do"] is None else x["do"][0:1, 0:1].float().numpy().astype(np.float64)
    kv = None if x["kv_len"] is None else int(x["kv_len"][0])
    bm = None if x["block_mask"] is None else x["block_mask"].numpy()
    return head, kv, bm


def oracle_config_timings(R_long: int) -> dict:
    """The fp64 oracle on each named workload: forward and backward timed separately on a
    bounded sample (head (0, 0); for the long workloads R query rows), with the sample's
    algorithmic GFLOP (4 d per allowed pair forward, 2.5x that backward)."""
    import numpy as np
    import oracle
    from exact_tiled_attention_32_amd import workloads
    out = {}
    for name, w in workloads.WORKLOADS.items():
        if name in ("long_causal_d32", "long_causal_d16"):
            continue
        head, kv, bm = _oracle_case(w)
        if w.N <= 1024:
            rows = np.arange(w.N)
            what = f"head (0,0), all {w.N} rows"
        elif w.sparse:
            rows = np.arange(16 * w.mask_block, 17 * w.mask_block)
            what = f"head (0,0), the {w.mask_block} rows of query block 16 against its kept key blocks"
        else:
            rows = np.arange(w.N - R_long, w.N)
            what = f"head (0,0), the last {R_long} rows with their full causal prefix"
        allow = oracle.allowed_pairs(rows, w.N, causal=w.causal, kv_len_b=kv, block_mask=bm,
                                     mask_block=w.mask_block)
        pairs = float(allow.sum())
        t0 = time.perf_counter()
        oracle.forward_rows(head["q"][0, 0, rows], head["k"][0, 0], head["v"][0, 0], w.scale, allow)
        t_fwd = time.perf_counter() - t0
        res = {"sample": what, "allowed_pairs": pairs, "fwd_s": round(t_fwd, 4),
               "fwd_gflops": round(4.0 * w.d * pairs / t_fwd / 1e9, 3)}
        if w.backward:
            t0 = time.perf_counter()
            oracle.attention_backward(head["q"], head["k"], head["v"], head["do"], w.scale, causal=w.causal,
                                      kv_len=None if kv is None else [kv], block_mask=bm,
                                      mask_block=w.mask_block, rows=rows)
            t_bwd = time.perf_counter() - t0
            res.update(bwd_s=round(t_bwd, 4), bwd_gflops=round(10.0 * w.d * pairs / t_bwd / 1e9, 3))
        out[name] = res
    return out


def cpu_baseline(target_s: float = 12.0) -> dict:
    """The fp64 oracle on a bounded sample of the step's workload: head (0, 0), the last R
    query rows (full causal prefix), forward + backward, for d = 64 and d = 128; then every
    named workload on a small sample (forward and backward separately)."""
    import numpy as np
    import oracle
    from exact_tiled_attention_32_amd import workloads
    info = cpu_info()
    threads = max([b["threads"] or 1 for b in info["blas"]] or [os.cpu_count() or 1])

    heads = {}
    for name in STEP_WORKLOADS:
        w = workloads.WORKLOADS[name]
        x = workloads.generate(w)
        heads[name] = (w, *(x[n][0:1, 0:1].float().numpy().astype(np.float64) for n in ("q", "k", "v", "do")))

    def run(R):
        flop, t0 = 0.0, time.perf_counter()
        for name in STEP_WORKLOADS:
            w, q, k, v, do = heads[name]
            rows = np.arange(w.N - R, w.N)
            allow = oracle.allowed_pairs(rows, w.N, causal=True, kv_len_b=None, block_mask=None, mask_block=128)
            oracle.forward_rows(q[0, 0, rows], k[0, 0], v[0, 0], w.scale, allow)
            oracle.attention_backward(q, k, v, do, w.scale, causal=True, rows=rows)
            pairs = float(np.sum(rows + 1))
            flop += 3.5 * 4.0 * w.d * pairs
        return flop, time.perf_counter() - t0

    # one warm-up on the single-head workload, then size R so that the timed run takes about
    # target_s (the work is close to linear in R; a second correction absorbs the start-up
    # share of the short calibration run)
    w1 = workloads.WORKLOADS["single_head_f32"]
    head1, _, _ = _oracle_case(w1)
    oracle.attention_forward(head1["q"], head1["k"], head1["v"], w1.scale)
    N = workloads.WORKLOADS[STEP_WORKLOADS[0]].N
    R = 512
    flop, dt = run(R)
    for _ in range(2):
        R = int(min(N, max(128, R * target_s / max(dt, 1e-3))))
        R = max(128, (R // 128) * 128)
        flop, dt = run(R)
        if dt >= 0.7 * target_s or R >= N:
            break
    per = oracle_config_timings(max(128, R // 8))
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 NumPy oracle, head (b=0,h=0) of the step's workloads (d=64 and d=128), the last {R} "
                      f"query rows of N=16384 with their full causal prefix, forward + backward; "
                      f"{flop / 1e9:.1f} GFLOP (same FLOP convention) in {dt:.1f} s",
            "host": info, "per_config": per, "note": "a baseline, not the target"}


def time_step(fa, runners, steps, warmup):
    """Exactly `warmup` untimed steps, then exactly `steps` timed steps with nothing but the
    library calls in them (the metric), then `steps` more with the library's per-kernel
    event markers armed (the per-kernel and per-phase figures; the markers cost the step
    about 1 %, so they stay out of the metric). Returns (ms per bare step, ms per
    instrumented step, the kernel clock)."""
    import torch
    # at ~7 ms a step, the default 10 warm-up steps also bring the engine clock up
    for _ in range(warmup):
        for r in runners:
            r.fwd()
            r.bwd()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        for r in runners:
            r.fwd()
            r.bwd()
    t1.record()
    torch.cuda.synchronize()
    bare_ms = t0.elapsed_time(t1) / steps
    clock = KernelClock()
    # the kernel clock's events are made before the instrumented region
    evs = [[(KernelClock.new_events(2), KernelClock.new_events(1 + len(r.bwd_kernels))) for r in runners]
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        for r, (ef, eb) in zip(runners, evs[i]):
            clock.arm(fa, f"fwd_d{r.w.d}", ef)
            r.fwd()
            clock.arm(fa, f"bwd_d{r.w.d}", eb)
            r.bwd()
    t1.record()
    torch.cuda.synchronize()
    return bare_ms, t0.elapsed_time(t1) / steps, clock


def sample_clock(fn, seconds: float = 3.0) -> dict:
    """Engine clock while `fn` (one step) runs back to back for `seconds`: rocm-smi (or
    amd-smi) is polled from a second thread; each reading is a child process."""
    import re
    import subprocess
    import threading

    import torch
    cmds = [["rocm-smi", "--showclocks"], ["amd-smi", "metric", "--clock"]]
    samples, tool = [], None
    stop = threading.Event()

    def poll():
        nonlocal tool
        while not stop.is_set():
            for c in cmds:
                try:
                    out = subprocess.run(c, capture_output=True, text=True, timeout=10).stdout
                except (OSError, subprocess.SubprocessError):
                    continue
                # rocm-smi: "sclk clock level: N: (1700Mhz)"; amd-smi: a GFX clock block "CLK: 1700 MHz"
                vals = [int(x) for x in re.findall(r"sclk[^\n]*?\((\d+)\s*mhz\)", out, flags=re.I)]
                if not vals:
                    vals = [int(x) for x in re.findall(r"gfx[_\s]*0?[^\n]*\n?[^\n]*?clk[^\d\n]*(\d+)\s*mhz",
                                                        out, flags=re.I)]
                if vals:
                    tool = c[0]
                    samples.append(vals[0])
                    break
            stop.wait(0.2)

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t_end = time.perf_counter() + seconds
    n = 0
    while time.perf_counter() < t_end:
        fn()
        n += 1
        if n % 20 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    if not samples:
        return {"source": None, "samples": 0, "note": "no clock reading from rocm-smi or amd-smi"}
    return {"source": tool, "samples": len(samples), "sclk_mhz_mean": round(sum(samples) / len(samples)),
            "sclk_mhz_min": min(samples), "sclk_mhz_max": max(samples),
            "during": f"the step run back to back for {seconds:.0f} s after the timed region"}


def decode_bytes(w, kv_len) -> float:
    """Algorithmic HBM bytes of one cache-forward call: every valid cached key and value
    read once (bf16), the queries read and the outputs written once."""
    lens = [w.Nk] * w.B if kv_len is None else [min(max(int(x), 0), w.Nk) for x in kv_len.tolist()]
    return 2.0 * 2 * w.H * w.d * sum(lens) + 2.0 * 2 * w.B * w.H * w.Nq * w.d


def report_decode(fa, w, dev, steps, warmup) -> dict:
    """Cache-forward timing of one decode workload: whole call and key-split kernel."""
    import torch
    from exact_tiled_attention_32_amd import workloads
    x = workloads.generate_decode(w)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    kv = None if x["kv_len"] is None else x["kv_len"].to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    ws = torch.empty(fa.fa_fwd_kvcache_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d), dtype=torch.uint8, device=dev)

    def call():
        fa.fa_fwd_kvcache(q, k, v, x["scale"], w.causal, kv, o=o, lse=lse, workspace=ws)

    warm_up(call, warmup)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        call()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    # second pass with the library's events around the key-split kernel (their records
    # add gaps between launches, so the whole-call time above is taken without them)
    clock = KernelClock()
    evs = [KernelClock.new_events(3) for _ in range(steps)]
    for e in evs:
        clock.arm(fa, "split", e)
        call()
    torch.cuda.synchronize()
    split_ms = clock.kernel_ms("split", 0)
    nbytes = decode_bytes(w, x["kv_len"])
    return {"shape": {"B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d}, "causal": w.causal,
            "padding": w.padding, "algorithmic_bytes": nbytes, "ms": ms, "split_kernel_ms": split_ms,
            "gbs": nbytes / ms / 1e6, "split_kernel_gbs": nbytes / split_ms / 1e6,
            "frac_of_hbm_peak": nbytes / ms / 1e6 / PEAK_HBM_GBS}


def allowed_pair_count(n: int, causal: bool, wl: int, wr: int) -> int:
    """Query-key pairs a sequence of n tokens attends under the causal / window rules."""
    import numpy as np
    i = np.arange(n, dtype=np.int64)
    lo = np.maximum(i - wl, 0) if wl >= 0 else np.zeros_like(i)
    right = 0 if causal else wr
    hi = np.minimum(i + right, n - 1) if right >= 0 else np.full_like(i, n - 1)
    return int(np.maximum(hi - lo + 1, 0).sum())


def report_varlen(fa, w, dev, steps, warmup) -> dict:
    """Forward and backward timing of one packed workload. FLOP: 4 d per allowed pair
    (forward) and 2.5x that (backward), counted exactly over the sequences."""
    import torch
    from exact_tiled_attention_32_amd import workloads
    x = workloads.generate_varlen(w)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    cu = x["cu_seqlens"].to(dev)
    lens = (x["cu_seqlens"][1:] - x["cu_seqlens"][:-1]).tolist()
    pairs = sum(allowed_pair_count(n, w.causal, w.window_left, w.window_right) for n in lens)
    fwd_flop = 4.0 * w.d * w.H * pairs
    kw = dict(causal=w.causal, window_left=w.window_left, window_right=w.window_right)
    o = torch.empty_like(q)
    lse = torch.empty((w.H, q.shape[0]), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_varlen_workspace_bytes(w.H, q.shape[0], w.d), dtype=torch.uint8, device=dev)
    fns = {
        "fwd": lambda: fa.fa_fwd_varlen(q, k, v, cu, x["max_seqlen"], x["scale"], o=o, lse=lse, **kw),
        "bwd": lambda: fa.fa_bwd_varlen(q, k, v, o, do, lse, cu, x["max_seqlen"], x["scale"], dq=dq, dk=dk, dv=dv,
                                        workspace=ws, **kw),
    }
    res = {"sequences": len(lens), "tokens": int(q.shape[0]), "H": w.H, "d": w.d, "causal": w.causal,
           "window_left": w.window_left, "window_right": w.window_right, "allowed_pairs_per_head": pairs}
    for phase, fn in fns.items():
        warm_up(fn, warmup)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        flop = fwd_flop * (2.5 if phase == "bwd" else 1.0)
        res[phase] = {"ms": round(ms, 4), "tflops": round(flop / ms / 1e9, 1),
                      "frac_of_peak": round(flop / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
    return res


def report_dropout(fa, w, dev, steps, warmup) -> dict:
    """Forward and backward with dropout (p = DROPOUT_P) on one of the step's workloads,
    whole calls timed with events, plus the dominant kernel of each (forward kernel; dK/dV
    kernel) through the library's event hook. FLOP as in the step; the generator's work is
    not counted."""
    import torch
    from exact_tiled_attention_32_amd import workloads
    x = workloads.generate(w)
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    fns = {
        "fwd": lambda: fa.fa_fwd_dropout(q, k, v, x["scale"], DROPOUT_P, DROPOUT_SEED, w.causal, o=o, lse=lse),
        "bwd": lambda: fa.fa_bwd_dropout(q, k, v, o, do, lse, x["scale"], DROPOUT_P, DROPOUT_SEED, w.causal,
                                         dq=dq, dk=dk, dv=dv, workspace=ws),
    }
    res = {"p": DROPOUT_P, "d": w.d}
    kernels = {"fwd": ["fwd"], "bwd": ["bwd_dq", "bwd_dkdv"]}
    for phase, fn in fns.items():
        warm_up(fn, warmup)
        clock = KernelClock()
        evs = [KernelClock.new_events(1 + len(kernels[phase])) for _ in range(steps)]
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for e in evs:
            clock.arm(fa, phase, e)
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        flop = attn_flops(w) * (2.5 if phase == "bwd" else 1.0)
        res[phase] = {"ms": round(ms, 4), "tflops": round(flop / ms / 1e9, 1),
                      "frac_of_peak": round(flop / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
        for i, kname in enumerate(kernels[phase]):
            res[phase][kname + "_kernel_ms"] = round(clock.kernel_ms(phase, i), 4)
    return res


def report_graph(fa, w, dev, steps, warmup) -> dict:
    """Forward + backward of a short-sequence workload: eager calls against the same two
    calls captured once in a HIP graph (torch.cuda.CUDAGraph) and replayed. At these sizes
    the kernels last tens of microseconds, so launch overheads and the gaps between
    launches are a visible part of a call."""
    import torch
    r = Runner(fa, w, dev)

    def step():
        r.fwd()
        r.bwd()
    warm_up(step, warmup)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    def timed(fn):
        warm_up(fn, warmup)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    eager_ms, graph_ms = timed(step), timed(g.replay)
    flop = 3.5 * attn_flops(w)
    del g, r
    return {"shape": [w.B, w.H, w.N, w.d], "causal": w.causal, "padding": w.padding,
            "eager_ms": round(eager_ms, 4), "graph_ms": round(graph_ms, 4),
            "eager_tflops": round(flop / eager_ms / 1e9, 1), "graph_tflops": round(flop / graph_ms / 1e9, 1)}


GRAPH_PASS_WORKLOADS = ("bert_padded", "gpt2_causal")
GRAPH_PASS_WARM = 5


def graph_pass(fa, dev, steps) -> dict:
    """Eager steps against replays of the same step captured in a HIP graph, for the short
    workloads: four blocks per workload (eager, graph, eager, graph) of GRAPH_PASS_WARM
    untimed and `steps` timed steps; per block the GPU time per step (HIP events) and the
    host time to issue a step. Under a kernel trace the blocks give the kernel timeline of
    both modes (summarize_graph_trace)."""
    import time
    import torch
    from exact_tiled_attention_32_amd import workloads
    out = {}
    for name in GRAPH_PASS_WORKLOADS:
        r = Runner(fa, workloads.WORKLOADS[name], dev)

        def step():
            r.fwd()
            r.bwd()
        for _ in range(GRAPH_PASS_WARM):  # a fixed count: the trace summary counts dispatches
            step()
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        blocks = []
        for mode, fn in (("eager", step), ("graph", g.replay), ("eager", step), ("graph", g.replay)):
            for _ in range(GRAPH_PASS_WARM):
                fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            h0 = time.perf_counter()
            for _ in range(steps):
                fn()
            h1 = time.perf_counter()
            b.record()
            torch.cuda.synchronize()
            blocks.append({"mode": mode, "gpu_ms_per_step": round(a.elapsed_time(b) / steps, 4),
                           "host_ms_per_step": round((h1 - h0) * 1e3 / steps, 4)})
        out[name] = blocks
        print(f"[graph-pass] {name}: " + json.dumps(blocks), flush=True)
        del g, r
        torch.cuda.empty_cache()
    return out


def summarize_graph_trace(trace_csv: str, steps: int) -> str:
    """Markdown table of a kernel trace of `--graph-pass`: per workload and block, the median
    kernel durations, the idle gaps inside a step and between steps, and the step span."""
    import statistics
    rows = [r for r in csv.DictReader(open(trace_csv)) if "fa::" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    seq = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows]
    trip = [seq[i:i + 3] for i in range(0, len(seq) - 2, 3)]  # forward, dQ, dK/dV
    per = GRAPH_PASS_WARM + 1 + 4 * (GRAPH_PASS_WARM + steps)  # warm-up, side stream, blocks
    if len(seq) != 3 * per * len(GRAPH_PASS_WORKLOADS):
        raise ValueError(f"{len(seq)} library dispatches in the trace, expected "
                         f"{3 * per * len(GRAPH_PASS_WORKLOADS)} for --graph-pass --steps {steps}")
    lines = ["| workload | mode | forward | dQ | dK/dV | idle gap forward→dQ | idle gap between steps | step span |",
             "|---|---|---|---|---|---|---|---|"]
    med = lambda xs: round(statistics.median(xs) / 1000, 1)
    for wi, name in enumerate(GRAPH_PASS_WORKLOADS):
        st = trip[wi * per:(wi + 1) * per]
        for blk in range(4):
            lo = GRAPH_PASS_WARM + 1 + blk * (GRAPH_PASS_WARM + steps) + GRAPH_PASS_WARM
            seg = st[lo:lo + steps]
            if len(seg) < 2:
                continue
            dur = [[e - s for s, e in t] for t in seg]
            gap = [max(t[1][0] - t[0][1], 0) for t in seg]
            inter = [max(seg[i][0][0] - seg[i - 1][2][1], 0) for i in range(1, len(seg))]
            span = [t[2][1] - t[0][0] for t in seg]
            lines.append(f"| {name} | {'eager' if blk % 2 == 0 else 'graph'} | " +
                         " | ".join(str(med(x)) for x in zip(*dur)) +
                         f" | {med(gap)} | {med(inter)} | {med(span)} |")
    return "\n".join(lines)


def compulsory_bytes(w, phase: str) -> float:
    """Algorithmic HBM bytes of one call: forward Q, K, V read and O written once plus lse;
    backward Q, K, V, O, dO read and dQ, dK, dV written once, lse read, D written and read."""
    el = 4 if w.dtype == "f32" else 2
    nd = w.B * w.H * w.N * w.d
    rows = w.B * w.H * w.N
    return (4 * nd * el + 4 * rows) if phase == "fwd" else (8 * nd * el + 12 * rows)


def kept_pair_flops(w, kv_len) -> float:
    """Forward FLOP over the allowed pairs only (4 d per pair) for key padding: each of the N
    query rows of batch b attends its L_b valid keys (non-causal)."""
    return 4.0 * w.H * w.d * w.N * float(sum(min(max(int(x), 0), w.N) for x in kv_len))


def phase_figures(ms: float, flop: float, nbytes: float, peak: float = PEAK_BF16_TFLOPS) -> dict:
    """ms, TFLOP/s, fraction of `peak` (the dense MFMA peak of the call's dtype) and HBM rate
    of the compulsory bytes."""
    return {"ms": round(ms, 4), "tflops": round(flop / ms / 1e9, 1),
            "frac_of_peak": round(flop / ms / 1e9 / peak, 4),
            "hbm_gbs": round(nbytes / ms / 1e6, 1), "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)}


def report_config(fa, w, dev, steps=50, warmup=3) -> dict:
    """Forward and backward of one named workload, timed separately: `steps` back-to-back
    whole calls between two HIP events on the launch stream (the mean, `ms`), then `steps`
    more with the library's per-kernel events armed (each kernel's mean, and the median of
    the calls' first-to-last-kernel time, `median_call_ms`). TFLOP/s by the headline
    convention (dense N^2, halved for causal; kept blocks for a block mask), and by allowed
    pairs for key padding; HBM GB/s of the compulsory bytes."""
    import torch
    r = Runner(fa, w, dev)
    ff = attn_flops(w, r.kept)
    peak = PEAK_F32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS
    res = {"shape": [w.B, w.H, w.N, w.d], "dtype": w.dtype, "causal": w.causal, "padding": w.padding,
           "sparse": w.sparse, "fwd_gflop": round(ff / 1e9, 3), "peak_tflops": peak}
    if r.kept is not None:
        res["kept_block_fraction"] = round(r.kept, 5)
        res["flop_convention"] = "kept 128x128 blocks only"
    kept_ff = None
    if r.kv is not None:
        kept_ff = kept_pair_flops(w, r.kv.cpu().tolist())
        res["flop_convention"] = "dense N^2 (tflops); allowed pairs only (tflops_kept_pairs)"
        res["kept_pair_fraction"] = round(kept_ff / attn_flops(w), 4)
    kernels = {"fwd": ["fwd"], "bwd": r.bwd_kernels if w.backward else []}
    for phase in ("fwd", "bwd") if w.backward else ("fwd",):
        fn = r.fwd if phase == "fwd" else r.bwd
        warm_up(fn, warmup)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        clock = KernelClock()
        evs = [KernelClock.new_events(1 + len(kernels[phase])) for _ in range(steps)]
        torch.cuda.synchronize()
        for e in evs:
            clock.arm(fa, phase, e)
            fn()
        torch.cuda.synchronize()
        mult = 2.5 if phase == "bwd" else 1.0
        fig = phase_figures(ms, ff * mult, compulsory_bytes(w, phase), peak)
        if kept_ff is not None:
            fig["tflops_kept_pairs"] = round(kept_ff * mult / ms / 1e9, 1)
            fig["frac_of_peak_kept_pairs"] = round(kept_ff * mult / ms / 1e9 / peak, 4)
        if w.dtype == "f32":
            fig["us"] = round(ms * 1e3, 2)
        fig["median_call_ms"] = round(clock.call_ms_median(phase), 4)
        for i, kname in enumerate(kernels[phase]):
            fig[kname + "_kernel_ms"] = round(clock.kernel_ms(phase, i), 4)
        res[phase] = fig
    del r
    torch.cuda.empty_cache()
    return res


def report_all(fa, dev, path, steps=10, warmup=3):
    """Every workload (forward and backward separately), packed and decode workloads; written
    to `path` (not the metric line)."""
    import torch
    from exact_tiled_attention_32_amd import workloads
    out = {}
    for name, w in workloads.WORKLOADS.items():
        out[name] = report_config(fa, w, dev, steps, warmup)
        print(f"[report] {name}: " + json.dumps({k: v for k, v in out[name].items() if k in ("fwd", "bwd")}),
              flush=True)
    for name, w in workloads.VARLEN_WORKLOADS.items():
        out[name] = report_varlen(fa, w, dev, steps, warmup)
        print(f"[report] {name}: " + json.dumps({k: out[name][k] for k in ("fwd", "bwd")}), flush=True)
        torch.cuda.empty_cache()
    for name, w in workloads.DECODE_WORKLOADS.items():
        out[name] = report_decode(fa, w, dev, steps, warmup)
        print(f"[report] {name}: " + json.dumps({k: out[name][k] for k in ("ms", "split_kernel_ms", "gbs")}),
              flush=True)
        torch.cuda.empty_cache()
    with open(path, "w") as f:
        json.dump(out, f, indent=1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--report", default=None, help="also time every workload and write this JSON file")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/hbm_traffic.json from two rocprofv3 counter files and exit")
    ap.add_argument("--counter-pass", action="store_true",
                    help="for rocprofv3 --pmc / --kernel-trace: a calibration copy, then every workload once, "
                         "twice over; prints no metric line")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="SQ_CSV FETCH_CSV WRITE_CSV TRACE_CSV [VALU_CSV]: print the per-kernel counter table "
                         "of a --counter-pass and exit")
    ap.add_argument("--summarize-stalls", nargs=2, metavar=("A_CSV", "B_CSV"),
                    help="print the per-kernel wave-cycle table of a --counter-pass taken with the "
                         "STALL_COUNTERS_A and STALL_COUNTERS_B sets, and exit")
    ap.add_argument("--step-only", action="store_true",
                    help="time the step alone (no decode or packed workloads), e.g. under a kernel trace")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the key/value-cache forward on the decode workloads and print them")
    ap.add_argument("--graph-pass", action="store_true",
                    help="eager steps against replayed HIP-graph steps on the short workloads (four "
                         "blocks of --steps each); prints per-block times, no metric line")
    ap.add_argument("--summarize-graph-trace", metavar="TRACE_CSV",
                    help="print the kernel timeline table of a traced --graph-pass (same --steps) and exit")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="for rocprofv3 --pmc: one 256 MiB device copy (counter calibration), then one "
                         "untimed pass of the step; prints no metric line")
    args = ap.parse_args()
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters))
        return
    if args.summarize_stalls:
        print(summarize_stalls(*args.summarize_stalls))
        return
    if args.summarize_graph_trace:
        print(summarize_graph_trace(args.summarize_graph_trace, args.steps))
        return
    if args.summarize_pmc:
        res = summarize_pmc(*args.summarize_pmc, os.path.join(ROOT, "profiles", "hbm_traffic.json"))
        print(json.dumps(res, indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (got --gpus {args.gpus}); "
              "attention heads are independent, so a multi-GPU run would split B*H across GPUs", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_tiled_attention_32_amd as fa
    from exact_tiled_attention_32_amd import workloads
    fa.load()
    dev = "cuda:0"
    if args.counter_pass:
        counter_pass(fa, dev)
        return
    if args.graph_pass:
        graph_pass(fa, dev, args.steps)
        return
    if args.decode_only:
        for name, w in workloads.DECODE_WORKLOADS.items():
            print(json.dumps({"workload": name, **report_decode(fa, w, dev, args.steps, args.warmup)}), flush=True)
        return
    runners = [Runner(fa, workloads.WORKLOADS[n], dev) for n in STEP_WORKLOADS]
    if args.pmc_pass:
        src = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # reads and writes exactly CALIBRATION_BYTES each
        for r in runners:
            r.fwd()
            r.bwd()
        torch.cuda.synchronize()
        print(f"pmc pass done: calibration copy of {CALIBRATION_BYTES} bytes, one step", flush=True)
        return
    ms, ms_instr, clock = time_step(fa, runners, args.steps, args.warmup)
    step_flop = sum(3.5 * attn_flops(r.w) for r in runners)
    value = step_flop / (ms * 1e-3) / 1e12

    # per head dimension: the forward and backward phases of the step, and each kernel
    phases, kern = {}, {}
    for r in runners:
        d, f = r.w.d, attn_flops(r.w)
        k_ms = {"fwd": clock.kernel_ms(f"fwd_d{d}", 0)}
        for i, k in enumerate(r.bwd_kernels):
            k_ms[k] = clock.kernel_ms(f"bwd_d{d}", i)
        fwd_ms, bwd_ms = k_ms["fwd"], clock.call_ms(f"bwd_d{d}")
        phases[f"d{d}"] = {
            "fwd": phase_figures(fwd_ms, f, compulsory_bytes(r.w, "fwd")),
            "bwd": phase_figures(bwd_ms, 2.5 * f, compulsory_bytes(r.w, "bwd")),
            "fwd_bwd_tflops": round(3.5 * f / (fwd_ms + bwd_ms) / 1e9, 1),
        }
        for k, kms in k_ms.items():
            alg = KERNEL_FLOP_FACTOR[k] * f
            kern[f"{k}_d{d}"] = {"ms": round(kms, 4), "algorithmic_tflop_per_launch": round(alg / 1e12, 4),
                                 "tflops": round(alg / kms / 1e9, 1),
                                 "frac": round(alg / kms / 1e9 / PEAK_BF16_TFLOPS, 4),
                                 "executed_frac": round(KERNEL_EXECUTED_FACTOR[k] * f / kms / 1e9 / PEAK_BF16_TFLOPS,
                                                        4)}
    # dominant kernel: the one with the largest time per step
    dom_name = max(kern, key=lambda k: kern[k]["ms"])
    dom = kern[dom_name]
    roofline = {"bound": "mfma", "achieved": dom["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": dom["frac"], "traffic": load_traffic(dom_name), "kernel": dom_name, "kernel_ms": dom["ms"],
                "algorithmic_tflop_per_launch": dom["algorithmic_tflop_per_launch"],
                "kernels": {k: v["frac"] for k, v in kern.items()},
                "bwd_phase": {d: p["bwd"]["frac_of_peak"] for d, p in phases.items()},
                "fwd_phase": {d: p["fwd"]["frac_of_peak"] for d, p in phases.items()}}
    line = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic (iid N(0,1), seeded)",
            "config": {"workload": "long-sequence causal attention fwd+bwd, B=1 H=16 N=16384, d=64 and d=128",
                       "B": 1, "H": 16, "N": 16384, "d": [64, 128], "causal": True},
            "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
            "instrumented_ms_per_step": round(ms_instr, 4), "phases": phases, "kernels": kern,
            "roofline": roofline}

    def one_step():
        for r in runners:
            r.fwd()
            r.bwd()
    line["clock"] = sample_clock(one_step, 3.0)
    mhz = line["clock"].get("sclk_mhz_mean")
    if mhz:
        # context only: the matrix rate the sampled clock allows, and the dominant kernel
        # against it (the roofline fraction stays against the published peak)
        at_clock = PEAK_BF16_TFLOPS * mhz / PEAK_CLOCK_MHZ
        line["clock"]["bf16_peak_tflops_at_mean_clock"] = round(at_clock, 1)
        line["roofline"]["frac_at_mean_clock"] = round(roofline["achieved"] / at_clock, 4)
    if not args.step_only:
        # every named workload, forward and backward separately (the step's own two from the
        # step above)
        cfgs = {}
        for name, w in workloads.WORKLOADS.items():
            if name in STEP_WORKLOADS:
                p = phases[f"d{w.d}"]
                cfgs[name] = {"shape": [w.B, w.H, w.N, w.d], "causal": True, "from": "the timed step",
                              "fwd": p["fwd"], "bwd": p["bwd"]}
            elif name in ("long_causal_d32", "long_causal_d16"):
                continue
            else:
                cfgs[name] = report_config(fa, w, dev)
        line["configs"] = cfgs
    # the key/value-cache forward (HBM-bound) on its decode workloads, outside the step
    dec = {}
    for name, w in ({} if args.step_only else workloads.DECODE_WORKLOADS).items():
        r = report_decode(fa, w, dev, 20, 5)
        dec[name] = {"ms": round(r["ms"], 4), "split_kernel_ms": round(r["split_kernel_ms"], 4),
                     "gbs": round(r["gbs"], 1), "frac_of_hbm_peak": round(r["frac_of_hbm_peak"], 4),
                     "algorithmic_mb": round(r["algorithmic_bytes"] / 1e6, 1)}
        del r
        torch.cuda.empty_cache()
    if not args.step_only:
        line["kvcache_decode"] = dec
        # packed variable-length sequences and the sliding window, outside the step
        line["varlen"] = {name: report_varlen(fa, w, dev, 10, 3) for name, w in workloads.VARLEN_WORKLOADS.items()}
        torch.cuda.empty_cache()
        # dropout on the step's workloads, outside the step
        line["dropout"] = {name: report_dropout(fa, workloads.WORKLOADS[name], dev, 10, 3) for name in STEP_WORKLOADS}
        torch.cuda.empty_cache()
        # the short-sequence workloads (BERT- and GPT-2-shaped), fwd + bwd, eager and as a
        # replayed HIP graph (TFLOP/s by the step's convention, dense N^2 for key padding)
        # (a failed capture is recorded, not raised: it must not cost the metric line)
        short = {}
        for name in SHORT_WORKLOADS:
            try:
                short[name] = report_graph(fa, workloads.WORKLOADS[name], dev, 50, 10)
            except RuntimeError as e:
                torch.cuda.synchronize()
                short[name] = {"error": str(e)[:200]}
        line["short_n"] = short
        torch.cuda.empty_cache()
    if args.report:
        report_all(fa, dev, args.report)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
