"""Host-side logic of bench.py (no GPU): the FLOP and byte conventions behind the metric
line, the digest that gates the committed traffic figures, the dispatch sequence the
counter summary expects, and the refusal of more than one GPU."""
import json
import os
import shutil
import subprocess
import sys

import pytest
import torch

import bench
from exact_tiled_attention_32_amd import workloads


def test_attn_flops_convention():
    # 4 B H N^2 d for the forward, halved for causal attention
    assert bench.attn_flops(workloads.WORKLOADS["long_causal_d128"]) == 4.0 * 16 * 16384 ** 2 * 128 / 2
    assert bench.attn_flops(workloads.WORKLOADS["bert_padded"]) == 4.0 * 8 * 16 * 512 ** 2 * 64
    w = workloads.WORKLOADS["block_sparse_64k"]
    assert bench.attn_flops(w, 0.068) == pytest.approx(4.0 * 8 * 65536 ** 2 * 64 * 0.068)


@pytest.mark.parametrize("n", [0, 1, 2, 7, 33])
@pytest.mark.parametrize("causal,wl,wr", [(False, -1, -1), (True, -1, -1), (True, 3, -1), (False, 2, 5),
                                           (False, 0, 0), (False, -1, 4), (True, 0, -1), (True, 2, 9)])
def test_allowed_pair_count_brute_force(n, causal, wl, wr):
    # key j is allowed for query i iff i - wl <= j <= i + wr (each side unbounded when -1);
    # causal attention is wr = 0, whatever wr says
    count = 0
    for i in range(n):
        for j in range(n):
            if causal and j > i:
                continue
            if wl >= 0 and j < i - wl:
                continue
            if not causal and wr >= 0 and j > i + wr:
                continue
            count += 1
    assert bench.allowed_pair_count(n, causal, wl, wr) == count


def test_decode_bytes():
    w = workloads.DecodeWorkload("tiny", B=2, H=3, Nq=4, Nk=100, d=64, seed=0)
    q_and_o = 2 * 2 * (2 * 3 * 4 * 64)  # bf16 queries read, outputs written
    kv = lambda keys: 2 * 2 * 3 * 64 * keys  # bf16 keys and values of every valid position
    assert bench.decode_bytes(w, torch.tensor([100, 37])) == kv(137) + q_and_o
    assert bench.decode_bytes(w, None) == kv(200) + q_and_o
    assert bench.decode_bytes(w, torch.tensor([500, -3])) == kv(100) + q_and_o  # clamped to [0, Nk]


def test_traffic_gated_by_source_digest(monkeypatch):
    with open(os.path.join(bench.ROOT, "profiles", "hbm_traffic.json")) as f:
        entry = json.load(f)["kernels"]["bwd_dkdv_d128"]
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: entry["source_digest"])
    assert bench.load_traffic("bwd_dkdv_d128") == entry["bytes_per_launch"]
    assert bench.load_traffic("no_such_kernel") is None
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 16)
    assert bench.load_traffic("bwd_dkdv_d128") is None


def test_digest_ignores_comments_only(tmp_path, monkeypatch):
    src = os.path.join(bench.ROOT, "exact_tiled_attention_32_amd", "csrc")
    dst = tmp_path / "exact_tiled_attention_32_amd" / "csrc"
    dst.mkdir(parents=True)
    for f in ("fa_device.h", "fa_bwd.hip", "fa_fwd.hip", "fa_launch.h"):
        shutil.copy(os.path.join(src, f), dst / f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_source_digest()
    path = dst / "fa_fwd.hip"
    code = path.read_text()
    path.write_text("// a new comment\n/* and a block\n   comment */\n" + code.replace("\n", "\n\n", 3))
    assert bench.kernel_source_digest() == base
    path.write_text(code.replace("kRescaleLog2 = 8.0f", "kRescaleLog2 = 4.0f"))
    assert bench.kernel_source_digest() != base


def test_counter_sequence():
    seq = bench.counter_sequence(workloads)
    half = len(seq) // 2
    assert seq[:half] == seq[half:]  # two identical rounds, the second is summarised
    names = {w for w, _ in seq}
    assert set(workloads.WORKLOADS) | set(workloads.VARLEN_WORKLOADS) | set(workloads.DECODE_WORKLOADS) <= names
    assert {n + "_dropout" for n in bench.STEP_WORKLOADS} <= names
    kernels = {}
    for w, k in seq[:half]:
        kernels.setdefault(w, []).append(k.split("<")[0])
    # the backward: (block mask: the key-tile order,) the dQ kernel, whose prologue writes D,
    # then the dK/dV kernel that reads it
    assert kernels["block_sparse_64k"] == ["fwd_bf16_kernel", "bwd_order_kernel", "bwd_dq_kernel",
                                           "bwd_dkdv_kernel"]
    assert kernels["long_causal_d128"] == ["fwd_bf16_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel"]
    assert kernels["single_head_f32"] == ["fwd_f32_kernel"]
    assert kernels["decode_q1_d128"] == ["kvc_split_kernel", "kvc_merge_kernel"]


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=bench.ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_warm_up_runs_the_minimum_calls_and_time(monkeypatch):
    # at least `calls` calls and at least `min_s` seconds, with the device synchronised
    # after each call past the minimum count (so the time counted is device time)
    import time
    syncs = []
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: syncs.append(1))
    calls = []
    t0 = time.perf_counter()
    bench.warm_up(lambda: calls.append(1), 5, 0.05)
    assert len(calls) >= 5 and time.perf_counter() - t0 >= 0.05
    assert len(syncs) >= len(calls) - 4
    calls.clear()
    bench.warm_up(lambda: calls.append(1), 3, 0.0)
    assert len(calls) == 3


def test_compulsory_bytes():
    # forward: Q, K, V read and O written once (bf16) plus lse; backward: Q, K, V, O, dO read,
    # dQ, dK, dV written, lse read, D written and read
    w = workloads.WORKLOADS["long_causal_d128"]
    nd, rows = 16 * 16384 * 128, 16 * 16384
    assert bench.compulsory_bytes(w, "fwd") == 4 * nd * 2 + 4 * rows
    assert bench.compulsory_bytes(w, "bwd") == 8 * nd * 2 + 12 * rows
    w1 = workloads.WORKLOADS["single_head_f32"]
    assert bench.compulsory_bytes(w1, "fwd") == 4 * 128 * 64 * 4 + 4 * 128


def test_kept_pair_flops_brute_force():
    # key padding, non-causal: every query row of batch b attends its L_b valid keys
    w = workloads.Workload("tiny", B=3, H=2, N=10, d=8, dtype="bf16", seed=0, padding=True)
    lens = [10, 4, 0]
    pairs = sum(1 for b in range(3) for i in range(10) for j in range(10) if j < lens[b])
    assert bench.kept_pair_flops(w, lens) == 4.0 * 2 * 8 * pairs
    assert bench.kept_pair_flops(w, [12, -1, 3]) == 4.0 * 2 * 8 * 10 * (10 + 0 + 3)  # clamped to [0, N]


class _FakeEvent:
    def __init__(self, t):
        self.t = t

    def elapsed_time(self, other):
        return other.t - self.t


def test_kernel_clock_arithmetic(monkeypatch):
    # events[0] before the first kernel, events[i] after the i-th: kernel i lasts
    # events[i + 1] - events[i]; the call spans events[0] .. events[-1]
    class FakeFa:
        armed = []

        def fa_time_next_call(self, events):
            self.armed.append(events)

    fa = FakeFa()
    clock = bench.KernelClock()
    clock.arm(fa, "bwd", [_FakeEvent(t) for t in (0.0, 1.0, 4.0)])
    clock.arm(fa, "bwd", [_FakeEvent(t) for t in (10.0, 12.0, 14.0)])
    assert len(fa.armed) == 2
    assert clock.kernel_ms("bwd", 0) == pytest.approx(1.5)
    assert clock.kernel_ms("bwd", 1) == pytest.approx(2.5)
    assert clock.call_ms("bwd") == pytest.approx(4.0)


def test_summarize_graph_trace(tmp_path):
    """The graph-pass timeline table: per block, median kernel durations and idle gaps, from
    a synthetic kernel trace laid out as --graph-pass dispatches (warm-up, side-stream step,
    four blocks of warm-up + timed steps per workload)."""
    steps, warm = 4, bench.GRAPH_PASS_WARM
    per = warm + 1 + 4 * (warm + steps)
    rows, t = [], 0
    for wi in range(len(bench.GRAPH_PASS_WORKLOADS)):
        for i in range(per):
            blk = (i - warm - 1) // (warm + steps) if i >= warm + 1 else -1
            graph = blk in (1, 3)
            dur = (10_000 * (wi + 1), 20_000, 30_000)      # ns
            t += 8_000 if graph else 0                     # idle gap before each graph step
            for k, name in enumerate(("fa::fwd_bf16_kernel", "fa::bwd_dq_kernel", "fa::bwd_dkdv_kernel")):
                if k == 1 and not graph:
                    t += 2_000                             # host gap inside an eager step
                rows.append((name, t, t + dur[k]))
                t += dur[k]
    path = tmp_path / "trace.csv"
    with open(path, "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for n, s, e in rows:
            f.write(f"{n},{s},{e}\n")
    table = bench.summarize_graph_trace(str(path), steps).splitlines()
    body = [ln.split("|")[1:-1] for ln in table[2:]]
    assert len(body) == 8
    for cells in body:
        name, mode = cells[0].strip(), cells[1].strip()
        vals = [float(c) for c in cells[2:]]
        wi = bench.GRAPH_PASS_WORKLOADS.index(name)
        assert vals[:3] == [10.0 * (wi + 1), 20.0, 30.0]
        if mode == "graph":
            assert vals[3] == 0.0 and vals[4] == 8.0
            assert vals[5] == 10.0 * (wi + 1) + 50.0
        else:
            assert vals[3] == 2.0 and vals[4] == 0.0
            assert vals[5] == 10.0 * (wi + 1) + 52.0


def test_summarize_stalls(tmp_path):
    """The wave-cycle table of a --counter-pass: synthetic counter files laid out as its
    library dispatches (two rounds), each counter set to a value that makes every share known;
    a missing dispatch is an error."""
    seq = bench.counter_sequence(workloads)

    def write(path, names, values, drop_last=False):
        rows = seq[:-1] if drop_last else seq
        with open(path, "w") as f:
            f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
            f.write("0,__amd_rocclr_copyBuffer,SQ_WAVE_CYCLES,1\n")  # not a library kernel
            for i, (_, k) in enumerate(rows):
                for n in names:
                    f.write(f"{i + 1},void fa::(anonymous namespace)::{k}(fa::Args),{n},{values[n](i)}\n")

    a_vals = {"SQ_WAVE_CYCLES": lambda i: 1000.0, "SQ_WAIT_ANY": lambda i: 200.0,
              "SQ_WAIT_INST_ANY": lambda i: 450.0, "SQ_WAIT_INST_LDS": lambda i: 90.0,
              "SQ_ACTIVE_INST_ANY": lambda i: 350.0, "SQ_VALU_MFMA_COEXEC_CYCLES": lambda i: 60.0,
              "SQ_BUSY_CU_CYCLES": lambda i: 100.0, "SQ_VALU_MFMA_BUSY_CYCLES": lambda i: 240.0 + i}
    b_vals = {"SQ_WAVE_CYCLES": lambda i: 2000.0, "SQ_ACTIVE_INST_LDS": lambda i: 160.0,
              "SQ_ACTIVE_INST_VALU": lambda i: 400.0, "SQ_ACTIVE_INST_SCA": lambda i: 120.0,
              "SQ_ACTIVE_INST_MISC": lambda i: 1.0, "SQ_INST_LEVEL_LDS": lambda i: 1.0,
              "SQ_INSTS_LDS": lambda i: 1.0, "SQ_ACTIVE_INST_VMEM": lambda i: 1.0}
    a, b = tmp_path / "a.csv", tmp_path / "b.csv"
    write(a, bench.STALL_COUNTERS_A, a_vals)
    write(b, bench.STALL_COUNTERS_B, b_vals)
    table = bench.summarize_stalls(str(a), str(b)).splitlines()
    body = [[c.strip() for c in ln.split("|")[1:-1]] for ln in table[2:]]
    half = len(seq) // 2
    assert len(body) == len(seq) - half
    for j, cells in enumerate(body):
        i = half + j
        assert (cells[0], cells[1]) == seq[i]
        assert cells[2] == f"{100 * (240.0 + i) / 400.0:.1f} %"  # MFMA busy over 4 SIMDs
        assert cells[3:8] == ["35.0 %", "20.0 %", "45.0 %", "9.0 %", f"{100 * 60.0 / (240.0 + i):.1f} %"]
        assert cells[8:] == ["20.0 %", "8.0 %", "6.0 %"]
    write(b, bench.STALL_COUNTERS_B, b_vals, drop_last=True)
    with pytest.raises(RuntimeError, match="library dispatches"):
        bench.summarize_stalls(str(a), str(b))


def test_phase_figures_use_the_dtype_peak():
    # 157.3 GFLOP in 1 ms is the whole fp32 peak and 6.3 % of the bf16 one
    f32 = bench.phase_figures(1.0, 157.3e9, 8e9, bench.PEAK_F32_TFLOPS)
    bf16 = bench.phase_figures(1.0, 157.3e9, 8e9)
    assert f32["tflops"] == 157.3 and f32["frac_of_peak"] == 1.0
    assert bf16["frac_of_peak"] == round(157.3 / bench.PEAK_BF16_TFLOPS, 4)
    assert f32["hbm_frac"] == 1.0
