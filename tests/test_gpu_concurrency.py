"""Concurrent use of the library: calls from two host threads, each on its own stream,
give bitwise the results of the same calls made one after the other (the kernels are
deterministic, keep no state between calls, and each call runs on its caller's stream)."""
import threading

import pytest
import torch

from exact_tiled_attention_32_amd import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _run(fa, case):
    """Forward and backward of a case on the current stream (no device-wide sync)."""
    q, k, v, do = (case[n].to(DEV, non_blocking=False) for n in ("q", "k", "v", "do"))
    kv = None if case["kv_len"] is None else case["kv_len"].to(DEV)
    o, lse = fa.fa_fwd(q, k, v, case["scale"], case["causal"], kv)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, case["scale"], case["causal"], kv)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def test_two_threads_two_streams(gpu_lib):
    cases = [workloads.make_case(2, 3, 700, 64, seed=11, causal=True),
             workloads.make_case(2, 2, 513, 128, seed=12, kv_len=[513, 300])]
    ref = []
    for c in cases:
        r = _run(gpu_lib, c)
        torch.cuda.synchronize()
        ref.append({n: t.cpu() for n, t in r.items()})

    out, errors = [None, None], []
    start = threading.Barrier(2)

    def worker(i):
        try:
            s = torch.cuda.Stream(device=DEV)  # default priority
            with torch.cuda.stream(s):
                start.wait()
                runs = [_run(gpu_lib, cases[i]) for _ in range(4)]
            s.synchronize()
            out[i] = [{n: t.cpu() for n, t in r.items()} for r in runs]
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(2):
        for j, r in enumerate(out[i]):
            for n in ("o", "lse", "dq", "dk", "dv"):
                assert torch.equal(r[n], ref[i][n]), f"case {i} run {j}: {n} differs from the sequential call"
