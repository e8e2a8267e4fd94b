"""Benchmark of the causal kernelized linear-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

Workload: causal normalised linear attention, phi(x) = relu(x) + 1, bf16
inputs with fp32 state and accumulation, B=8, H=8, n=2048, d=64, chunk 64;
Q, K, V i.i.d. N(0,1)/sqrt(d) from the seeded generator in la_inputs.  One
step is one la_causal_forward call over the whole batch (every kernel of the
path).  Inputs are resident in HBM before timing starts; 10 copies of the
input/output set rotate so that the 640 MiB footprint is not served from the
256 MiB last-level (MALL) cache.

Prints one JSON line:
  value     tokens*heads per second (B * H * n per step / step time);
  roofline  algorithmic HBM bytes of one call (Q, K, V read once, out written
            once: 4 * B * H * n * d * 2 bytes) / the call's average duration,
            measured with HIP events on the stream the kernels run on,
            against the 8 TB/s HBM3E peak;
  cpu_baseline  the fp64 oracle (test infrastructure, untuned) timed on this
            host's cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

B, H, N, D, CHUNK = 8, 8, 2048, 64, 64
HBM_PEAK_GBS = 8000.0
ROTATE = 10


def algorithmic_bytes(B, Hq, Hkv, n, d, elem=2):
    return (2 * B * Hq * n * d + 2 * B * Hkv * n * d) * elem


def cpu_baseline(q, k, v, budget_s=12.0):
    """Time the oracle on slices of the workload's batch until about budget_s
    seconds of CPU work have been spent.  Each slice holds enough batch
    elements for every host thread to own one (batch, head) pair."""
    import oracle

    threads = oracle.num_threads()
    bs = max(1, min(B, -(-threads // H)))
    t0 = time.perf_counter()
    oracle.causal(q[:bs], k[:bs], v[:bs])
    one = time.perf_counter() - t0
    reps = max(1, int(budget_s / max(one, 1e-3)))
    t0 = time.perf_counter()
    for r in range(reps):
        b = (r * bs) % B
        oracle.causal(q[b:b + bs], k[b:b + bs], v[b:b + bs])
    el = time.perf_counter() - t0
    return {
        "value": reps * bs * H * N / el,
        "unit": "tokens*heads/s",
        "cores": min(threads, bs * H),
        "kind": "oracle",
        "sample": f"{reps} calls on {bs}-element slices of the workload's batch (H={H} n={N} d={D}, "
                  f"causal, fp64 oracle on the bf16 inputs), {el:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the benchmark, run plain device-to-device copies of 64 MiB "
                         "(the reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(batch x head sharding needs no communication; run one process per GPU).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import la_inputs as li
    import linear_attention_phi_amd as la

    la.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        # 10 rotating 64 MiB sources (640 MiB > the 256 MiB MALL); each copy
        # moves 64 MiB in and 64 MiB out
        src = [torch.full((64 << 20,), i, dtype=torch.uint8, device=dev) for i in range(ROTATE)]
        dst = torch.empty_like(src[0])
        for i in range(args.warmup + args.steps):
            dst.copy_(src[i % ROTATE])
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": 64 << 20, "copies": args.warmup + args.steps}))
        return
    q, k, v, _ = li.qkv(B, H, H, N, D, li.BF16, seed=0, scaled=True)
    qd, kd, vd = (li.to_torch(x).to(dev) for x in (q, k, v))
    sets = [(qd.clone(), kd.clone(), vd.clone(), torch.empty_like(qd)) for _ in range(ROTATE)]
    need = la.la_workspace_bytes(la.LA_OP_CAUSAL, B, H, H, N, D, la.LA_BF16, CHUNK)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)

    def step(i):
        qq, kk, vv, oo = sets[i % ROTATE]
        la.la_causal_forward(qq, kk, vv, chunk=CHUNK, out=oo, ws=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # the K steps run back to back, bracketed by two events on the stream the
    # kernels are launched on (an event between calls would add its own gap)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    nbytes = algorithmic_bytes(B, H, H, N, D)
    achieved = nbytes / (ms * 1e-3) / 1e9
    line = {
        "metric": "linear-attn fwd tokens*heads/s + HBM GB/s (% peak), causal bf16 n=2048 d=64",
        "value": B * H * N / (ms * 1e-3),
        "unit": "tokens*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal normalised linear attention, phi=relu+1, bf16 in, fp32 state",
                   "B": B, "H": H, "n": N, "d": D, "chunk": CHUNK,
                   "global_batch": B, "seq_len": N},
        "roofline": {
            "bound": "hbm",
            "kernel": "la_causal_forward (whole call)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": None,
            "algorithmic_bytes_per_call": nbytes,
            "call_us_mean": ms * 1e3,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(q, k, v)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
