"""Benchmark of the kernelized linear-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--workload NAME]

The default workload is causal normalised linear attention, phi(x) = relu(x)
+ 1, bf16 inputs with fp32 state and accumulation, B=8, H=8, n=2048, d=64,
chunk 64; Q, K, V i.i.d. N(0,1)/sqrt(d) from the seeded generator in
la_inputs.  One step is one la_causal_forward call over the whole batch (every
kernel of the path).  The other workloads (--workload) measure the other
forms of the method the same way: non-causal (B2 H8 n4096 d64, fp32 / bf16),
the unnormalised prefix-mask form (B4 H8 n8192 d64 fp32, causal and random
masks), the long-context grouped-query causal pass (B1 Hq32 Hkv8 n65536 d128
bf16) and the recurrent decode step (B128 Hq32 Hkv8 d128, state prefilled
from 4096 tokens; one step = one la_decode_step call).

Inputs are resident in HBM before timing starts; where one input/output set
is smaller than 640 MiB, several copies rotate so that the footprint is not
served from the 256 MiB last-level (MALL) cache.  W untimed steps (default
1000, a few milliseconds to under a second of work) bring the GPU to steady
clocks; then K steps run back to back between two HIP events recorded on the
stream the kernels are launched on.

Prints one JSON line per workload:
  value     tokens*heads per second (B * Hq * n per call; B * Hq per decode step);
  roofline  algorithmic HBM bytes of one call (inputs read once, outputs
            written once; for decode the state read and written once) / the
            call's average duration, against the 8 TB/s HBM3E peak, plus the
            MFMA fraction of the algorithmic flops at the input dtype's peak;
  cpu_baseline  the fp64 oracle (test infrastructure, untuned) timed on this
            host's cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F32_PEAK_TFS = 157.3
MFMA_BF16_PEAK_TFS = 2500.0
FOOTPRINT = 640 << 20  # rotate input/output sets up to this many bytes

WORKLOADS = {
    "causal": dict(form="causal", B=8, Hq=8, Hkv=8, n=2048, d=64, dt="bf16", chunk=64, scaled=True, steps=200),
    "forward_f32": dict(form="forward", B=2, Hq=8, Hkv=8, n=4096, d=64, dt="f32", scaled=False, steps=200),
    "forward_bf16": dict(form="forward", B=2, Hq=8, Hkv=8, n=4096, d=64, dt="bf16", scaled=False, steps=200),
    "prefix_causal": dict(form="prefix", B=4, Hq=8, Hkv=8, n=8192, d=64, dt="f32", chunk=64, scaled=True,
                          mask="causal", steps=50),
    "prefix_random": dict(form="prefix", B=4, Hq=8, Hkv=8, n=8192, d=64, dt="f32", chunk=64, scaled=True,
                          mask="random", steps=50),
    "prefix_random_batched": dict(form="prefix", B=4, Hq=8, Hkv=8, n=8192, d=64, dt="f32", chunk=64, scaled=True,
                                  mask="random", batched=True, steps=50),
    "gqa_causal": dict(form="causal", B=1, Hq=32, Hkv=8, n=65536, d=128, dt="bf16", chunk=0, scaled=True, steps=20),
    "decode": dict(form="decode", B=128, Hq=32, Hkv=8, d=128, dt="bf16", prefix=4096, scaled=True, steps=256),
    # the ELU + 1 feature map (la_*_phi), on the general kernels
    "causal_elu": dict(form="causal", B=8, Hq=8, Hkv=8, n=2048, d=64, dt="bf16", chunk=64, scaled=True, steps=200,
                       phi="elu1"),
    "forward_elu": dict(form="forward", B=2, Hq=8, Hkv=8, n=4096, d=64, dt="bf16", scaled=False, steps=200,
                        phi="elu1"),
    "gqa_elu": dict(form="causal", B=1, Hq=32, Hkv=8, n=65536, d=128, dt="bf16", chunk=0, scaled=True, steps=20,
                    phi="elu1"),
    # the next rows: sliding window, strided and packed sequences, a feature
    # map of the caller's choice, the backward
    "window": dict(form="window", B=8, Hq=8, Hkv=8, n=2048, d=64, dt="bf16", window=512, scaled=True, steps=200),
    "causal_bnhd": dict(form="strided", B=8, Hq=8, Hkv=8, n=2048, d=64, dt="bf16", scaled=True, steps=200),
    "varlen": dict(form="varlen", B=16, Hq=8, Hkv=8, n=2048, d=64, dt="bf16", scaled=True, steps=200),
    "causal_features": dict(form="causal", B=8, Hq=8, Hkv=8, n=2048, d=64, dt="bf16", chunk=64, scaled=True,
                            steps=200, phi="features"),
    "backward": dict(form="backward", B=8, Hq=8, Hkv=8, n=2048, d=64, dt="bf16", scaled=True, steps=50),
    # grouped query heads at d = 64 (four per key/value head) on the single-launch kernel
    "gqa_d64": dict(form="causal", B=4, Hq=16, Hkv=4, n=2048, d=64, dt="bf16", chunk=64, scaled=True, steps=200),
    # d = 128 with one and with eight query heads per key/value head
    "mha_d128": dict(form="causal", B=8, Hq=8, Hkv=8, n=2048, d=128, dt="bf16", chunk=0, scaled=True, steps=100),
    "gqa_r8_d128": dict(form="causal", B=2, Hq=32, Hkv=4, n=8192, d=128, dt="bf16", chunk=0, scaled=True,
                        steps=100),
}

DESCRIPTIONS = {
    "causal": "causal normalised linear attention, phi=relu+1, bf16 in, fp32 state",
    "forward_f32": "non-causal normalised linear attention, phi=relu+1, fp32",
    "forward_bf16": "non-causal normalised linear attention, phi=relu+1, bf16 in, fp32 accumulation",
    "prefix_causal": "unnormalised QK^T V with prefix mask m=arange(n), fp32",
    "prefix_random": "unnormalised QK^T V with prefix mask m_i ~ U{0..n-1}, fp32",
    "prefix_random_batched": "unnormalised QK^T V with a prefix mask per batch, m[b, i] ~ U{0..n-1}, fp32",
    "gqa_causal": "long-context GQA causal normalised linear attention, bf16 in, fp32 state",
    "decode": "recurrent decode step, fp32 state prefilled from a 4096-token prefix, bf16 q/k/v",
    "causal_elu": "causal normalised linear attention, phi=ELU+1, bf16 in, fp32 state",
    "forward_elu": "non-causal normalised linear attention, phi=ELU+1, bf16 in, fp32 accumulation",
    "gqa_elu": "long-context GQA causal normalised linear attention, phi=ELU+1, bf16 in, fp32 state",
    "window": "sliding-window (512 keys) causal normalised linear attention, phi=relu+1, bf16 in, fp32 state",
    "causal_bnhd": "causal normalised linear attention on [batch, seq, heads, d] rows (strided), bf16",
    "varlen": "causal normalised linear attention on 16 packed sequences of 128..2048 tokens (cu_seqlens), bf16",
    "causal_features": "causal normalised linear attention on caller-applied features (softplus), bf16",
    "backward": "gradients dQ, dK, dV of the causal form (phi=relu+1), bf16 in, fp32 products",
    "gqa_d64": "causal normalised linear attention, four query heads per key/value head, d 64, bf16",
    "mha_d128": "causal normalised linear attention, one query head per key/value head, d 128, bf16",
    "gqa_r8_d128": "causal normalised linear attention, eight query heads per key/value head, d 128, bf16",
}

# The packed-sequence workload's lengths: 16 sequences drawn uniformly from
# 128 .. 2048 tokens (seed 0); the pages give no length mix.
VARLEN_SEED = 0


def varlen_lengths(w):
    import numpy as np

    return np.random.default_rng(VARLEN_SEED).integers(128, w["n"] + 1, size=w["B"])


def elem_bytes(dt):
    return 4 if dt == "f32" else 2


def algorithmic_bytes(w):
    """Bytes the method must move per call: inputs read once, outputs written once."""
    e = elem_bytes(w["dt"])
    if w["form"] == "varlen":
        T = int(varlen_lengths(w).sum())
        return (2 * w["Hq"] + 2 * w["Hkv"]) * T * w["d"] * e + 8 * (w["B"] + 1)
    if w["form"] == "backward":  # q, k, v, dO read; dq, dk, dv written
        B, Hq, Hkv, n, d = w["B"], w["Hq"], w["Hkv"], w["n"], w["d"]
        return (3 * B * Hq * n * d + 4 * B * Hkv * n * d) * e
    if w["form"] == "decode":
        B, Hq, Hkv, d = w["B"], w["Hq"], w["Hkv"], w["d"]
        return 2 * B * Hkv * (d * d + d) * 4 + B * (2 * Hq + 2 * Hkv) * d * e
    B, Hq, Hkv, n, d = w["B"], w["Hq"], w["Hkv"], w["n"], w["d"]
    extra = 8 * n * (w["B"] if w.get("batched") else 1) if w["form"] == "prefix" else 0
    return (2 * B * Hq * n * d + 2 * B * Hkv * n * d) * e + extra


def algorithmic_flops(w):
    """Multiply-add work of the chunked method at chunk C (2 flops per MAC)."""
    if w["form"] == "decode":
        B, Hq, Hkv, d = w["B"], w["Hq"], w["Hkv"], w["d"]
        return 2 * (B * Hkv * d * d + B * Hq * d * d)
    B, Hq, Hkv, n, d = w["B"], w["Hq"], w["Hkv"], w["n"], w["d"]
    if w["form"] == "forward":
        return 2 * (B * Hkv * n * d * d + B * Hq * n * d * d)
    if w["form"] == "backward":
        # per token and head, at chunk C = 32 (the backward's fp32 tiles): six
        # d x d state products (phi(q) S, S g, U v, U^T phi(k), dS, dU) and six
        # C-long intra-chunk ones (P, P V, A, A phi(K), A^T phi(Q), P^T G)
        return 2 * B * Hq * n * 6 * (d * d + 32 * d)
    if w["form"] == "varlen":
        n = int(varlen_lengths(w).sum()) // B  # mean length: the products scale with the tokens
    C = w.get("chunk") or 64
    # state build per KV head; per query head phi(Q) S_prev, the masked C x C
    # score block and its product with V
    return 2 * (B * Hkv * n * d * d + B * Hq * (n * d * d + 2 * n * C * d))


# Counter-based HBM traffic of the workloads whose call is one launch: taken
# with rocprofv3 (FETCH_SIZE and WRITE_SIZE passes, scaled by the same
# counters' readings for a plain 64 MiB device copy) and recorded under
# profiles/ together with a hash of the kernel's sources; reported only while
# the sources still hash the same (null once the kernel has changed).
_FUSED_SRC = ["la_fused.hip", "la_bf16.h", "la_ctl.h", "la_device.h", "la_internal.h"]
COUNTERS = {
    "causal": ("k_causal_fused_causal_bf16_B8H8n2048d64_counters.md", _FUSED_SRC),
    "causal_bnhd": ("k_causal_fused_causal_bnhd_bf16_B8n2048H8d64_counters.md", _FUSED_SRC),
    "varlen": ("k_causal_fused_varlen_bf16_16seqs_128to2048_H8d64_counters.md", _FUSED_SRC),
    "gqa_d64": ("k_causal_fused_gqa_d64_bf16_B4Hq16Hkv4n2048d64_counters.md", _FUSED_SRC),
    "window": ("k_window_fused_window_bf16_B8H8n2048d64_w512_counters.md",
               ["la_window_fused.hip", "la_bf16.h", "la_ctl.h", "la_device.h", "la_internal.h"]),
    "forward_bf16": ("k_fwd_one_forward_bf16_B2H8n4096d64_counters.md",
                     ["la_forward_bf16.hip", "la_bf16.h", "la_ctl.h", "la_device.h", "la_internal.h"]),
    "decode": ("k_decode128_decode_B128Hq32Hkv8d128_counters.md",
               ["la_kernels.hip", "la_bf16.h", "la_ctl.h", "la_device.h", "la_internal.h"]),
}
SINGLE_LAUNCH = {"causal": "k_causal_fused", "forward_bf16": "k_fwd_one", "decode": "k_decode128",
                 "causal_elu": "k_causal_fused", "forward_elu": "k_fwd_one", "causal_features": "k_causal_fused",
                 "causal_bnhd": "k_causal_fused", "varlen": "k_causal_fused", "window": "k_window_fused",
                 "gqa_d64": "k_causal_fused"}


def kernel_source_hash(files):
    import hashlib

    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "linear_attention_phi_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_traffic(name):
    """HBM bytes per launch of workload name from the recorded counters, or None."""
    if name not in COUNTERS:
        return None
    fname, sources = COUNTERS[name]
    try:
        with open(os.path.join(ROOT, "profiles", fname)) as fh:
            text = fh.read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        line = line.strip().strip("`").strip()
        for key in ("source_sha256:", "hbm_bytes_per_launch:"):
            if line.startswith(key):
                vals[key[:-1]] = line[len(key):].strip()
    if vals.get("source_sha256") != kernel_source_hash(sources) or "hbm_bytes_per_launch" not in vals:
        return None
    return float(vals["hbm_bytes_per_launch"])


def tokens_heads(w):
    if w["form"] == "decode":
        return w["B"] * w["Hq"]
    if w["form"] == "varlen":
        return int(varlen_lengths(w).sum()) * w["Hq"]
    return w["B"] * w["Hq"] * w["n"]


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, q, k, v, m=None, S=None, z=None, budget_s=12.0):
    """Time the untuned oracle on a bounded sample of the workload: slices of
    the batch (causal, non-causal, prefix), the first tokens of every head
    (long context) or a few steps on the whole batch (decode), repeated until
    about budget_s seconds of CPU work have been spent."""
    import numpy as np

    import la_inputs as li
    import oracle

    threads = oracle.num_threads()
    form = w["form"]
    phi = w.get("phi", "relu1")
    if form == "decode":
        B, Hq, Hkv, d = w["B"], w["Hq"], w["Hkv"], w["d"]
        rng = np.random.default_rng(1)
        toks = [tuple(li.gaussian(rng, (B, h, d), 1.0 / math.sqrt(d), li.BF16) for h in (Hq, Hkv, Hkv))
                for _ in range(4)]
        Sd = S.astype(np.float64)
        zd = z.astype(np.float64)
        steps, el = 0, 0.0
        while el < budget_s:
            qs, ks, vs = toks[steps % 4]
            t0 = time.perf_counter()
            oracle.decode_step(qs, ks, vs, Sd, zd)
            el += time.perf_counter() - t0
            steps += 1
        return {"value": steps * B * Hq / el, "unit": "tokens*heads/s", "cores": min(threads, B * Hkv),
                "kind": "oracle",
                "sample": f"{steps} decode steps on the whole batch (B={B} Hq={Hq} Hkv={Hkv} d={d}), "
                          f"fp64 oracle, {el:.1f} s", "cpu": cpu_model()}
    B, Hq, Hkv, n, d = w["B"], w["Hq"], w["Hkv"], w["n"], w["d"]
    if form == "causal" and B * Hkv < threads:
        # long context: the first n_s tokens of every head (the causal output of
        # a prefix does not depend on later tokens)
        n_s = 4096
        qs, ks, vs = (np.ascontiguousarray(x[:, :, :n_s]) for x in (q, k, v))

        def call():
            oracle.causal(qs, ks, vs, phi=phi)

        per = B * Hq * n_s
        what = f"the first {n_s} tokens of all {Hq} query heads (causal, d={d})"
        cores = min(threads, B * Hkv)
    elif form == "backward":
        bs = 1
        do = li.gaussian(np.random.default_rng(5), q.shape, None, li.BF16 if q.dtype == np.uint16 else li.F32)

        def call():
            oracle.causal_backward(q[:1], k[:1], v[:1], do[:1])

        per = Hq * n
        what = f"1-element slices of the batch (Hq={Hq} n={n} d={d}, pairwise O(n^2) gradients)"
        cores = min(threads, Hkv)
    else:
        bs = max(1, min(B, -(-threads // Hkv)))
        fn = {"causal": lambda a, b_, c: oracle.causal(a, b_, c, phi=phi),
              "strided": lambda a, b_, c: oracle.causal(a, b_, c, phi=phi),
              "varlen": lambda a, b_, c: oracle.causal(a, b_, c, phi=phi),
              "window": lambda a, b_, c: oracle.window(a, b_, c, w["window"], phi=phi),
              "forward": lambda a, b_, c: oracle.forward(a, b_, c, phi=phi),
              "prefix": None}[form]
        state = {"r": 0}

        def call():
            b0 = (state["r"] * bs) % B
            state["r"] += 1
            if form == "prefix":  # the batches' own mask rows when there is one per batch
                oracle.prefix_mask(q[b0:b0 + bs], k[b0:b0 + bs], v[b0:b0 + bs], m if m.ndim == 1 else m[b0:b0 + bs])
            else:
                fn(q[b0:b0 + bs], k[b0:b0 + bs], v[b0:b0 + bs])

        per = bs * Hq * n
        what = f"{bs}-element slices of the batch (Hq={Hq} n={n} d={d})"
        cores = min(threads, bs * Hkv)
    call()  # first-call costs (allocation, thread start) outside the timing
    reps, el = 0, 0.0
    t0 = time.perf_counter()
    while el < budget_s:
        call()
        reps += 1
        el = time.perf_counter() - t0
    return {"value": reps * per / el, "unit": "tokens*heads/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} oracle calls on {what}, fp64, {el:.1f} s", "cpu": cpu_model()}


def run(name, args):
    import numpy as np
    import torch

    import la_inputs as li
    import linear_attention_phi_amd as la

    w = dict(WORKLOADS[name])
    steps = args.steps if args.steps is not None else w["steps"]
    warmup = args.warmup
    dev = torch.device("cuda", 0)
    dtc = li.BF16 if w["dt"] == "bf16" else li.F32
    ladt = la.LA_BF16 if w["dt"] == "bf16" else la.LA_F32
    form = w["form"]
    m = S0 = z0 = q = k = v = None
    if form == "decode":
        B, Hq, Hkv, d, P = w["B"], w["Hq"], w["Hkv"], w["d"], w["prefix"]
        # state prefilled by a state-only causal pass over a 4096-token prefix
        # (drawn one sequence at a time, K then V, to bound host memory)
        rng = np.random.default_rng(0)
        kp = torch.empty((B, Hkv, P, d), dtype=torch.bfloat16 if dtc == li.BF16 else torch.float32, device=dev)
        vp = torch.empty_like(kp)
        for b in range(B):
            kp[b] = li.to_torch(li.gaussian(rng, (Hkv, P, d), 1.0 / math.sqrt(d), dtc)).to(dev)
            vp[b] = li.to_torch(li.gaussian(rng, (Hkv, P, d), 1.0 / math.sqrt(d), dtc)).to(dev)
        S0, z0 = la.la_causal_forward(None, kp, vp, chunk=0, Hq=Hq)
        del kp, vp
        state_bytes = (S0.numel() + z0.numel()) * 4
        rot = max(1, min(8, -(-FOOTPRINT // state_bytes)))
        states = [(S0.clone(), z0.clone()) for _ in range(rot)]
        T = 8  # distinct per-step token sets (their values do not change the work)
        toks = []
        for _ in range(T):
            qs, ks, vs = (li.to_torch(li.gaussian(rng, (B, h, d), 1.0 / math.sqrt(d), dtc)).to(dev)
                          for h in (Hq, Hkv, Hkv))
            toks.append((qs, ks, vs, torch.empty_like(qs)))

        def step(i):
            S, z = states[i % rot]
            qs, ks, vs, o = toks[i % T]
            la.la_decode_step(qs, ks, vs, S, z, out=o)
    elif form in ("window", "strided", "varlen", "backward"):
        B, Hq, Hkv, n, d = w["B"], w["Hq"], w["Hkv"], w["n"], w["d"]
        tdt = torch.bfloat16 if dtc == li.BF16 else torch.float32
        if form == "varlen":
            lens = varlen_lengths(w)
            cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
            T = int(cu[-1])
            q, k, v, rng = li.qkv(1, Hq, Hkv, T, d, dtc, seed=0, scaled=w["scaled"])
            cud = torch.from_numpy(cu).to(dev)
            # packed [T, H, d] rows
            pk = lambda x: li.to_torch(np.ascontiguousarray(x[0].transpose(1, 0, 2))).to(dev)
            first = (pk(q), pk(k), pk(v))
        else:
            q, k, v, rng = li.qkv(B, Hq, Hkv, n, d, dtc, seed=0, scaled=w["scaled"])
            if form == "strided":  # [B, n, H, d] buffers, viewed as [B, H, n, d]
                bn = lambda x: li.to_torch(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).to(dev).transpose(1, 2)
                first = (bn(q), bn(k), bn(v))
            else:
                first = tuple(li.to_torch(x).to(dev) for x in (q, k, v))
        set_bytes = 2 * (first[0].numel() + first[1].numel()) * first[0].element_size()
        rot = max(1, min(16, -(-FOOTPRINT // set_bytes)))
        sets = [first] + [tuple(x.clone() for x in first) for _ in range(rot - 1)]
        if form == "strided":  # clone() of a transposed view keeps its strides
            assert all(x.stride() == first[0].stride() for x in sets[-1][:1])
        outs = [torch.empty_like(s_[0]) for s_ in sets]
        if form == "backward":
            dos = [li.to_torch(li.gaussian(rng, (B, Hq, n, d), None, dtc)).to(dev) for _ in range(rot)]
            need = la.la_workspace_bytes(la.LA_OP_CAUSAL_BACKWARD, B, Hq, Hkv, n, d, ladt, 0)
        else:
            need = la.la_workspace_bytes(la.LA_OP_SEQS, B, Hq, Hkv, n, d, ladt, 0)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        phi = w.get("phi", "relu1")

        def step(i):
            qq, kk, vv = sets[i % rot]
            if form == "window":
                la.la_window_forward(qq, kk, vv, w["window"], out=outs[i % rot], phi=phi)
            elif form == "strided":
                la.la_causal_forward_strided(qq, kk, vv, out=outs[i % rot], ws=ws, phi=phi)
            elif form == "varlen":
                la.la_causal_forward_strided(qq, kk, vv, cu_seqlens=cud, max_len=n, out=outs[i % rot], ws=ws, phi=phi)
            else:
                la.la_causal_backward(qq, kk, vv, dos[i % rot], ws=ws, phi=phi)
    else:
        B, Hq, Hkv, n, d = w["B"], w["Hq"], w["Hkv"], w["n"], w["d"]
        q, k, v, rng = li.qkv(B, Hq, Hkv, n, d, dtc, seed=0, scaled=w["scaled"])
        if w.get("phi") == "features":  # the caller's map (softplus) applied beforehand, in fp32
            sp = lambda x: li.as_dtype(np.log1p(np.exp(li.to_f32(x))).astype(np.float32), dtc)
            q, k = sp(q), sp(k)
        md = None
        if form == "prefix":
            if w.get("batched"):
                m = np.stack([li.mask(n, w["mask"], rng=rng) for _ in range(B)])
            else:
                m = li.mask(n, w["mask"], rng=rng)
            md = li.to_torch(m).to(dev)
        qd, kd, vd = (li.to_torch(x).to(dev) for x in (q, k, v))
        set_bytes = 2 * (qd.numel() + kd.numel()) * qd.element_size()
        rot = max(1, min(16, -(-FOOTPRINT // set_bytes)))
        sets = [(qd, kd, vd, torch.empty_like(qd))] + [
            (qd.clone(), kd.clone(), vd.clone(), torch.empty_like(qd)) for _ in range(rot - 1)]
        op = {"causal": la.LA_OP_CAUSAL, "forward": la.LA_OP_FORWARD,
              "prefix": la.LA_OP_PREFIX_MASK_BATCHED if w.get("batched") else la.LA_OP_PREFIX_MASK}[form]
        chunk = w.get("chunk", 0)
        need = la.la_workspace_bytes(op, B, Hq, Hkv, n, d, ladt, chunk)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)

        phi = w.get("phi", "relu1")

        def step(i):
            qq, kk, vv, oo = sets[i % rot]
            if form == "causal":
                la.la_causal_forward(qq, kk, vv, chunk=chunk, out=oo, ws=ws, phi=phi)
            elif form == "forward":
                la.la_forward(qq, kk, vv, out=oo, ws=ws, phi=phi)
            else:
                la.la_prefix_mask_forward(qq, kk, vv, md, chunk=chunk, out=oo, ws=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # the K steps run back to back, bracketed by two events on the stream the
    # kernels are launched on (an event between calls would add its own gap)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # a spin kernel ahead of the start event keeps the GPU busy while the host
    # enqueues the first calls, so that no host launch gap falls inside the
    # bracket (the K calls then run back to back on the device)
    torch.cuda._sleep(2_000_000)
    e0.record(stream)
    for i in range(steps):
        step(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps

    # the per-call distribution, from a separate run with an event pair around
    # every call (the events add their own gaps, so it is not the headline)
    ndist = min(steps, 100)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ndist)]
    torch.cuda._sleep(2_000_000)
    for i, (ea, eb) in enumerate(evs):
        ea.record(stream)
        step(warmup + steps + i)
        eb.record(stream)
    torch.cuda.synchronize()
    per_call = sorted(ea.elapsed_time(eb) * 1e3 for ea, eb in evs)

    def pct(p):
        return per_call[min(len(per_call) - 1, int(round(p * (len(per_call) - 1))))]

    dist = {"median": pct(0.5), "p10": pct(0.1), "p90": pct(0.9), "calls": ndist, "unit": "us"}

    nbytes = algorithmic_bytes(w)
    flops = algorithmic_flops(w)
    achieved = nbytes / (ms * 1e-3) / 1e9
    single = SINGLE_LAUNCH.get(name)
    roof = {
        "bound": "hbm",
        "kernel": f"{single} (the call's one launch)" if single else f"la_{form} (whole call)",
        "achieved": achieved,
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": achieved / HBM_PEAK_GBS,
        "traffic": counter_traffic(name),
        "algorithmic_bytes_per_call": nbytes,
        "algorithmic_flops_per_call": flops,
        "call_us_mean": ms * 1e3,
        "rotating_sets": rot,
    }
    tfs = flops / (ms * 1e-3) / 1e12
    # the backward's products are fp32 MFMA for either input type
    mpeak = MFMA_F32_PEAK_TFS if w["dt"] == "f32" or form == "backward" else MFMA_BF16_PEAK_TFS
    roof["mfma"] = {"achieved": tfs, "peak": mpeak, "unit": "TFLOP/s", "frac": tfs / mpeak}
    if form != "decode" and flops / (mpeak * 1e12) > nbytes / (HBM_PEAK_GBS * 1e9):
        roof["note"] = "the MFMA time of the algorithmic flops exceeds their HBM time: compare both fractions"
    cfg = {"workload": DESCRIPTIONS[name], "name": name}
    cfg.update({kk: w[kk] for kk in ("B", "Hq", "Hkv", "n", "d", "chunk", "mask", "prefix", "phi", "batched",
                                     "window") if kk in w})
    if form == "varlen":
        cfg["lengths"] = [int(x) for x in varlen_lengths(w)]
    if form != "decode":
        cfg.update({"global_batch": w["B"], "seq_len": w["n"]})
    line = {
        "metric": "linear-attn fwd tokens*heads/s + HBM GB/s (% peak), causal bf16 n=2048 d=64"
                  if name == "causal" else f"linear-attn tokens*heads/s + HBM GB/s (% peak), {name}",
        "value": tokens_heads(w) / (ms * 1e-3),
        "unit": "tokens*heads/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dt"],
        "data": "synthetic",
        "config": cfg,
        "roofline": roof,
        "per_call_us": dist,
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        if form == "decode":
            line["cpu_baseline"] = cpu_baseline(w, None, None, None, S=S0.cpu().numpy(), z=z0.cpu().numpy())
        elif form == "varlen":
            line["cpu_baseline"] = None  # per-sequence oracle calls: see the causal workload
        else:
            line["cpu_baseline"] = cpu_baseline(w, q, k, v, m=m)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: per workload)")
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps first (the GPU reaches steady clocks only after some "
                         "milliseconds of work: after 10 the headline measured ~1 us slower per call)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--workload", default="causal", help="one of: " + ", ".join(WORKLOADS) + ", or all")
    ap.add_argument("--copy-calibration", nargs="?", const="vector", choices=["vector", "blit"], default=None,
                    help="instead of the benchmark, run plain device-to-device copies of 64 MiB "
                         "(the reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters): "
                         "'vector' (default) an elementwise copy, 'blit' the runtime's copy kernel")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(batch x head sharding needs no communication; run one process per GPU).",
              file=sys.stderr)
        sys.exit(2)
    names = list(WORKLOADS) if args.workload == "all" else [args.workload]
    for nm in names:
        if nm not in WORKLOADS:
            print(f"unknown workload {nm!r}; choose from {', '.join(WORKLOADS)} or all", file=sys.stderr)
            sys.exit(2)

    import torch

    import linear_attention_phi_amd as la

    la.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        # 10 rotating 64 MiB sources (640 MiB > the 256 MiB MALL); each copy
        # moves 64 MiB in and 64 MiB out.  "blit": the runtime's copy kernel;
        # "vector": an elementwise copy (x * 1) whose lanes load and store 16
        # contiguous bytes each over whole rows, the access pattern of the
        # kernels measured here (the counters' request-size accounting
        # depends on the pattern)
        src = [torch.full((16 << 20,), float(i), dtype=torch.float32, device=dev) for i in range(10)]
        dst = torch.empty_like(src[0])
        n = args.warmup + (args.steps or 200)
        for i in range(n):
            if args.copy_calibration == "blit":
                dst.copy_(src[i % 10])
            else:
                torch.mul(src[i % 10], 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": args.copy_calibration, "bytes_each_way": 64 << 20, "copies": n}))
        return
    for nm in names:
        run(nm, args)
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
