"""GPU tests of the boundary's promises beyond the numbers themselves: calls
captured into a HIP graph and replayed with new inputs, calls on other
streams, bounded waits that give up (forced from the host, every kernel still
exits normally), prefix-mask values out of range, many repeated calls giving
the same bits, and full-size checks of every output row through closed forms.

Parity metric and tolerances as in test_parity_gpu.py (row-wise max-norm
relative error; 1e-4 fp32, 2e-2 bf16)."""
import os

import numpy as np
import pytest

import la_inputs as li
import oracle

pytestmark = pytest.mark.gpu

TOL = {li.F32: 1e-4, li.BF16: 2e-2}


def dev(x):
    return li.to_torch(x).cuda()


def host(t):
    return li.to_f32(li.from_torch(t)).astype(np.float64)


def rel_rows(g, o):
    return float((np.abs(g - o).max(axis=-1) / np.maximum(np.abs(o).max(axis=-1), 1e-30)).max())


def check(g, o, dtype, what):
    err = rel_rows(g, o)
    print(f"{what}: row-wise rel err {err:.3e} (tol {TOL[dtype]:.0e})", flush=True)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    assert err <= TOL[dtype], f"{what}: {err:.3e} > {TOL[dtype]}"
    return err


def new_ws(gpu, op, B, Hq, Hkv, n, d, dt, chunk=0):
    import torch
    return gpu.new_workspace(gpu.la_workspace_bytes(op, B, Hq, Hkv, n, d, dt, chunk), torch.device("cuda"))


# ------------------------------------------------------------- graph replay
@pytest.mark.parametrize("form", ["causal_B8_H8_n2048_d64", "forward_B2_H8_n4096_d64"])
def test_graph_capture_replays_with_new_inputs(gpu, form):
    """A call captured into a graph and replayed four times, new inputs
    copied into the static buffers before each replay, eager calls on the
    same workspace and host synchronisations between the replays: every
    replay matches the oracle and the eager call on the same inputs bit for
    bit.  The single-launch kernels order their workgroups by flags; the
    epoch they compare with comes from the workspace's control block, so a
    replay cannot mistake the previous replay's flags for its own."""
    import torch
    causal = form.startswith("causal")
    B, H, n, d = (8, 8, 2048, 64) if causal else (2, 8, 4096, 64)
    op = gpu.LA_OP_CAUSAL if causal else gpu.LA_OP_FORWARD
    ws = new_ws(gpu, op, B, H, H, n, d, gpu.LA_BF16, 64 if causal else 0)
    ws_eager = new_ws(gpu, op, B, H, H, n, d, gpu.LA_BF16, 64 if causal else 0)
    shape = (B, H, n, d)
    qs, ks, vs = (torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    out = torch.empty_like(qs)

    def call(q, k, v, o, w):
        if causal:
            return gpu.la_causal_forward(q, k, v, chunk=64, out=o, ws=w)
        return gpu.la_forward(q, k, v, out=o, ws=w)

    q0, k0, v0, _ = li.qkv(B, H, H, n, d, li.BF16, seed=40, scaled=causal)
    qs.copy_(dev(q0)); ks.copy_(dev(k0)); vs.copy_(dev(v0))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        call(qs, ks, vs, out, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(qs, ks, vs, out, ws)
    for rep in range(4):
        q, k, v, _ = li.qkv(B, H, H, n, d, li.BF16, seed=41 + rep, scaled=causal)
        qs.copy_(dev(q)); ks.copy_(dev(k)); vs.copy_(dev(v))
        graph.replay()
        torch.cuda.synchronize()
        got = li.from_torch(out)
        ref = oracle.causal(q, k, v) if causal else oracle.forward(q, k, v)
        check(li.to_f32(got).astype(np.float64), ref, li.BF16, f"{form} replay {rep}")
        eager = li.from_torch(call(qs, ks, vs, None, ws_eager))
        assert np.array_equal(got, eager), f"replay {rep} differs from the eager call"
        # an eager call on the captured workspace between replays advances its epoch too
        call(qs, ks, vs, torch.empty_like(qs), ws)
        assert gpu.la_workspace_status(ws) == 0
        assert gpu.la_workspace_status(ws_eager) == 0


@pytest.mark.parametrize("form", ["packed_sequences", "gqa_B4_Hq16_Hkv4_n1500"])
def test_graph_capture_single_launch_variants(gpu, form):
    """Graph replays of the single-launch causal kernel's other variants:
    packed sequences (lengths 0 .. 1800, so that many workgroups of the grid
    find their sequence ended and only count themselves in to the control
    block) and grouped query heads (the XCD-grouped dispatch order).  Four
    replays with new inputs copied into the static buffers, each against the
    oracle and the eager call on the same inputs, bit for bit."""
    import torch
    packed = form == "packed_sequences"
    if packed:
        lengths = [700, 0, 1800, 65, 1, 512, 1025]
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
        total, H, d = int(cu[-1]), 2, 64
        cud = torch.from_numpy(cu).cuda()
        ws = new_ws(gpu, gpu.LA_OP_SEQS, len(lengths), H, H, max(lengths), d, gpu.LA_BF16)
        ws_eager = new_ws(gpu, gpu.LA_OP_SEQS, len(lengths), H, H, max(lengths), d, gpu.LA_BF16)
        shapes = [(total, H, d)] * 3

        def call(q, k, v, o, w):
            return gpu.la_causal_forward_strided(q, k, v, cu_seqlens=cud, max_len=max(lengths), out=o, ws=w)

        def inputs(seed):
            q, k, v, _ = li.qkv(1, H, H, total, d, li.BF16, seed=seed, scaled=True)
            return [np.ascontiguousarray(x[0].transpose(1, 0, 2)) for x in (q, k, v)], (q, k, v)

        def reference(qkv):
            q, k, v = qkv
            outs = np.zeros((total, H, d))
            for s_, L in enumerate(lengths):
                if L:
                    a, b = int(cu[s_]), int(cu[s_ + 1])
                    sl = lambda x: np.ascontiguousarray(x[:, :, a:b])
                    outs[a:b] = oracle.causal(sl(q), sl(k), sl(v))[0].transpose(1, 0, 2)
            return outs
    else:
        B, Hq, Hkv, n, d = 4, 16, 4, 1500, 64
        ws = new_ws(gpu, gpu.LA_OP_CAUSAL, B, Hq, Hkv, n, d, gpu.LA_BF16, 64)
        ws_eager = new_ws(gpu, gpu.LA_OP_CAUSAL, B, Hq, Hkv, n, d, gpu.LA_BF16, 64)
        shapes = [(B, Hq, n, d), (B, Hkv, n, d), (B, Hkv, n, d)]

        def call(q, k, v, o, w):
            return gpu.la_causal_forward(q, k, v, chunk=64, out=o, ws=w)

        def inputs(seed):
            q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, li.BF16, seed=seed, scaled=True)
            return [q, k, v], (q, k, v)

        def reference(qkv):
            return oracle.causal(*qkv)
    qs, ks, vs = (torch.empty(sh, dtype=torch.bfloat16, device="cuda") for sh in shapes)
    out = torch.empty_like(qs)
    (q0, k0, v0), _ = inputs(50)
    qs.copy_(dev(q0)); ks.copy_(dev(k0)); vs.copy_(dev(v0))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        call(qs, ks, vs, out, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(qs, ks, vs, out, ws)
    for rep in range(4):
        (q, k, v), raw = inputs(51 + rep)
        qs.copy_(dev(q)); ks.copy_(dev(k)); vs.copy_(dev(v))
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = li.from_torch(out)
        check(li.to_f32(got).astype(np.float64), reference(raw), li.BF16, f"{form} replay {rep}")
        eager = li.from_torch(call(qs, ks, vs, torch.zeros_like(qs), ws_eager))
        assert np.array_equal(got, eager), f"replay {rep} differs from the eager call"
        call(qs, ks, vs, torch.empty_like(qs), ws)
        assert gpu.la_workspace_status(ws) == 0
        assert gpu.la_workspace_status(ws_eager) == 0


# ------------------------------------------------------------------ streams
def test_calls_on_other_streams(gpu):
    """Calls issued on two non-default streams at once, each with the
    binding's workspace for its stream, give the oracle's outputs."""
    import torch
    B, H, n, d = 2, 4, 3000, 64
    cases = [li.qkv(B, H, H, n, d, li.BF16, seed=50 + i, scaled=True)[:3] for i in range(2)]
    streams = [torch.cuda.Stream() for _ in cases]
    ins = [tuple(dev(x) for x in c) for c in cases]
    torch.cuda.synchronize()
    outs = []
    for s, (q, k, v) in zip(streams, ins):
        with torch.cuda.stream(s):
            outs.append((gpu.la_causal_forward(q, k, v, chunk=64), gpu.la_forward(q, k, v)))
    torch.cuda.synchronize()
    for i, ((q, k, v), (oc, of)) in enumerate(zip(cases, outs)):
        check(host(oc), oracle.causal(q, k, v), li.BF16, f"causal on stream {i}")
        check(host(of), oracle.forward(q, k, v), li.BF16, f"forward on stream {i}")


# ------------------------------------------------------ waits that give up
def test_bounded_wait_timeout_is_reported(gpu):
    """The host makes every flag wait give up (la_workspace_set_wait: 64
    polls, and an expected epoch no flag holds); the kernels still run to
    their end, and la_workspace_status reports LA_ERR_TIMEOUT once, then
    LA_OK.  With the defaults restored the same workspace gives the oracle's
    outputs again."""
    import torch
    B, H, n, d = 8, 8, 2048, 64  # four segments per head: segments 1..3 wait
    q, k, v, _ = li.qkv(B, H, H, n, d, li.BF16, seed=60, scaled=True)
    qd, kd, vd = dev(q), dev(k), dev(v)
    ws = new_ws(gpu, gpu.LA_OP_CAUSAL, B, H, H, n, d, gpu.LA_BF16, 64)
    gpu.la_workspace_set_wait(ws, 64, 1)
    gpu.la_causal_forward(qd, kd, vd, chunk=64, ws=ws)
    torch.cuda.synchronize()
    assert gpu.la_workspace_status(ws) == gpu.LA_ERR_TIMEOUT
    assert gpu.la_workspace_status(ws) == 0  # read and cleared
    wf = new_ws(gpu, gpu.LA_OP_FORWARD, 2, 8, 8, 4096, 64, gpu.LA_BF16)
    qf, kf, vf, _ = li.qkv(2, 8, 8, 4096, 64, li.BF16, seed=61)
    gpu.la_workspace_set_wait(wf, 64, 1)
    gpu.la_forward(dev(qf), dev(kf), dev(vf), ws=wf)
    assert gpu.la_workspace_status(wf) == gpu.LA_ERR_TIMEOUT
    gpu.la_workspace_set_wait(ws, 0, 0)
    out = gpu.la_causal_forward(qd, kd, vd, chunk=64, ws=ws)
    assert gpu.la_workspace_status(ws) == 0
    check(host(out), oracle.causal(q, k, v), li.BF16, "causal after the defaults are restored")
    gpu.la_workspace_set_wait(wf, 0, 0)
    g = gpu.la_forward(dev(qf), dev(kf), dev(vf), ws=wf)
    assert gpu.la_workspace_status(wf) == 0
    check(host(g), oracle.forward(qf, kf, vf), li.BF16, "forward after the defaults are restored")


def test_binding_raises_on_device_errors_in_debug_mode(gpu, monkeypatch):
    """LA_DEBUG_CHECKS=1: the binding synchronises after each call and raises
    the status the device recorded (here a forced wait timeout)."""
    B, H, n, d = 1, 2, 1000, 64
    q, k, v, _ = li.qkv(B, H, H, n, d, li.BF16, seed=62, scaled=True)
    ws = new_ws(gpu, gpu.LA_OP_CAUSAL, B, H, H, n, d, gpu.LA_BF16, 64)
    gpu.la_workspace_set_wait(ws, 16, 1)
    monkeypatch.setenv("LA_DEBUG_CHECKS", "1")
    with pytest.raises(gpu.LAError) as e:
        gpu.la_causal_forward(dev(q), dev(k), dev(v), chunk=64, ws=ws)
    assert e.value.code == gpu.LA_ERR_TIMEOUT
    gpu.la_workspace_set_wait(ws, 0, 0)
    out = gpu.la_causal_forward(dev(q), dev(k), dev(v), chunk=64, ws=ws)  # no error now
    check(host(out), oracle.causal(q, k, v), li.BF16, "debug-checked causal")


# ----------------------------------------------------- mask values in range
@pytest.mark.parametrize("dtype,d", [(li.F32, 64), (li.F32, 32), (li.BF16, 64)])
def test_prefix_mask_out_of_range_is_reported(gpu, dtype, d, monkeypatch):
    """A mask value outside [0, n - 1] is recorded by the bucket sort (the
    fp32 d = 64 state launch's sort block, or k_bucket) and reported as
    LA_ERR_RANGE; a valid mask on the same workspace then reports LA_OK.
    With LA_DEBUG_CHECKS=1 the binding raises instead."""
    B, H, n = 2, 2, 1000
    q, k, v, rng = li.qkv(B, H, H, n, d, dtype, seed=63, scaled=True)
    m = li.mask(n, "random", rng=rng)
    bad = m.copy()
    bad[5], bad[700] = n, -3
    dt = gpu.LA_F32 if dtype == li.F32 else gpu.LA_BF16
    ws = new_ws(gpu, gpu.LA_OP_PREFIX_MASK, B, H, H, n, d, dt)
    gpu.la_prefix_mask_forward(dev(q), dev(k), dev(v), dev(bad), ws=ws)
    assert gpu.la_workspace_status(ws) == gpu.LA_ERR_RANGE
    g = gpu.la_prefix_mask_forward(dev(q), dev(k), dev(v), dev(m), ws=ws)
    assert gpu.la_workspace_status(ws) == 0
    check(host(g), oracle.prefix_mask(q, k, v, m), dtype, f"prefix {dtype} d{d} after a bad mask")
    monkeypatch.setenv("LA_DEBUG_CHECKS", "1")
    with pytest.raises(gpu.LAError) as e:
        gpu.la_prefix_mask_forward(dev(q), dev(k), dev(v), dev(bad), ws=ws)
    assert e.value.code == gpu.LA_ERR_RANGE
    bad2 = np.stack([m, bad])  # per-batch masks: batch 1's row is bad
    with pytest.raises(gpu.LAError):
        gpu.la_prefix_mask_forward(dev(q), dev(k), dev(v), dev(bad2))


# ------------------------------------------- the fp32 causal output kernel
@pytest.mark.parametrize("phi", ["relu1", "elu1"])
@pytest.mark.parametrize("shape", [(1, 1, 65536), (1, 2, 40000)], ids=lambda c: "B%d_H%d_n%d" % c)
def test_causal_f32_d64_output_kernel_several_chunks_per_workgroup(gpu, phi, shape):
    """fp32 d = 64 causal with one query head per KV head at sizes where each
    output workgroup walks two or three chunks (the state and z carried from
    chunk to chunk inside the workgroup), both feature maps, every row
    against the oracle."""
    B, H, n = shape
    q, k, v, _ = li.qkv(B, H, H, n, 64, li.F32, seed=64, scaled=True)
    out = gpu.la_causal_forward(dev(q), dev(k), dev(v), phi=phi)
    check(host(out), oracle.causal(q, k, v, phi=phi), li.F32, f"causal f32 d64 {phi} B{B} H{H} n{n}")


# ---------------------------------------------------------- repeated calls
@pytest.mark.parametrize("path", ["single_launch", "noncausal_bf16", "noncausal_f32", "gqa_output",
                                  "prefix_per_batch"])
def test_hundred_calls_bitwise(gpu, path):
    """Workgroups that hand data to each other finish in a different order
    from call to call; every sum they form runs in a fixed order, so 100
    calls on the same inputs give the same bits."""
    if path == "single_launch":
        q, k, v, _ = li.qkv(1, 4, 4, 16384, 64, li.BF16, seed=65, scaled=True)
        qd, kd, vd = dev(q), dev(k), dev(v)
        call = lambda: gpu.la_causal_forward(qd, kd, vd, chunk=64)
    elif path.startswith("noncausal"):
        dt = li.BF16 if path.endswith("bf16") else li.F32
        q, k, v, _ = li.qkv(2, 8, 8, 4096, 64, dt, seed=66)
        qd, kd, vd = dev(q), dev(k), dev(v)
        call = lambda: gpu.la_forward(qd, kd, vd)
    elif path == "gqa_output":
        q, k, v, _ = li.qkv(1, 8, 2, 8192, 128, li.BF16, seed=67, scaled=True)
        qd, kd, vd = dev(q), dev(k), dev(v)
        call = lambda: gpu.la_causal_forward(qd, kd, vd)
    else:
        q, k, v, rng = li.qkv(3, 2, 2, 2000, 64, li.F32, seed=68, scaled=True)
        qd, kd, vd = dev(q), dev(k), dev(v)
        m = dev(np.stack([li.mask(2000, "random", rng=rng) for _ in range(3)]))
        call = lambda: gpu.la_prefix_mask_forward(qd, kd, vd, m, chunk=64)
    ref = li.from_torch(call())
    for i in range(99):
        assert np.array_equal(li.from_torch(call()), ref), (path, i)


# ---------------------------------------------- every row, by closed forms
def test_gqa_long_context_every_row_closed_form(gpu):
    """The long-context GQA shape (B1 Hq32 Hkv8 n65536 d128 bf16) with every
    key row of a KV head equal: each key then has the same weight, so every
    output row is the running mean of V (for any Q) -- checked on all 65536
    rows of all 32 query heads."""
    B, Hq, Hkv, n, d = 1, 32, 8, 65536, 128
    q, _, v, rng = li.qkv(B, Hq, Hkv, n, d, li.BF16, seed=70, scaled=True)
    rows = li.as_dtype(rng.standard_normal((Hkv, d), dtype=np.float32) / np.sqrt(d), li.BF16)
    k = np.ascontiguousarray(np.broadcast_to(rows[None, :, None, :], (B, Hkv, n, d)))
    out = gpu.la_causal_forward(dev(q), dev(k), dev(v))
    worst = 0.0
    for g in range(Hkv):
        want = np.cumsum(li.to_f32(v[0, g]).astype(np.float64), axis=0) / np.arange(1, n + 1)[:, None]
        for h in range(g * (Hq // Hkv), (g + 1) * (Hq // Hkv)):
            worst = max(worst, rel_rows(host(out[0, h]), want))
    print(f"GQA n65536 closed form, all rows: {worst:.3e}", flush=True)
    assert worst <= TOL[li.BF16]


def test_decode_B128_every_sequence_closed_form(gpu):
    """Decode for all 128 sequences: with one key row per (sequence, KV head)
    used for the whole 4096-token prefix and for every step, each output is
    the mean of V over the prefix and the steps so far -- checked for every
    sequence and head at every 16th step and the last."""
    B, Hq, Hkv, d, P, T = 128, 32, 8, 128, 4096, 256
    rng = np.random.default_rng(71)
    s = 1 / np.sqrt(d)
    krow = li.gaussian(rng, (B, Hkv, 1, d), s, li.BF16)
    vp = li.gaussian(rng, (B, Hkv, P, d), s, li.BF16)
    kp = np.ascontiguousarray(np.broadcast_to(krow, (B, Hkv, P, d)))
    S, z = gpu.la_causal_forward(None, dev(kp), dev(vp), Hq=Hq)
    vsum = li.to_f32(vp).astype(np.float64).sum(axis=2)  # [B, Hkv, d]
    kstep = dev(np.ascontiguousarray(krow[:, :, 0]))
    R = Hq // Hkv
    worst = 0.0
    for t in range(T):
        qs = li.gaussian(rng, (B, Hq, d), s, li.BF16)
        vs = li.gaussian(rng, (B, Hkv, d), s, li.BF16)
        o = gpu.la_decode_step(dev(qs), kstep, dev(vs), S, z)
        vsum += li.to_f32(vs).astype(np.float64)
        if t % 16 == 0 or t == T - 1:
            want = np.repeat(vsum / (P + t + 1), R, axis=1)  # [B, Hq, d]
            worst = max(worst, rel_rows(host(o), want))
    print(f"decode closed form, all sequences: {worst:.3e}", flush=True)
    assert worst <= TOL[li.BF16]
