"""la_causal_forward_noalloc (workspace: the library's static per-GPU array)
against la_causal_forward with a caller workspace: two calls in a row, the
second smaller, on the single-launch path and on the general path, the same
bits and the oracle's values; and captured into a graph and replayed."""
import numpy as np
import pytest

import la_inputs as li
import oracle

pytestmark = pytest.mark.gpu


def dev(x):
    return li.to_torch(x).cuda()


def host(t):
    return li.to_f32(li.from_torch(t)).astype(np.float64)


def rel_rows(g, o):
    return float((np.abs(g - o).max(axis=-1) / np.maximum(np.abs(o).max(axis=-1), 1e-30)).max())


@pytest.mark.parametrize("dtype,d,chunk,shapes", [
    (li.BF16, 64, 64, [(8, 8, 8, 2048), (2, 3, 3, 700)]),   # single-launch kernel, then smaller
    (li.F32, 32, 32, [(2, 4, 2, 3000), (1, 2, 1, 130)]),     # general path (GQA), then smaller
], ids=["single_launch", "general"])
def test_noalloc_matches_the_workspace_entry_point(gpu, dtype, d, chunk, shapes):
    tol = 2e-2 if dtype == li.BF16 else 1e-4
    for i, (B, Hq, Hkv, n) in enumerate(shapes):
        print(f"noalloc call {i}: B{B} Hq{Hq} Hkv{Hkv} n{n} d{d} {dtype}", flush=True)
        q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, dtype, seed=80 + i, scaled=True)
        qd, kd, vd = dev(q), dev(k), dev(v)
        a, Sa, za = gpu.la_causal_forward(qd, kd, vd, chunk=chunk, want_state=True)
        b, Sb, zb = gpu.la_causal_forward_noalloc(qd, kd, vd, chunk=chunk, want_state=True)
        assert np.array_equal(li.from_torch(a), li.from_torch(b))
        assert np.array_equal(Sa.cpu().numpy(), Sb.cpu().numpy())
        assert np.array_equal(za.cpu().numpy(), zb.cpu().numpy())
        ref = oracle.causal(q, k, v)
        err = rel_rows(host(b), ref)
        print(f"  row-wise rel err {err:.3e}", flush=True)
        assert err <= tol


def test_noalloc_under_graph_capture(gpu):
    """The allocation-free call captured into a graph, replayed three times
    with new inputs in the static buffers: each replay matches the oracle."""
    import torch
    B, H, n, d = 4, 8, 2048, 64
    qs, ks, vs = (torch.empty((B, H, n, d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    out = torch.empty_like(qs)
    q0, k0, v0, _ = li.qkv(B, H, H, n, d, li.BF16, seed=90, scaled=True)
    qs.copy_(dev(q0)); ks.copy_(dev(k0)); vs.copy_(dev(v0))
    gpu.la_causal_forward_noalloc(qs, ks, vs, chunk=64, out=out)  # first call on the device: set-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gpu.la_causal_forward_noalloc(qs, ks, vs, chunk=64, out=out)
    for rep in range(3):
        q, k, v, _ = li.qkv(B, H, H, n, d, li.BF16, seed=91 + rep, scaled=True)
        qs.copy_(dev(q)); ks.copy_(dev(k)); vs.copy_(dev(v))
        graph.replay()
        torch.cuda.synchronize()
        err = rel_rows(host(out), oracle.causal(q, k, v))
        print(f"noalloc replay {rep}: {err:.3e}", flush=True)
        assert err <= 2e-2
        gpu.la_causal_forward_noalloc(qs, ks, vs, chunk=64)  # eager work between replays
        torch.cuda.synchronize()
