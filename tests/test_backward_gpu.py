"""GPU parity of the causal form's gradients (la_causal_backward) against
the oracle's pairwise derivative on the same seeded inputs.  Metric: the
row-wise max-norm relative error of each gradient (a row = one token's
d-vector in one head); tolerances 1e-4 (fp32 inputs) and 2e-2 (bf16).  One
row is zero by construction and left out of that metric: dQ of a sequence's
first token (its output is V_0 whatever Q_0 is); there the GPU's value must
stay within the tolerance times dQ's largest entry (it is rounding left over
from a cancellation)."""
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


def check_dq(g, o, dtype, what):
    """check() on rows 1 .. n - 1 of every head; row 0 (zero by construction)
    against the median row norm."""
    check(g[:, :, 1:], o[:, :, 1:], dtype, what)
    top = float(np.abs(o[:, :, 1:]).max())
    row0 = float(np.abs(g[:, :, 0]).max())
    print(f"{what}: row 0 (zero by construction) {row0:.3e} vs largest entry {top:.3e}", flush=True)
    assert row0 <= TOL[dtype] * top, f"{what}: row 0 {row0:.3e} > {TOL[dtype]} * {top:.3e}"


def inputs(B, Hq, Hkv, n, d, dtype, seed):
    q, k, v, rng = li.qkv(B, Hq, Hkv, n, d, dtype, seed=seed, scaled=True)
    dout = li.gaussian(rng, (B, Hq, n, d), None, dtype)
    return q, k, v, dout


CASES = [(1, 1, 1, 64, 64), (2, 4, 2, 300, 64), (1, 2, 2, 1000, 32), (1, 2, 1, 257, 16), (1, 1, 1, 5, 3),
         (1, 2, 2, 130, 40)]


@pytest.mark.parametrize("phi", ["relu1", "elu1"])
@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_Hq%d_Hkv%d_n%d_d%d" % c)
def test_backward_small(gpu, phi, dtype, case):
    B, Hq, Hkv, n, d = case
    q, k, v, dout = inputs(B, Hq, Hkv, n, d, dtype, seed=400 + n)
    dq, dk, dv = gpu.la_causal_backward(dev(q), dev(k), dev(v), dev(dout), phi=phi)
    rq, rk, rv = oracle.causal_backward(q, k, v, dout, phi=phi)
    check_dq(host(dq), rq, dtype, f"dq {phi} {dtype} {case}")
    check(host(dk), rk, dtype, f"dk {phi} {dtype} {case}")
    check(host(dv), rv, dtype, f"dv {phi} {dtype} {case}")


def test_backward_features(gpu):
    """Caller-applied features: gradients with respect to the features."""
    B, Hq, Hkv, n, d = 1, 4, 2, 400, 64
    q, k, v, dout = inputs(B, Hq, Hkv, n, d, li.BF16, seed=410)
    sp = lambda x: np.log1p(np.exp(x))
    fq, fk = (li.as_dtype(sp(li.to_f32(x)).astype(np.float32), li.BF16) for x in (q, k))
    dq, dk, dv = gpu.la_causal_backward(dev(fq), dev(fk), dev(v), dev(dout), phi="features")
    rq, rk, rv = oracle.causal_backward(fq, fk, v, dout, phi="features")
    check_dq(host(dq), rq, li.BF16, "dq features")
    for g, r, name in ((dk, rk, "dk"), (dv, rv, "dv")):
        check(host(g), r, li.BF16, f"{name} features")


@pytest.mark.parametrize("dtype", [li.BF16, li.F32])
def test_backward_long_sequence_segments(gpu, dtype):
    """n = 6000 with one head: many segments, each starting from the forward
    prefix and the suffix sums of the later segments."""
    B, H, n, d = 1, 1, 6000, 64
    q, k, v, dout = inputs(B, H, H, n, d, dtype, seed=411)
    dq, dk, dv = gpu.la_causal_backward(dev(q), dev(k), dev(v), dev(dout))
    rq, rk, rv = oracle.causal_backward(q, k, v, dout)
    check_dq(host(dq), rq, dtype, f"dq n6000 {dtype}")
    for g, r, name in ((dk, rk, "dk"), (dv, rv, "dv")):
        check(host(g), r, dtype, f"{name} n6000 {dtype}")


def test_backward_B8_H8_n2048_d64_bf16(gpu):
    """The causal workload's size: every row of every gradient against the
    oracle (the pairwise derivative over 64 heads of 2048 tokens)."""
    B, H, n, d = 8, 8, 2048, 64
    q, k, v, dout = inputs(B, H, H, n, d, li.BF16, seed=412)
    dq, dk, dv = gpu.la_causal_backward(dev(q), dev(k), dev(v), dev(dout))
    rq, rk, rv = oracle.causal_backward(q, k, v, dout)
    check_dq(host(dq), rq, li.BF16, "dq B8 H8 n2048 d64")
    for g, r, name in ((dk, rk, "dk"), (dv, rv, "dv")):
        check(host(g), r, li.BF16, f"{name} B8 H8 n2048 d64")


def test_backward_matches_torch_autograd_of_the_forward(gpu):
    """The GPU gradients against float64 autograd through torch's own
    transcription of the forward, on the CPU (a second reference)."""
    import torch
    B, Hq, Hkv, n, d = 1, 2, 1, 200, 32
    q, k, v, dout = inputs(B, Hq, Hkv, n, d, li.F32, seed=413)
    tq, tk, tv = (torch.tensor(x.astype(np.float64), requires_grad=True) for x in (q, k, v))
    kk, vv = tk.repeat_interleave(2, dim=1), tv.repeat_interleave(2, dim=1)
    w = torch.tril((torch.relu(tq) + 1) @ (torch.relu(kk) + 1).transpose(-1, -2))
    ((w @ vv) / w.sum(-1, keepdim=True) * torch.tensor(dout.astype(np.float64))).sum().backward()
    dq, dk, dv = gpu.la_causal_backward(dev(q), dev(k), dev(v), dev(dout))
    check_dq(host(dq), tq.grad.numpy(), li.F32, "dq vs autograd")
    for g, r, name in ((dk, tk.grad, "dk"), (dv, tv.grad, "dv")):
        check(host(g), r.numpy(), li.F32, f"{name} vs autograd")
