"""GPU parity for a feature map of the caller's choice (LinearTile 1.0.1,
"Features": phi replaceable at will).  The map is defined here: the caller
applies it to Q and K and passes the features (phi="features",
LA_PHI_FEATURES); the oracle applies the same map itself, in fp64, to the
raw Q and K (its function callback).  Metric and tolerances as in
test_parity_gpu.py."""
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


def softplus(x):
    return np.log1p(np.exp(x))


def half_exp(x):  # exp(x / 2): a positive map with no floor
    return np.exp(0.5 * x)


MAPS = {"softplus": softplus, "half_exp": half_exp}


def features(x, fn, dtype):
    """The caller's side: the map applied to the stored inputs in fp32, the
    result stored in the input dtype."""
    return li.as_dtype(fn(li.to_f32(x)).astype(np.float32), dtype)


CASES = [(2, 4, 2, 300, 64), (2, 3, 3, 700, 64), (1, 2, 2, 1000, 32), (1, 2, 1, 257, 128), (1, 1, 1, 5, 3)]


@pytest.mark.parametrize("mapname", sorted(MAPS))
@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_Hq%d_Hkv%d_n%d_d%d" % c)
def test_features_normalised_forms(gpu, mapname, dtype, case):
    fn = MAPS[mapname]
    B, Hq, Hkv, n, d = case
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, dtype, seed=100, scaled=True)
    fq, fk = dev(features(q, fn, dtype)), dev(features(k, fn, dtype))
    g = gpu.la_forward(fq, fk, dev(v), phi="features")
    check(host(g), oracle.forward(q, k, v, phi=fn), dtype, f"forward features {mapname}")
    out, S, z = gpu.la_causal_forward(fq, fk, dev(v), want_state=True, phi="features")
    ref, Sr, zr = oracle.causal(q, k, v, want_state=True, phi=fn)
    check(host(out), ref, dtype, f"causal features {mapname}")
    rtol = 1e-4 if dtype == li.F32 else 1e-2
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=rtol)
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=rtol, atol=rtol * np.abs(Sr).max())


@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
@pytest.mark.parametrize("d", [64, 128])
def test_features_decode_continues_the_causal_pass(gpu, dtype, d):
    """A state built over a prefix of caller-mapped features, continued by
    decode steps on mapped features, equals the oracle's causal pass with
    the map applied inside."""
    B, Hq, Hkv, n, T = 2, 8, 2, 200, 6
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, dtype, seed=101, scaled=True)
    full = oracle.causal(q, k, v, phi=softplus)
    fq, fk = features(q, softplus, dtype), features(k, softplus, dtype)
    S, z = gpu.la_causal_forward(None, dev(fk[:, :, : n - T].copy()), dev(v[:, :, : n - T].copy()), Hq=Hq,
                                 phi="features")
    for t in range(n - T, n):
        o = gpu.la_decode_step(dev(fq[:, :, t].copy()), dev(fk[:, :, t].copy()), dev(v[:, :, t].copy()), S, z,
                               phi="features")
        check(host(o), full[:, :, t], dtype, f"decode features step {t}")


def test_features_equal_keys_closed_form_full_scale(gpu):
    """At the causal workload's size (B8 H8 n2048 d64 bf16) with every key row
    equal, any positive map gives the running mean of V on every row."""
    B, H, n, d = 8, 8, 2048, 64
    q, _, v, rng = li.qkv(B, H, H, n, d, li.BF16, seed=102, scaled=True)
    row = li.as_dtype(rng.standard_normal(d, dtype=np.float32) / 8, li.BF16)
    k = np.ascontiguousarray(np.broadcast_to(row, (B, H, n, d)))
    out = gpu.la_causal_forward(dev(features(q, half_exp, li.BF16)), dev(features(k, half_exp, li.BF16)), dev(v),
                                phi="features")
    want = np.cumsum(li.to_f32(v).astype(np.float64), axis=2) / np.arange(1, n + 1)[None, None, :, None]
    check(host(out), want, li.BF16, "causal features, equal keys")
