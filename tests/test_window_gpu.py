"""GPU parity of the sliding-window form (LinearTile 1.0.1, "Features"):
query i sees keys i - w < j <= i.  Against the oracle's pairwise sums on
the same seeded inputs; metric and tolerances as in test_parity_gpu.py."""
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


# windows around the chunk sizes (32, 64) and the sequence end
WINDOWS = [1, 2, 31, 32, 33, 63, 64, 65, 100, 129, 300]


@pytest.mark.parametrize("dtype,d", [(li.BF16, 64), (li.BF16, 128), (li.BF16, 32), (li.F32, 64), (li.F32, 32),
                                     (li.BF16, 17), (li.F32, 40)])
@pytest.mark.parametrize("w", WINDOWS)
def test_window_small(gpu, dtype, d, w):
    B, Hq, Hkv, n = 2, 4, 2, 301  # ragged tail, several chunks, GQA
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, dtype, seed=200 + w, scaled=True)
    g = gpu.la_window_forward(dev(q), dev(k), dev(v), w)
    check(host(g), oracle.window(q, k, v, w), dtype, f"window w={w} d={d} {dtype}")


@pytest.mark.parametrize("phi", ["relu1", "elu1"])
@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
def test_window_feature_maps_and_long_segments(gpu, phi, dtype):
    """n = 3000 with w = 700: segments of several chunks after a warm-up of
    eleven (bf16 d = 64) or twenty-two (fp32) chunks; four query heads per
    key/value head."""
    B, Hq, Hkv, n, d, w = 1, 8, 2, 3000, 64, 700
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, dtype, seed=210, scaled=True)
    g = gpu.la_window_forward(dev(q), dev(k), dev(v), w, phi=phi)
    check(host(g), oracle.window(q, k, v, w, phi=phi), dtype, f"window {phi} {dtype} n{n} w{w}")


def test_window_features(gpu):
    """A caller-applied map (softplus) through the window form."""
    B, Hq, Hkv, n, d, w = 2, 2, 2, 500, 64, 77
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, li.BF16, seed=211, scaled=True)
    sp = lambda x: np.log1p(np.exp(x))
    fq, fk = (li.as_dtype(sp(li.to_f32(x)).astype(np.float32), li.BF16) for x in (q, k))
    g = gpu.la_window_forward(dev(fq), dev(fk), dev(v), w, phi="features")
    check(host(g), oracle.window(q, k, v, w, phi=sp), li.BF16, "window features softplus")


def test_window_covering_everything_is_causal(gpu):
    q, k, v, _ = li.qkv(2, 4, 4, 1000, 64, li.BF16, seed=212, scaled=True)
    g = gpu.la_window_forward(dev(q), dev(k), dev(v), 5000)
    check(host(g), oracle.causal(q, k, v), li.BF16, "window >= n")


def test_window_B8_H8_n2048_d64_bf16_w512(gpu):
    """The causal workload's size with a 512-token window (the benchmark's
    window workload): sampled rows against the oracle, and every row of an
    equal-keys input against the window mean of V."""
    B, H, n, d, w = 8, 8, 2048, 64, 512
    q, k, v, rng = li.qkv(B, H, H, n, d, li.BF16, seed=213, scaled=True)
    g = host(gpu.la_window_forward(dev(q), dev(k), dev(v), w))
    rows = np.unique(np.concatenate([rng.choice(n, 60, replace=False), [0, 63, 64, 511, 512, 513, n - 1]]))
    check(g[:, :, rows], oracle.window(q, k, v, w, rows=rows), li.BF16, "window B8 H8 n2048 w512 (sampled rows)")
    row = li.as_dtype(rng.standard_normal(d, dtype=np.float32) / 8, li.BF16)
    ke = np.ascontiguousarray(np.broadcast_to(row, (B, H, n, d)))
    ge = host(gpu.la_window_forward(dev(q), dev(ke), dev(v), w))
    c = np.cumsum(np.concatenate([np.zeros((B, H, 1, d)), li.to_f32(v).astype(np.float64)], axis=2), axis=2)
    lo = np.maximum(np.arange(n) - w + 1, 0)
    want = (c[:, :, np.arange(n) + 1] - c[:, :, lo]) / (np.arange(n) + 1 - lo)[None, None, :, None]
    check(ge, want, li.BF16, "window equal keys, every row")


# One query head per key/value head, bf16, d = 64: the single-launch window
# kernel (w < 576: up to seven chunks of halo).  Windows around every chunk
# boundary it treats differently: w < 64 (leading band only), multiples of
# 64 (one trailing chunk), w = 64 k + 1 .. 64 k + 63 (two trailing chunks).
FUSED_WINDOWS = [1, 2, 31, 63, 64, 65, 100, 127, 128, 129, 191, 192, 200, 300, 447, 448, 449, 511, 512, 513, 575]


@pytest.mark.parametrize("phi", ["relu1", "elu1"])
@pytest.mark.parametrize("w", FUSED_WINDOWS)
def test_window_single_launch(gpu, phi, w):
    """B2 H3 n1500 (three segments of eight chunks, the last ragged): every
    row against the oracle."""
    B, H, n, d = 2, 3, 1500, 64
    q, k, v, _ = li.qkv(B, H, H, n, d, li.BF16, seed=220 + w, scaled=True)
    g = gpu.la_window_forward(dev(q), dev(k), dev(v), w, phi=phi)
    check(host(g), oracle.window(q, k, v, w, phi=phi), li.BF16, f"window (single launch) {phi} w={w}")


def test_window_single_launch_equal_keys_every_row(gpu):
    """Equal keys make every weight equal: out_i is the mean of V over the
    window, a closed form that the halo and own parts must both respect
    (n = 4000, w = 383: two trailing chunks, five halo chunks)."""
    B, H, n, d, w = 1, 4, 4000, 64, 383
    q, k, v, rng = li.qkv(B, H, H, n, d, li.BF16, seed=230, scaled=True)
    row = li.as_dtype(rng.standard_normal(d, dtype=np.float32) / 8, li.BF16)
    ke = np.ascontiguousarray(np.broadcast_to(row, (B, H, n, d)))
    g = host(gpu.la_window_forward(dev(q), dev(ke), dev(v), w))
    c = np.cumsum(np.concatenate([np.zeros((B, H, 1, d)), li.to_f32(v).astype(np.float64)], axis=2), axis=2)
    lo = np.maximum(np.arange(n) - w + 1, 0)
    want = (c[:, :, np.arange(n) + 1] - c[:, :, lo]) / (np.arange(n) + 1 - lo)[None, None, :, None]
    check(g, want, li.BF16, "window w383 equal keys, every row")


@pytest.mark.parametrize("phi", ["relu1", "elu1"])
@pytest.mark.parametrize("shape", [(2, 16, 4, 1100, 300), (1, 6, 2, 900, 512), (1, 64, 8, 700, 64)],
                         ids=lambda c: "B%d_Hq%d_Hkv%d_n%d_w%d" % c)
def test_window_single_launch_gqa(gpu, phi, shape):
    """Grouped query heads on the single-launch window kernel (two to eight
    per key/value head; B2 Hq16 Hkv4 and B1 Hq64 Hkv8 take the XCD-grouped
    dispatch order): every row against the oracle."""
    B, Hq, Hkv, n, w = shape
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, 64, li.BF16, seed=240 + w, scaled=True)
    g = gpu.la_window_forward(dev(q), dev(k), dev(v), w, phi=phi)
    check(host(g), oracle.window(q, k, v, w, phi=phi), li.BF16, f"window GQA {phi} {shape}")
