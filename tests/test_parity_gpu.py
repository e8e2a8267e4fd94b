"""GPU parity: the HIP kernels (through the C ABI and its binding) against
the fp64 oracle on identical seeded inputs.

Metric: the largest row-wise max-norm relative error,
max_rows ||gpu_row - oracle_row||_inf / ||oracle_row||_inf, where a row is
one query's d-vector in one head.  Tolerances: 1e-4 for fp32 inputs and
2e-2 for bf16 inputs (fp32 accumulation in both).  Element-wise relative
error is not used: outputs near zero make it meaningless.
"""
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
    num = np.abs(g - o).max(axis=-1)
    den = np.abs(o).max(axis=-1)
    return float((num / np.maximum(den, 1e-30)).max())


def fit_chunk(gpu, dtype, d, chunk):
    """The requested chunk if the library offers it for this dtype and head
    dim (it must fit one CU's LDS), else the largest smaller one."""
    code = gpu.LA_F32 if dtype == li.F32 else gpu.LA_BF16
    for c in [chunk] + [c for c in (128, 64, 32) if c < (chunk or 65)]:
        if gpu.la_workspace_bytes(gpu.LA_OP_CAUSAL, 1, 1, 1, 64, d, code, c) > 0:
            return c
    raise AssertionError("no chunk size fits")


def check(g, o, dtype, what):
    err = rel_rows(g, o)
    print(f"{what}: row-wise rel err {err:.3e} (tol {TOL[dtype]:.0e})", flush=True)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    assert err <= TOL[dtype], f"{what}: {err:.3e} > {TOL[dtype]}"
    return err


# --------------------------------------------------------------- hand cases
@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
def test_hand_cases(gpu, dtype):
    """The nx page's gates through the GPU (d = 2: 30 masked feature lanes)."""
    for which, want_nc, want_c in (
            ("zero", [[4, 6], [4, 6]], [[2, 4], [4, 6]]),
            ("identity", [[34 / 9, 52 / 9], [38 / 9, 56 / 9]], [[2, 4], [38 / 9, 56 / 9]])):
        q, k, v = (li.as_dtype(x, dtype) for x in li.hand_case(which))
        nc = host(gpu.la_forward(dev(q), dev(k), dev(v)))[0, 0]
        ca = host(gpu.la_causal_forward(dev(q), dev(k), dev(v)))[0, 0]
        check(nc, np.array(want_nc, float), dtype, f"gate {which} non-causal")
        check(ca, np.array(want_c, float), dtype, f"gate {which} causal")
    # the page's state for gate 2
    q, k, v = (li.as_dtype(x, dtype) for x in li.hand_case("identity"))
    _, S, z = gpu.la_causal_forward(dev(q), dev(k), dev(v), want_state=True)
    np.testing.assert_allclose(S.cpu().numpy()[0, 0], [[10, 16], [14, 20]], rtol=1e-6)
    np.testing.assert_allclose(z.cpu().numpy()[0, 0], [3, 3], rtol=1e-6)


# ------------------------------------------------------------- small / ragged
SMALL = [
    # (B, Hq, Hkv, n, d, chunk)
    (1, 1, 1, 256, 16, 0),     # the tiny config
    (1, 1, 1, 1, 1, 32),
    (2, 2, 1, 2, 3, 64),
    (1, 3, 1, 63, 64, 32),
    (1, 2, 2, 65, 64, 64),
    (2, 4, 2, 100, 33, 64),
    (1, 2, 1, 257, 128, 64),
    (1, 1, 1, 300, 100, 128),
    (1, 4, 4, 129, 64, 128),
    (2, 8, 2, 200, 31, 32),
    (2, 4, 2, 1000, 64, 64),   # bf16 non-causal: state partials of several segments, GQA
    (1, 2, 1, 4500, 64, 32),   # 18 segments: the reduces' batches of sixteen and a remainder
    (1, 1, 1, 1, 64, 64),      # one token at d = 64
    (1, 4, 1, 300, 128, 32),   # bf16 causal: four query heads per chunk at once, ragged tail
    (2, 4, 2, 97, 128, 0),     # ... two query heads (default chunk 32)
]


def _small_id(c):
    return "B%d_Hq%d_Hkv%d_n%d_d%d_c%d" % c


@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
@pytest.mark.parametrize("case", SMALL, ids=_small_id)
def test_noncausal_small(gpu, dtype, case):
    B, Hq, Hkv, n, d, _ = case
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, dtype, seed=0)
    g = host(gpu.la_forward(dev(q), dev(k), dev(v)))
    check(g, oracle.forward(q, k, v), dtype, f"forward {_small_id(case)} {dtype}")


@pytest.mark.parametrize("fill", ["random", "ones"])
def test_workspace_contents_do_not_matter(gpu, fill):
    """Past the control block (zeroed by la_workspace_init), the kernels that
    hand data between workgroups (the non-causal passes, the single-launch
    causal kernel, the prefix form's sort and state) read no workspace word
    before this call wrote it: their flags must equal the call's epoch, so a
    workspace holding random bytes or all-ones bytes gives the same outputs
    as a zero-filled one."""
    import torch
    gen = torch.Generator(device="cpu").manual_seed(3)

    def ws(op, B, Hq, Hkv, n, d, dt, chunk=0):
        nbytes = gpu.la_workspace_bytes(op, B, Hq, Hkv, n, d, 1 if dt == li.BF16 else 0, chunk)
        if fill == "random":
            w = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=gen)
        else:
            w = torch.full((nbytes,), 255, dtype=torch.uint8)
        w = w.to("cuda")
        gpu.la_workspace_init(w)
        return w

    for dtype in (li.BF16, li.F32):
        B, Hq, Hkv, n, d = 2, 4, 2, 1000, 64
        q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, dtype, seed=4)
        g = gpu.la_forward(dev(q), dev(k), dev(v), ws=ws(gpu.LA_OP_FORWARD, B, Hq, Hkv, n, d, dtype))
        check(host(g), oracle.forward(q, k, v), dtype, f"forward {fill} workspace {dtype}")
    B, H, n, d = 2, 2, 1000, 64
    q, k, v, rng = li.qkv(B, H, H, n, d, li.BF16, seed=5, scaled=True)
    out = gpu.la_causal_forward(dev(q), dev(k), dev(v), chunk=64, ws=ws(gpu.LA_OP_CAUSAL, B, H, H, n, d, li.BF16, 64))
    check(host(out), oracle.causal(q, k, v), li.BF16, f"causal {fill} workspace")
    q, k, v, rng = li.qkv(B, H, H, n, d, li.F32, seed=6, scaled=True)
    m = li.mask(n, "random", rng=rng)
    g = gpu.la_prefix_mask_forward(dev(q), dev(k), dev(v), dev(m), chunk=64,
                                   ws=ws(gpu.LA_OP_PREFIX_MASK, B, H, H, n, d, li.F32, 64))
    check(host(g), oracle.prefix_mask(q, k, v, m), li.F32, f"prefix {fill} workspace")


@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
@pytest.mark.parametrize("case", SMALL, ids=_small_id)
def test_causal_small(gpu, dtype, case):
    B, Hq, Hkv, n, d, chunk = case
    chunk = fit_chunk(gpu, dtype, d, chunk)
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, dtype, seed=1, scaled=True)
    out, S, z = gpu.la_causal_forward(dev(q), dev(k), dev(v), chunk=chunk, want_state=True)
    ref, Sr, zr = oracle.causal(q, k, v, want_state=True)
    check(host(out), ref, dtype, f"causal {_small_id(case)} {dtype}")
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=1e-4, atol=1e-4 * np.abs(Sr).max())
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=1e-5)


@pytest.mark.parametrize("kind", ["random", "causal", "full", "first"])
@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
@pytest.mark.parametrize("case", SMALL[:8], ids=_small_id)
def test_prefix_small(gpu, dtype, kind, case):
    B, H, _, n, d, chunk = case
    chunk = fit_chunk(gpu, dtype, d, chunk)
    q, k, v, rng = li.qkv(B, H, H, n, d, dtype, seed=2, scaled=True)
    m = li.mask(n, kind, rng=rng)
    g = host(gpu.la_prefix_mask_forward(dev(q), dev(k), dev(v), dev(m), chunk=chunk))
    check(g, oracle.prefix_mask(q, k, v, m), dtype, f"prefix {kind} {_small_id(case)} {dtype}")


@pytest.mark.parametrize("kind", ["random", "causal", "full"])
@pytest.mark.parametrize("shape", [(1, 2, 1000), (2, 3, 300)], ids=lambda c: "B%d_H%d_n%d" % c)
def test_prefix_f32_d64_query_groups(gpu, kind, shape):
    """fp32, d = 64, chunk 64 (the 16x16x4 MFMA prefix kernel): ragged tails,
    several segments, and with the 'full' mask a single bucket of n queries,
    so that a chunk takes several groups of 128 queries.  Not the 'first'
    mask at these sizes: it makes every row the single dot product q_i . k_0
    times v_0, whose fp32 relative error is unbounded when the dot product
    cancels (seed 5, B1 H2 n1000 has a row with sum |q_a k_a| / |q . k| of
    about 15000, where numpy's own fp32 product is off by 1.2e-4)."""
    B, H, n = shape
    q, k, v, rng = li.qkv(B, H, H, n, 64, li.F32, seed=5, scaled=True)
    m = li.mask(n, kind, rng=rng)
    g = host(gpu.la_prefix_mask_forward(dev(q), dev(k), dev(v), dev(m), chunk=64))
    check(g, oracle.prefix_mask(q, k, v, m), li.F32, f"prefix {kind} B{B} H{H} n{n} d64 f32")


def test_prefix_f32_d64_bucket_sizes_every_row(gpu):
    """fp32, d = 64, chunk 64, a mask built for its bucket sizes (queries per
    chunk of keys): empty buckets, single queries, whole and partial 16-query
    blocks, groups of one to three blocks (which the four waves share block by
    block) and of four, and buckets of several groups ending in each of those.
    Every row of two batches and two heads against the oracle."""
    sizes = [5, 16, 21, 37, 48, 64, 70, 96, 130, 3, 0, 50, 200, 100, 90, 94]
    n, C = 64 * len(sizes), 64
    assert sum(sizes) == n
    rng = np.random.default_rng(21)
    m = np.concatenate([rng.integers(C * c, C * c + C, size=cnt) for c, cnt in enumerate(sizes)]).astype(np.int64)
    m = m[rng.permutation(n)]  # which query lands in which bucket: arbitrary
    q, k, v, _ = li.qkv(2, 2, 2, n, 64, li.F32, seed=22, scaled=True)
    g = host(gpu.la_prefix_mask_forward(dev(q), dev(k), dev(v), dev(m), chunk=64))
    check(g, oracle.prefix_mask(q, k, v, m), li.F32, "prefix f32 d64, chosen bucket sizes")


@pytest.mark.parametrize("phi", ["relu1", "elu1"])
@pytest.mark.parametrize("shape", [(1, 4, 2, 1500), (2, 8, 2, 700), (4, 16, 2, 600), (1, 64, 8, 300), (3, 6, 3, 513)],
                         ids=lambda c: "B%d_Hq%d_Hkv%d_n%d" % c)
def test_causal_gqa_single_launch(gpu, phi, shape):
    """bf16, d = 64, several query heads per key/value head (2 to 8): the
    single-launch causal kernel with each query head on its own segment
    chain (B4 Hq16 Hkv2 and B1 Hq64 Hkv8 hold whole blocks of eight groups:
    the XCD-grouped dispatch order).  Every row, and the final state of
    every key/value head."""
    B, Hq, Hkv, n = shape
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, 64, li.BF16, seed=13, scaled=True)
    out, S, z = gpu.la_causal_forward(dev(q), dev(k), dev(v), want_state=True, phi=phi)
    ref, Sr, zr = oracle.causal(q, k, v, want_state=True, phi=phi)
    check(host(out), ref, li.BF16, f"causal GQA {phi} B{B} Hq{Hq} Hkv{Hkv} n{n}")
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=1e-2)
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=1e-2, atol=1e-2 * np.abs(Sr).max())


@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
@pytest.mark.parametrize("kind", ["random", "causal"])
@pytest.mark.parametrize("batched", [False, True])
def test_prefix_sort_over_several_blocks(gpu, dtype, kind, batched):
    """n = 20000 queries: more than one block of the bucket sort (8192 mask
    values per pass in the fp32 state launch's sort blocks and in the sort
    launch of the other kernels), so the scatter pass reloads the mask block
    by block.  Sampled rows of every batch against the oracle."""
    B, H, n = (2, 1, 20000) if batched else (1, 2, 20000)
    q, k, v, rng = li.qkv(B, H, H, n, 64, dtype, seed=11, scaled=True)
    if batched:
        m = np.stack([li.mask(n, kind, rng=rng) for _ in range(B)])
        g = host(gpu.la_prefix_mask_forward(dev(q), dev(k), dev(v), dev(m)))
    else:
        m = li.mask(n, kind, rng=rng)
        g = host(gpu.la_prefix_mask_forward(dev(q), dev(k), dev(v), dev(m)))
    rows = np.unique(np.concatenate([rng.choice(n, 150, replace=False), [0, 8191, 8192, n - 1]]))
    for b in range(B):
        mb = m[b] if batched else m
        sl = lambda x: np.ascontiguousarray(x[b:b + 1])
        ref = oracle.prefix_mask(sl(q), sl(k), sl(v), mb, rows=rows)
        check(g[b:b + 1, :, rows], ref, dtype, f"prefix {dtype} {kind} n{n} batch {b} (sampled rows)")


@pytest.mark.parametrize("phi", ["relu1", "elu1"])
@pytest.mark.parametrize("shape", [(1, 2, 1000), (2, 3, 300), (1, 1, 64), (1, 1, 5)], ids=lambda c: "B%d_H%d_n%d" % c)
def test_causal_f32_d64_chunk64_output_kernel(gpu, phi, shape):
    """fp32, d = 64, one query head per KV head: the default chunk 64 runs the
    16x16x4 MFMA output kernel with the chunks as buckets, phi applied as the
    rows are staged and z carried beside S.  Ragged tails, several segments,
    a single chunk, a partial single chunk; the final state as well."""
    B, H, n = shape
    q, k, v, _ = li.qkv(B, H, H, n, 64, li.F32, seed=9, scaled=True)
    assert gpu.la_workspace_bytes(gpu.LA_OP_CAUSAL, B, H, H, n, 64, gpu.LA_F32, 0) == \
        gpu.la_workspace_bytes(gpu.LA_OP_CAUSAL, B, H, H, n, 64, gpu.LA_F32, 64)
    out, S, z = gpu.la_causal_forward(dev(q), dev(k), dev(v), want_state=True, phi=phi)
    ref, Sr, zr = oracle.causal(q, k, v, want_state=True, phi=phi)
    check(host(out), ref, li.F32, f"causal f32 d64 {phi} B{B} H{H} n{n}")
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=1e-4, atol=1e-4 * np.abs(Sr).max())
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=1e-5)


@pytest.mark.parametrize("phi", ["relu1", "elu1"])
@pytest.mark.parametrize("shape", [(1, 1, 65536), (1, 2, 40000)], ids=lambda c: "B%d_H%d_n%d" % c)
def test_causal_f32_d64_chunk64_walks_several_chunks(gpu, phi, shape):
    """Shapes where each output workgroup walks several chunks (two at
    B1 H1 n65536, three at B1 H2 n40000), so that S and z are carried from
    chunk to chunk inside the workgroup: every row against the oracle, both
    feature maps, and the final state."""
    B, H, n = shape
    q, k, v, _ = li.qkv(B, H, H, n, 64, li.F32, seed=23, scaled=True)
    out, S, z = gpu.la_causal_forward(dev(q), dev(k), dev(v), want_state=True, phi=phi)
    ref, Sr, zr = oracle.causal(q, k, v, want_state=True, phi=phi)
    check(host(out), ref, li.F32, f"causal f32 d64 {phi} B{B} H{H} n{n}")
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=1e-4, atol=1e-4 * np.abs(Sr).max())
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=1e-5)


def test_causal_f32_d64_full_scale_sampled(gpu):
    """The same kernel at B4 H8 n8192 (512 output workgroups, each walking
    one state segment of eight chunks): sampled rows against the oracle's
    closed form per row."""
    B, H, n, d = 4, 8, 8192, 64
    q, k, v, _ = li.qkv(B, H, H, n, d, li.F32, seed=13, scaled=True)
    g = host(gpu.la_causal_forward(dev(q), dev(k), dev(v)))
    rng = np.random.default_rng(3)
    for b, h, i in zip(rng.integers(0, B, 12), rng.integers(0, H, 12), list(rng.integers(0, n, 10)) + [0, n - 1]):
        pk = np.maximum(k[b, h, : i + 1].astype(np.float64), 0) + 1
        pq = np.maximum(q[b, h, i].astype(np.float64), 0) + 1
        sc = pk @ pq
        ref = (sc @ v[b, h, : i + 1].astype(np.float64)) / sc.sum()
        err = np.abs(g[b, h, i] - ref).max() / np.abs(ref).max()
        assert err <= 1e-4, (b, h, i, err)


def test_prefix_page_mask(gpu):
    """m = [2, 0, 1] (the trim-transformer page's example) on the GPU."""
    q, k, v, _ = li.qkv(1, 2, 2, 3, 4, li.F32, seed=11)
    m = np.array([2, 0, 1], dtype=np.int64)
    g = host(gpu.la_prefix_mask_forward(dev(q), dev(k), dev(v), dev(m)))
    check(g, oracle.prefix_mask(q, k, v, m), li.F32, "prefix [2,0,1]")


@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
def test_chunk_size_invariance(gpu, dtype):
    """The chunk length only changes rounding: 32, 64 and 128 agree with the oracle."""
    q, k, v, _ = li.qkv(2, 4, 2, 777, 64, dtype, seed=5, scaled=True)
    ref = oracle.causal(q, k, v)
    code = gpu.LA_F32 if dtype == li.F32 else gpu.LA_BF16
    chunks = [c for c in (32, 64, 128)
              if gpu.la_workspace_bytes(gpu.LA_OP_CAUSAL, 2, 4, 2, 777, 64, code, c) > 0]
    assert len(chunks) >= 2
    for chunk in chunks:
        g = host(gpu.la_causal_forward(dev(q), dev(k), dev(v), chunk=chunk))
        check(g, ref, dtype, f"causal chunk {chunk}")


@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
def test_decode_continues_causal(gpu, dtype):
    """State-only causal pass over n - T tokens, then T decode steps, equals the
    causal pass over all n tokens (outputs and final state)."""
    B, Hq, Hkv, n, d, T = 3, 4, 2, 150, 64, 6
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, dtype, seed=6, scaled=True)
    full, Sf, zf = oracle.causal(q, k, v, want_state=True)
    qd, kd, vd = dev(q), dev(k), dev(v)
    S, z = gpu.la_causal_forward(None, kd[:, :, :n - T].contiguous(), vd[:, :, :n - T].contiguous(), Hq=Hq)
    for t in range(n - T, n):
        o = gpu.la_decode_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), S, z)
        check(host(o), full[:, :, t], dtype, f"decode step {t}")
    np.testing.assert_allclose(S.cpu().numpy(), Sf, rtol=1e-4, atol=1e-4 * np.abs(Sf).max())
    np.testing.assert_allclose(z.cpu().numpy(), zf, rtol=1e-5)


@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
@pytest.mark.parametrize("d", [1, 3, 4, 16, 33, 100, 128])
def test_decode_head_dims(gpu, dtype, d):
    """Decode steps over head dims that take the 16-byte path (powers of two)
    and the scalar path (the others), continuing a causal prefix."""
    B, Hq, Hkv, n, T = 2, 4, 2, 40, 3
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, dtype, seed=11 + d, scaled=True)
    full, Sf, zf = oracle.causal(q, k, v, want_state=True)
    qd, kd, vd = dev(q), dev(k), dev(v)
    S, z = gpu.la_causal_forward(None, kd[:, :, :n - T].contiguous(), vd[:, :, :n - T].contiguous(), Hq=Hq)
    for t in range(n - T, n):
        o = gpu.la_decode_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), S, z)
        check(host(o), full[:, :, t], dtype, f"decode d={d} step {t}")
    np.testing.assert_allclose(S.cpu().numpy(), Sf, rtol=1e-4, atol=1e-4 * np.abs(Sf).max())
    np.testing.assert_allclose(z.cpu().numpy(), zf, rtol=1e-5)


@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (6, 3), (64, 1), (65, 1)])
def test_decode_d128_group_sizes(gpu, dtype, Hq, Hkv):
    """Decode at d = 128 over query-group sizes R = Hq / Hkv: 1, 2, 64 (the
    largest group whose phi(q) the step stages in LDS) and 65 (past it, the
    step with per-head LDS reductions)."""
    B, n, T, d = 2, 24, 2, 128
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, dtype, seed=5 + Hq, scaled=True)
    full, Sf, zf = oracle.causal(q, k, v, want_state=True)
    qd, kd, vd = dev(q), dev(k), dev(v)
    S, z = gpu.la_causal_forward(None, kd[:, :, :n - T].contiguous(), vd[:, :, :n - T].contiguous(), Hq=Hq)
    for t in range(n - T, n):
        o = gpu.la_decode_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), S, z)
        check(host(o), full[:, :, t], dtype, f"decode Hq={Hq} Hkv={Hkv} step {t}")
    np.testing.assert_allclose(S.cpu().numpy(), Sf, rtol=1e-4, atol=1e-4 * np.abs(Sf).max())
    np.testing.assert_allclose(z.cpu().numpy(), zf, rtol=1e-5)


def test_state_only_matches_full_pass(gpu):
    q, k, v, _ = li.qkv(2, 4, 2, 300, 64, li.BF16, seed=7, scaled=True)
    _, S1, z1 = gpu.la_causal_forward(dev(q), dev(k), dev(v), want_state=True)
    S2, z2 = gpu.la_causal_forward(None, dev(k), dev(v), Hq=4)
    assert np.array_equal(S1.cpu().numpy(), S2.cpu().numpy())
    assert np.array_equal(z1.cpu().numpy(), z2.cpu().numpy())


def test_run_to_run_bitwise(gpu):
    q, k, v, rng = li.qkv(2, 8, 8, 1000, 64, li.BF16, seed=8, scaled=True)
    qd, kd, vd = dev(q), dev(k), dev(v)
    bits = lambda t: li.from_torch(t)  # raw bf16 bit patterns
    a = bits(gpu.la_causal_forward(qd, kd, vd))
    b = bits(gpu.la_causal_forward(qd, kd, vd))
    assert np.array_equal(a, b)
    m = dev(li.mask(1000, "random", rng=rng))
    a = bits(gpu.la_prefix_mask_forward(qd, kd, vd, m))
    b = bits(gpu.la_prefix_mask_forward(qd, kd, vd, m))
    assert np.array_equal(a, b)
    a = bits(gpu.la_forward(qd, kd, vd))
    b = bits(gpu.la_forward(qd, kd, vd))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("path", ["single_launch_32_segments", "single_launch_elu1", "noncausal_f32",
                                  "gqa_output", "prefix_per_batch"])
def test_repeated_calls_bitwise(gpu, path):
    """Workgroups that hand data to each other finish in a different order
    from call to call; the sums they form are in a fixed order, so five calls
    give the same bits."""
    if path.startswith("single_launch"):
        q, k, v, _ = li.qkv(1, 4, 4, 16384, 64, li.BF16, seed=9, scaled=True)
        phi = "elu1" if path.endswith("elu1") else "relu1"
        call = lambda: gpu.la_causal_forward(dev(q), dev(k), dev(v), chunk=64, phi=phi)
    elif path == "noncausal_f32":
        q, k, v, _ = li.qkv(2, 8, 8, 4096, 64, li.F32, seed=10)
        call = lambda: gpu.la_forward(dev(q), dev(k), dev(v))
    elif path == "gqa_output":
        q, k, v, _ = li.qkv(1, 8, 2, 8192, 128, li.BF16, seed=11, scaled=True)
        call = lambda: gpu.la_causal_forward(dev(q), dev(k), dev(v))
    else:
        q, k, v, rng = li.qkv(3, 2, 2, 2000, 64, li.F32, seed=12, scaled=True)
        m = dev(np.stack([li.mask(2000, "random", rng=rng) for _ in range(3)]))
        call = lambda: gpu.la_prefix_mask_forward(dev(q), dev(k), dev(v), m, chunk=64)
    ref = li.from_torch(call())
    for _ in range(4):
        assert np.array_equal(li.from_torch(call()), ref), path


# ------------------------------------------------------- the workloads' sizes
@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
def test_noncausal_B2_H8_n4096_d64(gpu, dtype):
    q, k, v, _ = li.qkv(2, 8, 8, 4096, 64, dtype, seed=0)
    g = host(gpu.la_forward(dev(q), dev(k), dev(v)))
    check(g, oracle.forward(q, k, v), dtype, f"non-causal B2 H8 n4096 d64 {dtype}")


def test_causal_B8_H8_n2048_d64_bf16(gpu):
    q, k, v, _ = li.qkv(8, 8, 8, 2048, 64, li.BF16, seed=0, scaled=True)
    out, S, z = gpu.la_causal_forward(dev(q), dev(k), dev(v), chunk=64, want_state=True)
    ref, Sr, zr = oracle.causal(q, k, v, want_state=True)
    check(host(out), ref, li.BF16, "causal B8 H8 n2048 d64 bf16")
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=1e-4, atol=1e-5 * np.abs(Sr).max())
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=1e-5)


def test_causal_uniform_keys_closed_form_full_scale(gpu):
    """All key rows equal: out_i = mean(V_0..V_i) exactly (every key has the
    same weight), at the causal workload's full size."""
    B, H, n, d = 8, 8, 2048, 64
    q, _, v, rng = li.qkv(B, H, H, n, d, li.BF16, seed=3, scaled=True)
    row = li.as_dtype(rng.standard_normal(d, dtype=np.float32) / 8, li.BF16)
    k = np.broadcast_to(row, (B, H, n, d)).copy()
    g = host(gpu.la_causal_forward(dev(q), dev(k), dev(v)))
    vf = li.to_f32(v).astype(np.float64)
    want = np.cumsum(vf, axis=2) / np.arange(1, n + 1)[None, None, :, None]
    check(g, want, li.BF16, "causal uniform keys")


@pytest.mark.parametrize("kind", ["causal", "random"])
def test_prefix_B4_H8_n8192_d64_f32(gpu, kind):
    """At chunk 64, the launch configuration the benchmark times."""
    q, k, v, rng = li.qkv(4, 8, 8, 8192, 64, li.F32, seed=0, scaled=True)
    m = li.mask(8192, kind, rng=rng)
    g = host(gpu.la_prefix_mask_forward(dev(q), dev(k), dev(v), dev(m), chunk=64))
    check(g, oracle.prefix_mask(q, k, v, m), li.F32, f"prefix {kind} B4 H8 n8192 d64 f32")


def test_gqa_causal_B1_Hq32_Hkv8_n65536_d128_bf16(gpu):
    n = 65536
    q, k, v, rng = li.qkv(1, 32, 8, n, 128, li.BF16, seed=0, scaled=True)
    out, S, z = gpu.la_causal_forward(dev(q), dev(k), dev(v), want_state=True)
    rows = np.unique(np.concatenate([rng.choice(n, 62, replace=False), [0, 63, 64, n - 1]]))
    ref, Sr, zr = oracle.causal(q, k, v, rows=rows, want_state=True)
    g = host(out[:, :, rows.tolist()])
    check(g, ref, li.BF16, "GQA causal n65536 d128 (sampled rows)")
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=1e-4, atol=1e-5 * np.abs(Sr).max())
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=1e-5)


def test_decode_B128_Hq32_Hkv8_d128_256_steps(gpu):
    """Prefill a 4096-token prefix (state-only causal pass), then 256 decode
    steps for 128 sequences; the oracle follows 4 sampled sequences."""
    import torch
    B, Hq, Hkv, d, P, T = 128, 32, 8, 128, 4096, 256
    rng = np.random.default_rng(0)
    s = 1 / np.sqrt(d)
    kp = li.gaussian(rng, (B, Hkv, P, d), s, li.BF16)
    vp = li.gaussian(rng, (B, Hkv, P, d), s, li.BF16)
    steps = [tuple(li.gaussian(rng, shp, s, li.BF16) for shp in ((B, Hq, d), (B, Hkv, d), (B, Hkv, d)))
             for _ in range(T)]
    S, z = gpu.la_causal_forward(None, dev(kp), dev(vp), Hq=Hq)
    sample = np.array([0, 37, 90, 127])
    _, Sr, zr = oracle.causal(None, kp[sample], vp[sample], want_state=True, Hq=Hq)
    np.testing.assert_allclose(S.cpu().numpy()[sample], Sr, rtol=1e-4, atol=1e-5 * np.abs(Sr).max())
    worst = 0.0
    for t, (qs, ks, vs) in enumerate(steps):
        o = gpu.la_decode_step(dev(qs), dev(ks), dev(vs), S, z)
        ref = oracle.decode_step(qs[sample], ks[sample], vs[sample], Sr, zr)
        if t % 32 == 0 or t == T - 1:
            worst = max(worst, check(host(o)[sample], ref, li.BF16, f"decode step {t}"))
    torch.cuda.synchronize()
    np.testing.assert_allclose(S.cpu().numpy()[sample], Sr, rtol=1e-4, atol=1e-5 * np.abs(Sr).max())
    np.testing.assert_allclose(z.cpu().numpy()[sample], zr, rtol=1e-5)


# ------------------------------------------ the single-launch causal kernel
# bf16, d = 64, chunk 64, one query head per key/value head takes the
# single-launch path (segments of 8 chunks that wait on the aggregates of
# earlier segments); these cases cover ragged tails, one to many segments,
# and a deep wait chain (B3 H8 n4500: more than four earlier segments, whose
# aggregates are read in two batches).
SINGLE = [(1, 1, 1), (1, 1, 63), (1, 2, 64), (2, 1, 65), (1, 3, 257), (2, 4, 1000), (1, 2, 20000),
          (1, 8, 1500), (3, 8, 4500)]


@pytest.mark.parametrize("case", SINGLE, ids=lambda c: "B%d_H%d_n%d" % c)
def test_causal_single_launch_path(gpu, case):
    B, H, n = case
    q, k, v, _ = li.qkv(B, H, H, n, 64, li.BF16, seed=n, scaled=True)
    out, S, z = gpu.la_causal_forward(dev(q), dev(k), dev(v), chunk=64, want_state=True)
    ref, Sr, zr = oracle.causal(q, k, v, want_state=True)
    check(host(out), ref, li.BF16, f"single-launch causal B{B} H{H} n{n}")
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=1e-4, atol=1e-5 * np.abs(Sr).max())
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=1e-5)


def test_gqa_output_kernel_matches_general_path(gpu):
    """bf16, d = 128, GQA: chunk 32 (query heads of a chunk at once) and chunk
    64 (the general output kernel) both match the oracle."""
    q, k, v, _ = li.qkv(1, 8, 2, 1500, 128, li.BF16, seed=12, scaled=True)
    ref = oracle.causal(q, k, v)
    a = host(gpu.la_causal_forward(dev(q), dev(k), dev(v), chunk=32))
    b = host(gpu.la_causal_forward(dev(q), dev(k), dev(v), chunk=64))
    check(a, ref, li.BF16, "GQA chunk 32")
    check(b, ref, li.BF16, "GQA chunk 64")


@pytest.mark.parametrize("phi", ["relu1", "elu1"])
@pytest.mark.parametrize("shape", [(1, 1, 100), (2, 3, 1000), (1, 2, 20000)], ids=lambda c: "B%d_H%d_n%d" % c)
def test_causal_mha_d128_output_kernel(gpu, phi, shape):
    """bf16, d = 128, one query head per key/value head: the four-wave
    variant of the grouped-heads output kernel (chunk 32, a ragged tail, one
    to several chunks per workgroup); every row against the oracle, and the
    final state."""
    B, H, n = shape
    q, k, v, _ = li.qkv(B, H, H, n, 128, li.BF16, seed=31, scaled=True)
    out, S, z = gpu.la_causal_forward(dev(q), dev(k), dev(v), want_state=True, phi=phi)
    ref, Sr, zr = oracle.causal(q, k, v, want_state=True, phi=phi)
    check(host(out), ref, li.BF16, f"causal MHA d128 {phi} B{B} H{H} n{n}")
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=1e-2)
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=1e-2, atol=1e-2 * np.abs(Sr).max())


@pytest.mark.parametrize("phi", ["relu1", "elu1", "features"])
@pytest.mark.parametrize("shape", [(1, 8, 1, 300), (2, 16, 2, 1000), (1, 16, 2, 12000)],
                         ids=lambda c: "B%d_Hq%d_Hkv%d_n%d" % c)
def test_causal_gqa_r8_d128_output_kernel(gpu, phi, shape):
    """bf16, d = 128, eight query heads per key/value head: the grouped-heads
    output kernel with one wave per query head, its output tiles over the
    query tiles; every row against the oracle, and the final state.  With
    caller-applied features the inputs are softplus of Gaussian rows."""
    B, Hq, Hkv, n = shape
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, 128, li.BF16, seed=37, scaled=True)
    if phi == "features":
        sp = lambda x: np.log1p(np.exp(x))
        q, k = (li.as_dtype(sp(li.to_f32(x)).astype(np.float32), li.BF16) for x in (q, k))
    out, S, z = gpu.la_causal_forward(dev(q), dev(k), dev(v), want_state=True, phi=phi)
    ref, Sr, zr = oracle.causal(q, k, v, want_state=True, phi=phi)
    check(host(out), ref, li.BF16, f"causal GQA R8 d128 {phi} B{B} Hq{Hq} Hkv{Hkv} n{n}")
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=1e-2)
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=1e-2, atol=1e-2 * np.abs(Sr).max())


def test_single_launch_matches_three_launch_path(gpu):
    """The same inputs through chunk 64 (single launch) and chunk 32 (three
    launches) agree to bf16 rounding, and the workspace can be shared."""
    q, k, v, _ = li.qkv(4, 8, 8, 3000, 64, li.BF16, seed=4, scaled=True)
    a = host(gpu.la_causal_forward(dev(q), dev(k), dev(v), chunk=64))
    b = host(gpu.la_causal_forward(dev(q), dev(k), dev(v), chunk=32))
    c = host(gpu.la_causal_forward(dev(q), dev(k), dev(v), chunk=64))
    assert np.array_equal(a, c)
    check(a, b, li.BF16, "single vs three launches")


# ---------------------------------------------------------------------------
# The ELU + 1 feature map (la_*_phi with LA_PHI_ELU1): the general state,
# scan and output kernels and the decode kernels, against the oracle.
# ---------------------------------------------------------------------------
ELU_CASES = [
    (2, 3, 3, 1500, 64, 64),   # bf16: the single-launch causal kernel, 3 segments, ragged tail
    (1, 4, 1, 700, 128, 32),   # bf16: the GQA state and output kernels, four query heads per KV head
    (2, 4, 2, 333, 128, 0),    # ... two per KV head (default chunk 32)
    (1, 1, 1, 256, 16, 0),
    (2, 4, 2, 1000, 64, 64),
    (1, 2, 2, 300, 128, 32),
    (2, 3, 1, 129, 33, 0),
    (1, 4, 1, 65, 100, 0),
]


@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
@pytest.mark.parametrize("case", ELU_CASES, ids=_small_id)
def test_elu1_noncausal(gpu, dtype, case):
    B, Hq, Hkv, n, d, _ = case
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, dtype, seed=30, scaled=True)
    g = host(gpu.la_forward(dev(q), dev(k), dev(v), phi="elu1"))
    check(g, oracle.forward(q, k, v, phi="elu1"), dtype, f"elu1 forward {_small_id(case)} {dtype}")


@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
@pytest.mark.parametrize("case", ELU_CASES, ids=_small_id)
def test_elu1_causal_and_state(gpu, dtype, case):
    B, Hq, Hkv, n, d, chunk = case
    chunk = fit_chunk(gpu, dtype, d, chunk)
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, dtype, seed=31, scaled=True)
    out, S, z = gpu.la_causal_forward(dev(q), dev(k), dev(v), chunk=chunk, want_state=True, phi="elu1")
    ref, Sr, zr = oracle.causal(q, k, v, want_state=True, phi="elu1")
    check(host(out), ref, dtype, f"elu1 causal {_small_id(case)} {dtype}")
    tol = 1e-4 if dtype == li.F32 else 1e-2  # phi(K) rounded to the input dtype
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=tol, atol=tol * np.abs(Sr).max())
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=tol)


@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_elu1_causal_chunks_bf16(gpu, chunk):
    B, H, n, d = 1, 2, 700, 64
    chunk = fit_chunk(gpu, li.BF16, d, chunk)
    q, k, v, _ = li.qkv(B, H, H, n, d, li.BF16, seed=32, scaled=True)
    out = gpu.la_causal_forward(dev(q), dev(k), dev(v), chunk=chunk, phi="elu1")
    check(host(out), oracle.causal(q, k, v, phi="elu1"), li.BF16, f"elu1 causal chunk {chunk}")


@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
@pytest.mark.parametrize("d", [16, 64, 128, 33])
def test_elu1_decode_continues_causal(gpu, dtype, d):
    B, Hq, Hkv, n, T = 2, 4, 2, 48, 3
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, dtype, seed=33, scaled=True)
    full, Sf, zf = oracle.causal(q, k, v, want_state=True, phi="elu1")
    qd, kd, vd = dev(q), dev(k), dev(v)
    S, z = gpu.la_causal_forward(None, kd[:, :, :n - T].contiguous(), vd[:, :, :n - T].contiguous(), Hq=Hq,
                                 phi="elu1")
    for t in range(n - T, n):
        o = gpu.la_decode_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), S, z,
                               phi="elu1")
        check(host(o), full[:, :, t], dtype, f"elu1 decode d={d} step {t}")
    tol = 1e-4 if dtype == li.F32 else 1e-2
    np.testing.assert_allclose(S.cpu().numpy(), Sf, rtol=tol, atol=tol * np.abs(Sf).max())
    np.testing.assert_allclose(z.cpu().numpy(), zf, rtol=tol)


@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
def test_elu1_equals_relu1_on_positive_inputs(gpu, dtype):
    """On strictly positive Q and K both maps are x + 1: the ELU path (general
    kernels) and the relu + 1 path (the single-launch causal and the d = 64
    non-causal kernels) agree to the arithmetic's rounding."""
    import torch
    B, H, n, d = 2, 2, 1000, 64
    q, k, v, _ = li.qkv(B, H, H, n, d, dtype, seed=34, scaled=True)
    qd, kd, vd = dev(q).abs() + 0.01, dev(k).abs() + 0.01, dev(v)
    for f, kw in ((gpu.la_forward, {}), (gpu.la_causal_forward, {"chunk": 64})):
        a = f(qd, kd, vd, phi="elu1", **kw).float()
        b = f(qd, kd, vd, **kw).float()
        err = ((a - b).abs().amax(dim=-1) / b.abs().amax(dim=-1)).max().item()
        assert err < (1e-5 if dtype == li.F32 else 1e-2), (f.__name__, dtype, err)


# ---------------------------------------------------------------------------
# Per-batch prefix masks (la_prefix_mask_forward_batched, m [B, n]).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
@pytest.mark.parametrize("case,kinds", [
    ((3, 2, 1000, 64, 64), ("random", "causal", "full")),     # fp32: the chunk-64 state / output kernels
    ((2, 3, 300, 64, 0), ("causal", "random")),
    ((4, 1, 130, 33, 0), ("first", "random", "full", "causal")),
    ((2, 2, 257, 128, 32), ("random", "first")),
], ids=["B3H2n1000d64c64", "B2H3n300d64", "B4H1n130d33", "B2H2n257d128c32"])
def test_prefix_per_batch_masks(gpu, dtype, case, kinds):
    B, H, n, d, chunk = case
    chunk = fit_chunk(gpu, dtype, d, chunk) if chunk else 0
    q, k, v, rng = li.qkv(B, H, H, n, d, dtype, seed=50, scaled=True)
    m = np.stack([li.mask(n, kinds[b], rng=rng) for b in range(B)])
    g = host(gpu.la_prefix_mask_forward(dev(q), dev(k), dev(v), dev(m), chunk=chunk))
    check(g, oracle.prefix_mask(q, k, v, m), dtype, f"prefix per-batch {case} {kinds} {dtype}")


# ---------------------------------------------------------------------------
# The specialised paths at their size limits.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [131072, 131072 + 100])
def test_causal_at_the_single_launch_limit(gpu, n):
    """131072 tokens (256 segments per head) is the longest sequence the
    single-launch causal kernel takes; 100 more go to the general path.
    Sampled rows (the first, around segment boundaries, the last) against the
    oracle."""
    B, H, d = 1, 2, 64
    q, k, v, _ = li.qkv(B, H, H, n, d, li.BF16, seed=60, scaled=True)
    rows = np.array(sorted({0, 1, 511, 512, 513, 65535, 65536, n - 2, n - 1}), dtype=np.int64)
    g = host(gpu.la_causal_forward(dev(q), dev(k), dev(v), chunk=64))[:, :, rows]
    check(g, oracle.causal(q, k, v, rows=rows), li.BF16, f"causal n={n} sampled rows")


@pytest.mark.parametrize("dtype,n", [(li.BF16, 1 << 23), (li.F32, 1 << 22)])
def test_noncausal_at_the_single_path_limit(gpu, dtype, n):
    """The longest sequence of the d = 64 non-causal kernels (2^23 tokens for
    bf16, 2^22 for fp32), checked by a property that holds at any size: with
    every key row equal, every output row is the mean of V.  Inputs drawn on
    the GPU from a seeded generator (1 GiB per tensor)."""
    import torch
    d = 64
    tdt = torch.bfloat16 if dtype == li.BF16 else torch.float32
    gen = torch.Generator(device="cuda").manual_seed(61)
    q = torch.randn((1, 1, n, d), generator=gen, device="cuda").div_(8).to(tdt)
    v = torch.randn((1, 1, n, d), generator=gen, device="cuda").to(tdt)
    row = torch.randn((1, 1, 1, d), generator=gen, device="cuda").div_(8).to(tdt)
    k = row.expand(1, 1, n, d).contiguous()
    out = gpu.la_forward(q, k, v)
    want = v.double().mean(dim=2, keepdim=True)
    err = ((out.double() - want).abs().amax(dim=-1) / want.abs().amax(dim=-1)).max().item()
    print(f"non-causal n={n} {dtype}: row-wise rel err {err:.3e}", flush=True)
    assert err < TOL[dtype], err
