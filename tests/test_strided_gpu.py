"""GPU parity of the causal and sliding-window forms over sequence tables
(la_causal_forward_strided): strided [B, n, H, d] inputs (trim-transformer
0.1.0's [batch, seq, dim] layout) and packed sequences of different lengths
with cu_seqlens offsets (LinearTile 1.0.1, "Features": variable sequence
length with no padding).  Each sequence is compared with the oracle on that
sequence alone; metric and tolerances as in test_parity_gpu.py."""
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


def bnhd(x):
    """A [B, H, n, d] array stored as a [B, n, H, d] GPU buffer, returned as
    the [B, H, n, d] view of that buffer (strides n H d, d, H d, 1)."""
    return dev(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).transpose(1, 2)


@pytest.mark.parametrize("dtype,d", [(li.BF16, 64), (li.BF16, 128), (li.F32, 32), (li.F32, 64), (li.F32, 128),
                                     (li.BF16, 17)])
@pytest.mark.parametrize("window", [0, 45, 64, 200])
def test_bnhd_layout(gpu, dtype, d, window):
    B, Hq, Hkv, n = 2, 4, 2, 300
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, dtype, seed=300 + d, scaled=True)
    qd, kd, vd = bnhd(q), bnhd(k), bnhd(v)
    if dtype == li.F32 and d > 64 and window:  # the window form's tiles do not fit in LDS there
        with pytest.raises(gpu.LAError) as e:
            gpu.la_causal_forward_strided(qd, kd, vd, window=window)
        assert e.value.code == 4  # LA_ERR_UNSUPPORTED, nothing launched
        return
    assert qd.stride() == (n * Hq * d, d, Hq * d, 1)
    if window:
        out = gpu.la_causal_forward_strided(qd, kd, vd, window=window)
        ref = oracle.window(q, k, v, window)
    else:
        out, S, z = gpu.la_causal_forward_strided(qd, kd, vd, want_state=True)
        ref, Sr, zr = oracle.causal(q, k, v, want_state=True)
        rtol = 1e-4 if dtype == li.F32 else 1e-2
        np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=rtol)
        np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=rtol, atol=rtol * np.abs(Sr).max())
    assert out.stride() == qd.stride()
    check(host(out.contiguous()), ref, dtype, f"BNHD {dtype} d{d} window {window}")


LENGTHS = [1, 63, 64, 65, 300, 7, 1000, 0, 129]


@pytest.mark.parametrize("dtype,d", [(li.BF16, 64), (li.F32, 64), (li.BF16, 128), (li.F32, 32)])
@pytest.mark.parametrize("window", [0, 50])
@pytest.mark.parametrize("phi", ["relu1", "elu1"])
def test_packed_sequences(gpu, dtype, d, window, phi):
    """Packed [total, H, d] rows, sequence s at rows cu[s] .. cu[s+1] - 1
    (lengths from 0 to 1000, no padding); each sequence against the oracle
    on that sequence alone, and its final state (causal form)."""
    import torch
    Hq, Hkv = 4, 2
    cu = np.concatenate([[0], np.cumsum(LENGTHS)]).astype(np.int64)
    total = int(cu[-1])
    q, k, v, _ = li.qkv(1, Hq, Hkv, total, d, dtype, seed=310, scaled=True)
    # [1, H, total, d] -> packed [total, H, d]
    pk = lambda x: dev(np.ascontiguousarray(x[0].transpose(1, 0, 2)))
    qd, kd, vd = pk(q), pk(k), pk(v)
    cud = torch.from_numpy(cu).cuda()
    if window:
        out = gpu.la_causal_forward_strided(qd, kd, vd, cu_seqlens=cud, window=window, phi=phi)
    else:
        out, S, z = gpu.la_causal_forward_strided(qd, kd, vd, cu_seqlens=cud, want_state=True, phi=phi)
    g = host(out)  # [total, Hq, d]
    for s, L in enumerate(LENGTHS):
        if L == 0:
            continue
        a, b = int(cu[s]), int(cu[s + 1])
        sl = lambda x: np.ascontiguousarray(x[:, :, a:b])
        if window:
            ref = oracle.window(sl(q), sl(k), sl(v), window, phi=phi)
        else:
            ref, Sr, zr = oracle.causal(sl(q), sl(k), sl(v), want_state=True, phi=phi)
            rtol = 1e-4 if dtype == li.F32 else 1e-2
            np.testing.assert_allclose(z.cpu().numpy()[s], zr[0], rtol=rtol)
            np.testing.assert_allclose(S.cpu().numpy()[s], Sr[0], rtol=rtol, atol=rtol * np.abs(Sr).max())
        check(g[a:b].transpose(1, 0, 2)[None], ref, dtype, f"packed seq {s} (length {L}) {phi} window {window}")


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2)])
def test_packed_sequences_bad_table_is_reported(gpu, Hq, Hkv):
    """A decreasing cu_seqlens entry: that sequence is left alone, the rest are
    right, and la_workspace_status reports LA_ERR_RANGE (Hq == Hkv: the
    single-launch kernel; Hq > Hkv: the general kernels)."""
    import torch
    d = 64
    lengths = [100, 200, 50]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    total = int(cu[-1])
    q, k, v, _ = li.qkv(1, Hq, Hkv, total, d, li.BF16, seed=320, scaled=True)
    pk = lambda x: dev(np.ascontiguousarray(x[0].transpose(1, 0, 2)))
    bad = cu.copy()
    bad[2] = 50  # sequence 1 would run from 100 back to 50: inconsistent
    ws = gpu.new_workspace(gpu.la_workspace_bytes(gpu.LA_OP_SEQS, 3, Hq, Hkv, 300, d, gpu.LA_BF16, 0),
                           torch.device("cuda"))
    out = torch.zeros((total, Hq, d), dtype=torch.bfloat16, device="cuda")
    gpu.la_causal_forward_strided(pk(q), pk(k), pk(v), cu_seqlens=torch.from_numpy(bad).cuda(), max_len=300,
                                  out=out, ws=ws)
    assert gpu.la_workspace_status(ws) == gpu.LA_ERR_RANGE
    g = host(out)
    ref = oracle.causal(np.ascontiguousarray(q[:, :, :100]), np.ascontiguousarray(k[:, :, :100]),
                        np.ascontiguousarray(v[:, :, :100]))
    check(g[:100].transpose(1, 0, 2)[None], ref, li.BF16, "sequence 0 of a bad table")


def test_bnhd_B8_n2048_H8_d64_bf16(gpu):
    """The causal workload's size in trim-transformer's [batch, seq, dim]
    layout: sampled rows against the oracle, every row of an equal-keys input
    against the running mean of V."""
    B, H, n, d = 8, 8, 2048, 64
    q, k, v, rng = li.qkv(B, H, H, n, d, li.BF16, seed=330, scaled=True)
    g = host(gpu.la_causal_forward_strided(bnhd(q), bnhd(k), bnhd(v)).contiguous())
    rows = np.unique(np.concatenate([rng.choice(n, 40, replace=False), [0, 63, 64, n - 1]]))
    check(g[:, :, rows], oracle.causal(q, k, v, rows=rows), li.BF16, "BNHD B8 n2048 H8 d64 (sampled rows)")
    row = li.as_dtype(rng.standard_normal(d, dtype=np.float32) / 8, li.BF16)
    ke = np.ascontiguousarray(np.broadcast_to(row, (B, H, n, d)))
    ge = host(gpu.la_causal_forward_strided(bnhd(q), bnhd(ke), bnhd(v)).contiguous())
    want = np.cumsum(li.to_f32(v).astype(np.float64), axis=2) / np.arange(1, n + 1)[None, None, :, None]
    check(ge, want, li.BF16, "BNHD equal keys, every row")


def softplus(x):
    return np.log1p(np.exp(x))


# Hq == Hkv, bf16, d = 64: the single-launch causal kernel takes the table.
# Lengths over several 512-token segments, ragged tails, empty sequences.
LONG_LENGTHS = [1, 600, 0, 513, 64, 1100, 7, 2100, 512]


@pytest.mark.parametrize("phi", ["relu1", "elu1", "softplus"])
def test_packed_sequences_multi_segment(gpu, phi):
    """Packed [total, H, d] sequences of 0 .. 2100 tokens (up to five
    segments of the single-launch kernel, whose look-back stays inside each
    sequence): every sequence against the oracle on that sequence alone, its
    final state, and zero state for the empty one.  softplus: features the
    caller applies (phi="features")."""
    import torch
    H, d = 3, 64
    cu = np.concatenate([[0], np.cumsum(LONG_LENGTHS)]).astype(np.int64)
    total = int(cu[-1])
    q, k, v, _ = li.qkv(1, H, H, total, d, li.BF16, seed=340, scaled=True)
    if phi == "softplus":
        fq = li.as_dtype(softplus(li.to_f32(q)).astype(np.float32), li.BF16)
        fk = li.as_dtype(softplus(li.to_f32(k)).astype(np.float32), li.BF16)
        call_phi, ref_phi = "features", softplus
    else:
        fq, fk, call_phi, ref_phi = q, k, phi, phi
    pk = lambda x: dev(np.ascontiguousarray(x[0].transpose(1, 0, 2)))
    cud = torch.from_numpy(cu).cuda()
    out, S, z = gpu.la_causal_forward_strided(pk(fq), pk(fk), pk(v), cu_seqlens=cud, want_state=True, phi=call_phi)
    g = host(out)
    S, z = S.cpu().numpy(), z.cpu().numpy()
    for s, L in enumerate(LONG_LENGTHS):
        if L == 0:
            assert not S[s].any() and not z[s].any(), "an empty sequence's state must be zero"
            continue
        a, b = int(cu[s]), int(cu[s + 1])
        sl = lambda x: np.ascontiguousarray(x[:, :, a:b])
        ref, Sr, zr = oracle.causal(sl(q), sl(k), sl(v), want_state=True, phi=ref_phi)
        np.testing.assert_allclose(z[s], zr[0], rtol=1e-2)
        np.testing.assert_allclose(S[s], Sr[0], rtol=1e-2, atol=1e-2 * np.abs(Sr).max())
        check(g[a:b].transpose(1, 0, 2)[None], ref, li.BF16, f"packed seq {s} (length {L}) {phi}")


def test_fused_qkv_buffer_layout(gpu):
    """q, k, v as slices of one [B, n, 3, H, d] projection buffer (token
    stride 3 H d) and out a slice of another: B2 n1500 H4 d64 bf16, every row
    and the final state against the oracle."""
    import torch
    B, H, n, d = 2, 4, 1500, 64
    q, k, v, _ = li.qkv(B, H, H, n, d, li.BF16, seed=350, scaled=True)
    buf = np.stack([x.transpose(0, 2, 1, 3) for x in (q, k, v)], axis=2)  # [B, n, 3, H, d]
    bd = dev(np.ascontiguousarray(buf))
    views = [bd[:, :, i].transpose(1, 2) for i in range(3)]  # [B, H, n, d] views
    ob = torch.zeros_like(bd)
    out = ob[:, :, 0].transpose(1, 2)
    assert out.stride() == (n * 3 * H * d, d, 3 * H * d, 1)
    _, S, z = gpu.la_causal_forward_strided(*views, out=out, want_state=True)
    ref, Sr, zr = oracle.causal(q, k, v, want_state=True)
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=1e-2)
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=1e-2, atol=1e-2 * np.abs(Sr).max())
    check(host(out.contiguous()), ref, li.BF16, "fused QKV buffer B2 n1500 H4 d64")
    assert not host(ob[:, :, 1:].contiguous()).any(), "nothing may be written outside out's rows"


def test_unaligned_token_stride_takes_general_path(gpu):
    """Rows of 68 elements (136 bytes, not a multiple of 16): the table goes
    to the general kernels; same result as the oracle."""
    B, H, n, d = 1, 2, 700, 64
    q, k, v, _ = li.qkv(B, H, H, n, d, li.BF16, seed=360, scaled=True)

    def padded(x):  # [B, H, n, d] stored as [B, n, H, 68]
        p = np.zeros((B, n, H, 68), dtype=x.dtype)
        p[..., :d] = x.transpose(0, 2, 1, 3)
        return dev(p)[..., :d].transpose(1, 2)

    qd, kd, vd = padded(q), padded(k), padded(v)
    import torch
    ob = torch.zeros((B, n, H, 68), dtype=torch.bfloat16, device="cuda")
    out = ob[..., :d].transpose(1, 2)
    gpu.la_causal_forward_strided(qd, kd, vd, out=out)
    check(host(out.contiguous()), oracle.causal(q, k, v), li.BF16, "token stride 136 bytes")


@pytest.mark.parametrize("w", [50, 64, 300, 512])
def test_packed_window_single_launch(gpu, w):
    """The sliding window over packed sequences of 0 .. 2100 tokens with one
    query head per key/value head (the single-launch window kernel through
    the table): every sequence against the oracle on that sequence alone."""
    import torch
    H, d = 3, 64
    cu = np.concatenate([[0], np.cumsum(LONG_LENGTHS)]).astype(np.int64)
    total = int(cu[-1])
    q, k, v, _ = li.qkv(1, H, H, total, d, li.BF16, seed=370 + w, scaled=True)
    pk = lambda x: dev(np.ascontiguousarray(x[0].transpose(1, 0, 2)))
    out = gpu.la_causal_forward_strided(pk(q), pk(k), pk(v), cu_seqlens=torch.from_numpy(cu).cuda(), window=w)
    g = host(out)
    for s, L in enumerate(LONG_LENGTHS):
        if L == 0:
            continue
        a, b = int(cu[s]), int(cu[s + 1])
        sl = lambda x: np.ascontiguousarray(x[:, :, a:b])
        check(g[a:b].transpose(1, 0, 2)[None], oracle.window(sl(q), sl(k), sl(v), w), li.BF16,
              f"packed window w={w} seq {s} (length {L})")


def test_bnhd_window_single_launch(gpu):
    """[B, n, H, d] rows with a 200-token window, H = Hkv = 4, n = 1300."""
    B, H, n, d, w = 2, 4, 1300, 64, 200
    q, k, v, _ = li.qkv(B, H, H, n, d, li.BF16, seed=380, scaled=True)
    out = gpu.la_causal_forward_strided(bnhd(q), bnhd(k), bnhd(v), window=w)
    check(host(out.contiguous()), oracle.window(q, k, v, w), li.BF16, "BNHD window w200")
