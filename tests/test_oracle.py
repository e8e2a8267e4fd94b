"""Pins for the fp64 oracle, run on the CPU.

Each test checks the oracle against something other than itself: values the
pages print for their worked examples (tests/golden/), closed forms,
invariants of the method, or an independent O(n^2) brute force written here
with numpy.  They are chosen so that a plausible slip in the oracle (a
dropped feature map, a transposed state, an exclusive instead of inclusive
causal prefix, a wrong head mapping, an off-by-one in the prefix mask, a
decode step that reads before it writes) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import la_inputs as li
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Independent brute force (pairwise weights), numpy fp64.  Not the oracle's
# algorithm: it never forms the d x d state.
# ---------------------------------------------------------------------------
def _relu1(x):
    return np.maximum(x, 0.0) + 1.0


def brute_normalised(q, k, v, causal):
    q, k, v = (li.to_f32(x).astype(np.float64) for x in (q, k, v))
    B, Hq, n, d = q.shape
    R = Hq // k.shape[1]
    out = np.empty_like(q)
    for b in range(B):
        for h in range(Hq):
            g = h // R
            w = _relu1(q[b, h]) @ _relu1(k[b, g]).T  # w[i, j]
            if causal:
                w = np.tril(w)
            out[b, h] = (w @ v[b, g]) / w.sum(axis=1, keepdims=True)
    return out


def brute_prefix(q, k, v, mask2d_zeroed):
    """out_i = sum_j [not zeroed(i, j)] (Q_i . K_j) V_j."""
    q, k, v = (li.to_f32(x).astype(np.float64) for x in (q, k, v))
    keep = ~np.asarray(mask2d_zeroed, dtype=bool)
    out = np.empty_like(q)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            a = (q[b, h] @ k[b, h].T) * keep
            out[b, h] = a @ v[b, h]
    return out


def mask2d_from_m(m):
    """Two-dimensional mask of a prefix mask: element (i, j) is zeroed iff j > m_i."""
    m = np.asarray(m)
    n = m.size
    return np.arange(n)[None, :] > m[:, None]


def rel_rows(a, b):
    """Largest row-wise max-norm relative error."""
    num = np.abs(a - b).max(axis=-1)
    den = np.abs(b).max(axis=-1)
    return float((num / np.maximum(den, 1e-300)).max())


# ---------------------------------------------------------------------------
# Worked examples printed on the nx_f32_linear_attention.nx page.
# ---------------------------------------------------------------------------
def test_gate1_uniform_keys_gives_mean_of_v():
    g = _golden("nx_hand_cases.json")
    q, k, v = li.hand_case("zero")
    assert np.array_equal(v[0, 0], np.array(g["V"], dtype=np.float32))
    out = oracle.forward(q, k, v)[0, 0]
    np.testing.assert_allclose(out, np.array(g["cases"]["zero"]["out"], float), rtol=0, atol=1e-12)


def test_gate2_identity_state_and_output():
    g = _golden("nx_hand_cases.json")["cases"]["identity"]
    q, k, v = li.hand_case("identity")
    assert np.array_equal(q[0, 0], np.array(g["Q"], dtype=np.float32))
    out = oracle.forward(q, k, v)[0, 0]
    want = np.array(g["out_num"], float) / g["out_den"]
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-12)
    # The state after all keys (the causal sweep's final state) is the page's S and z.
    _, S, z = oracle.causal(q, k, v, want_state=True)
    np.testing.assert_array_equal(S[0, 0], np.array(g["S"], float))
    np.testing.assert_array_equal(z[0, 0], np.array(g["z"], float))


def test_hand_cases_causal():
    """Causal reading of the two gates: query 0 sees only key 0 (so it returns
    V_0 whatever its weight); query 1 sees both keys, as in the non-causal gate."""
    q, k, v = li.hand_case("zero")
    np.testing.assert_allclose(oracle.causal(q, k, v)[0, 0], [[2, 4], [4, 6]], atol=1e-12)
    q, k, v = li.hand_case("identity")
    np.testing.assert_allclose(oracle.causal(q, k, v)[0, 0],
                               [[2, 4], [38 / 9, 56 / 9]], atol=1e-12)


# ---------------------------------------------------------------------------
# Closed forms and invariants.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
@pytest.mark.parametrize("kind", ["equal_rows", "nonpositive"])
def test_uniform_key_weights_closed_form(dtype, kind):
    """If phi(K_j) is the same for every j, every visible key gets the same
    weight: non-causal out_i = mean(V); causal out_i = mean(V_0..V_i)."""
    B, Hq, Hkv, n, d = 2, 4, 2, 300, 16
    rng = np.random.default_rng(5)
    q = li.as_dtype(rng.standard_normal((B, Hq, n, d), dtype=np.float32), dtype)
    v = li.as_dtype(rng.standard_normal((B, Hkv, n, d), dtype=np.float32), dtype)
    if kind == "equal_rows":
        row = rng.standard_normal(d, dtype=np.float32)
        k = np.broadcast_to(row, (B, Hkv, n, d)).copy()
    else:
        k = -np.abs(rng.standard_normal((B, Hkv, n, d), dtype=np.float32))
    k = li.as_dtype(k, dtype)
    vf = li.to_f32(v).astype(np.float64)
    R = Hq // Hkv
    mean_all = np.repeat(vf.mean(axis=2, keepdims=True), R, axis=1)
    mean_prefix = np.repeat(np.cumsum(vf, axis=2) / np.arange(1, n + 1)[None, None, :, None], R, axis=1)
    np.testing.assert_allclose(oracle.forward(q, k, v), np.broadcast_to(mean_all, (B, Hq, n, d)),
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.causal(q, k, v), mean_prefix, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("shape", [(1, 1, 1, 17, 1), (2, 4, 2, 33, 3), (1, 2, 2, 40, 8), (1, 6, 3, 19, 5)])
def test_normalised_forms_match_brute_force(seed, shape):
    B, Hq, Hkv, n, d = shape
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, li.F32, seed=seed)
    np.testing.assert_allclose(oracle.forward(q, k, v), brute_normalised(q, k, v, False),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.causal(q, k, v), brute_normalised(q, k, v, True),
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 3])
@pytest.mark.parametrize("kind", ["random", "causal", "full", "first"])
def test_prefix_mask_matches_brute_force(seed, kind):
    B, H, n, d = 2, 3, 37, 6
    q, k, v, rng = li.qkv(B, H, H, n, d, li.F32, seed=seed)
    m = li.mask(n, kind, rng=rng)
    got = oracle.prefix_mask(q, k, v, m)
    np.testing.assert_allclose(got, brute_prefix(q, k, v, mask2d_from_m(m)), rtol=1e-11, atol=1e-11)


def test_prefix_mask_page_example():
    """m = [2, 0, 1] against the page's own two-dimensional mask."""
    g = _golden("trim_mask_example.json")
    m = np.array(g["m"], dtype=np.int64)
    page_mask = np.array(g["mask2d_true_means_zeroed"], dtype=bool)
    assert np.array_equal(mask2d_from_m(m), page_mask)
    q, k, v, _ = li.qkv(1, 2, 2, 3, 4, li.F32, seed=11)
    np.testing.assert_allclose(oracle.prefix_mask(q, k, v, m), brute_prefix(q, k, v, page_mask),
                               rtol=1e-12, atol=1e-12)
    # arange(n) is the causal mask: its 2-D form keeps exactly the lower triangle.
    assert np.array_equal(~mask2d_from_m(li.mask(5, "causal")), np.tril(np.ones((5, 5), bool)))


def test_cross_form_identities():
    """Causal normalised = num/den of the prefix form with m = arange(n) on
    (phi(Q), phi(K), [V | 1]); non-causal = the same with m_i = n - 1."""
    B, Hq, n, d = 2, 2, 29, 5
    q, k, v, _ = li.qkv(B, Hq, Hq, n, d, li.F32, seed=4)
    # inputs on a 2^-8 grid, so that phi(x) = relu(x) + 1 is exact in fp32
    q, k = (np.round(x * 256) / 256 for x in (q, k))
    q, k = q.astype(np.float32), k.astype(np.float32)
    pad = lambda x: np.concatenate([x, np.zeros(x.shape[:-1] + (1,), np.float32)], -1)
    fq = pad(_relu1(q).astype(np.float32))
    fk = pad(_relu1(k).astype(np.float32))
    v1 = np.concatenate([v, np.ones(v.shape[:-1] + (1,), np.float32)], -1)
    for kind, ref in (("causal", oracle.causal(q, k, v)), ("full", oracle.forward(q, k, v))):
        nd = oracle.prefix_mask(fq, fk, v1, li.mask(n, kind))
        np.testing.assert_allclose(nd[..., :d] / nd[..., d:], ref, rtol=1e-12, atol=1e-13)


def test_permutation_and_prefix_invariance():
    B, Hq, Hkv, n, d = 1, 2, 1, 50, 7
    q, k, v, rng = li.qkv(B, Hq, Hkv, n, d, li.F32, seed=9)
    perm = rng.permutation(n)
    np.testing.assert_allclose(oracle.forward(q, k[:, :, perm], v[:, :, perm]),
                               oracle.forward(q, k, v), rtol=1e-12, atol=1e-13)
    full = oracle.causal(q, k, v)
    for n2 in (1, 17, 49):
        part = oracle.causal(q[:, :, :n2].copy(), k[:, :, :n2].copy(), v[:, :, :n2].copy())
        np.testing.assert_allclose(part, full[:, :, :n2], rtol=1e-13, atol=1e-14)


def test_linear_in_v():
    B, Hq, n, d = 1, 1, 40, 6
    q, k, v1, rng = li.qkv(B, Hq, Hq, n, d, li.F32, seed=12)
    v2 = rng.standard_normal(v1.shape, dtype=np.float32)
    for f in (oracle.forward, oracle.causal):
        lhs = f(q, k, (v1 + 2 * v2).astype(np.float32))
        rhs = f(q, k, v1) + 2 * f(q, k, v2)
        np.testing.assert_allclose(lhs, rhs, rtol=1e-6, atol=1e-6)


def test_d1_output_does_not_depend_on_q():
    """With d = 1 phi(q) cancels: out_i = sum_j phi(k_j) v_j / sum_j phi(k_j)."""
    B, H, n = 1, 1, 64
    _, k, v, rng = li.qkv(B, H, H, n, 1, li.F32, seed=2)
    q1 = rng.standard_normal((B, H, n, 1), dtype=np.float32)
    q2 = 10 * rng.standard_normal((B, H, n, 1), dtype=np.float32)
    pk = _relu1(k[0, 0, :, 0].astype(np.float64))
    vv = v[0, 0, :, 0].astype(np.float64)
    want_causal = np.cumsum(pk * vv) / np.cumsum(pk)
    for q in (q1, q2):
        np.testing.assert_allclose(oracle.forward(q, k, v)[0, 0, :, 0],
                                   np.full(n, want_causal[-1]), rtol=1e-12)
        np.testing.assert_allclose(oracle.causal(q, k, v)[0, 0, :, 0], want_causal, rtol=1e-12)


def test_outputs_are_convex_combinations():
    B, Hq, n, d = 2, 2, 120, 8
    q, k, v, _ = li.qkv(B, Hq, Hq, n, d, li.F32, seed=21, scaled=True)
    vf = v.astype(np.float64)
    out = oracle.forward(q, k, v)
    assert np.all(out <= vf.max(axis=2, keepdims=True) + 1e-12)
    assert np.all(out >= vf.min(axis=2, keepdims=True) - 1e-12)
    outc = oracle.causal(q, k, v)
    assert np.all(outc <= np.maximum.accumulate(vf, axis=2) + 1e-12)
    assert np.all(outc >= np.minimum.accumulate(vf, axis=2) - 1e-12)


def test_gqa_equals_repeated_kv_heads():
    B, Hq, Hkv, n, d = 2, 6, 2, 31, 4
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, li.F32, seed=8)
    kr = np.repeat(k, Hq // Hkv, axis=1)  # head h -> kv head h // (Hq/Hkv)
    vr = np.repeat(v, Hq // Hkv, axis=1)
    np.testing.assert_array_equal(oracle.forward(q, k, v), oracle.forward(q, kr, vr))
    np.testing.assert_array_equal(oracle.causal(q, k, v), oracle.causal(q, kr, vr))


def test_bf16_inputs_are_widened_exactly():
    q, k, v, _ = li.qkv(1, 2, 1, 23, 9, li.BF16, seed=3)
    qf, kf, vf = (li.to_f32(x) for x in (q, k, v))
    np.testing.assert_array_equal(oracle.forward(q, k, v), oracle.forward(qf, kf, vf))
    np.testing.assert_array_equal(oracle.causal(q, k, v), oracle.causal(qf, kf, vf))
    m = li.mask(23, "random", seed=1)
    q1, qf1 = q[:, :1].copy(), qf[:, :1].copy()
    np.testing.assert_array_equal(oracle.prefix_mask(q1, k, v, m), oracle.prefix_mask(qf1, kf, vf, m))


def test_row_selection_matches_full_output():
    B, Hq, Hkv, n, d = 2, 4, 2, 45, 5
    q, k, v, rng = li.qkv(B, Hq, Hkv, n, d, li.F32, seed=13)
    rows = np.array([0, 7, 8, 30, 44])
    np.testing.assert_array_equal(oracle.forward(q, k, v, rows=rows), oracle.forward(q, k, v)[:, :, rows])
    np.testing.assert_array_equal(oracle.causal(q, k, v, rows=rows), oracle.causal(q, k, v)[:, :, rows])
    qh, kh, vh = q[:, :2].copy(), k[:, :2].copy(), v[:, :2].copy()
    m = li.mask(n, "random", rng=rng)
    np.testing.assert_array_equal(oracle.prefix_mask(qh, kh, vh, m, rows=rows),
                                  oracle.prefix_mask(qh, kh, vh, m)[:, :, rows])


@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
def test_decode_steps_continue_the_causal_pass(dtype):
    """Causal over n tokens == causal state over the first n - T tokens, then T
    decode steps (each adds its token before its queries read the state)."""
    B, Hq, Hkv, n, d, T = 2, 4, 2, 24, 6, 5
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, dtype, seed=17)
    full, S_full, z_full = oracle.causal(q, k, v, want_state=True)
    _, S, z = oracle.causal(None, k[:, :, :n - T].copy(), v[:, :, :n - T].copy(), want_state=True, Hq=Hq)
    for t in range(n - T, n):
        out = oracle.decode_step(q[:, :, t].copy(), k[:, :, t].copy(), v[:, :, t].copy(), S, z)
        np.testing.assert_allclose(out, full[:, :, t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, S_full, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z, z_full, rtol=1e-12, atol=1e-12)


def test_decode_step_matches_brute_force():
    """One decode step from an empty state over a single token equals the
    brute-force causal output of a length-1 sequence (which is V_0)."""
    B, Hq, Hkv, d = 3, 4, 2, 5
    q, k, v, _ = li.qkv(B, Hq, Hkv, 1, d, li.F32, seed=19)
    S = np.zeros((B, Hkv, d, d)); z = np.zeros((B, Hkv, d))
    out = oracle.decode_step(q[:, :, 0].copy(), k[:, :, 0].copy(), v[:, :, 0].copy(), S, z)
    np.testing.assert_allclose(out, np.repeat(v[:, :, 0], Hq // Hkv, axis=1), rtol=1e-12)
    np.testing.assert_allclose(z, _relu1(k[:, :, 0].astype(np.float64)), rtol=0)


def test_bf16_rounding_helper_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3, 0.0, -0.0], dtype=np.float32)
    bits = li.f32_to_bf16_bits(x)
    back = li.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa -> 1.0
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: even -> 1 + 2^-6
    np.testing.assert_array_equal(back[:4], np.array([1.0, 1.0, 1.015625, -2.5], np.float32))
    assert abs(back[4] - 3.0e-3) <= 3.0e-3 * 2 ** -8
    assert np.array_equal(bits[5:], np.array([0x0000, 0x8000], np.uint16))


# ---------------------------------------------------------------------------
# The ELU + 1 feature map (LinearTile 1.0.1, "How It Works"): phi(x) = x + 1
# for x > 0 and exp(x) otherwise (ELU with alpha = 1).
# ---------------------------------------------------------------------------
def _elu1(x):
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def brute_normalised_elu1(q, k, v, causal):
    q, k, v = (li.to_f32(x).astype(np.float64) for x in (q, k, v))
    B, Hq, n, d = q.shape
    R = Hq // k.shape[1]
    out = np.empty_like(q)
    for b in range(B):
        for h in range(Hq):
            w = _elu1(q[b, h]) @ _elu1(k[b, h // R]).T
            if causal:
                w = np.tril(w)
            out[b, h] = (w @ v[b, h // R]) / w.sum(axis=1, keepdims=True)
    return out


def test_elu1_feature_map_at_chosen_points():
    """d = 1 (phi(q) cancels): out_i = sum_{j<=i} phi(k_j) v_j / sum_{j<=i} phi(k_j),
    with phi written out by hand at k = 0, -1, 1, -2.5, 3 (the branches meet
    at 0: ELU(0) + 1 = 1)."""
    import math
    kv = [0.0, -1.0, 1.0, -2.5, 3.0]
    vv = [1.0, 2.0, -3.0, 4.0, 0.5]
    phis = [1.0, math.exp(-1.0), 2.0, math.exp(-2.5), 4.0]
    k = np.array(kv, dtype=np.float32).reshape(1, 1, 5, 1)
    v = np.array(vv, dtype=np.float32).reshape(1, 1, 5, 1)
    q = np.array([0.3, -2.0, 5.0, -0.1, 1.0], dtype=np.float32).reshape(1, 1, 5, 1)
    want = [sum(p * x for p, x in zip(phis[:i + 1], vv[:i + 1])) / sum(phis[:i + 1]) for i in range(5)]
    np.testing.assert_allclose(oracle.causal(q, k, v, phi="elu1")[0, 0, :, 0], want, rtol=1e-12)
    np.testing.assert_allclose(oracle.forward(q, k, v, phi="elu1")[0, 0, :, 0], np.full(5, want[-1]), rtol=1e-12)


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("shape", [(1, 1, 1, 17, 1), (2, 4, 2, 33, 3), (1, 6, 3, 19, 5)])
def test_elu1_forms_match_brute_force(seed, shape):
    B, Hq, Hkv, n, d = shape
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, li.F32, seed=seed)
    np.testing.assert_allclose(oracle.forward(q, k, v, phi="elu1"), brute_normalised_elu1(q, k, v, False),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.causal(q, k, v, phi="elu1"), brute_normalised_elu1(q, k, v, True),
                               rtol=1e-12, atol=1e-12)


def test_elu1_equals_relu1_on_positive_inputs():
    """For x > 0 both maps are x + 1, so strictly positive Q and K give the
    same outputs under either; mixed signs do not."""
    B, Hq, Hkv, n, d = 1, 2, 1, 40, 6
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, li.F32, seed=4)
    qp, kp = np.abs(q) + 0.01, np.abs(k) + 0.01
    for f in (oracle.forward, oracle.causal):
        np.testing.assert_allclose(f(qp, kp, v, phi="elu1"), f(qp, kp, v), rtol=1e-12, atol=1e-12)
        assert rel_rows(f(q, k, v, phi="elu1"), f(q, k, v)) > 1e-3


def test_elu1_equal_keys_give_mean_of_v():
    """Every key row equal: all weights of a query are equal whatever phi is,
    so the non-causal output is mean(V) and the causal one the running mean."""
    B, H, n, d = 1, 1, 30, 4
    q, _, v, rng = li.qkv(B, H, H, n, d, li.F32, seed=5)
    k = np.repeat(rng.standard_normal((1, 1, 1, d), dtype=np.float32), n, axis=2)
    vf = v.astype(np.float64)
    np.testing.assert_allclose(oracle.forward(q, k, v, phi="elu1"),
                               np.broadcast_to(vf.mean(axis=2, keepdims=True), vf.shape), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.causal(q, k, v, phi="elu1"),
                               np.cumsum(vf, axis=2) / np.arange(1, n + 1)[None, None, :, None], rtol=1e-12, atol=1e-12)


def test_elu1_decode_steps_continue_the_causal_pass():
    B, Hq, Hkv, n, d, T = 2, 4, 2, 20, 5, 3
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, li.F32, seed=6)
    full, Sf, zf = oracle.causal(q, k, v, want_state=True, phi="elu1")
    _, S, z = oracle.causal(None, k[:, :, :n - T], v[:, :, :n - T], want_state=True, Hq=Hq, phi="elu1")
    for t in range(n - T, n):
        o = oracle.decode_step(q[:, :, t].copy(), k[:, :, t].copy(), v[:, :, t].copy(), S, z, phi="elu1")
        np.testing.assert_allclose(o, full[:, :, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, Sf, rtol=1e-12)
    np.testing.assert_allclose(z, zf, rtol=1e-12)


# ---------------------------------------------------------------------------
# Per-batch prefix masks m [B, n]: batch b's queries use row b.
# ---------------------------------------------------------------------------
def test_prefix_mask_per_batch_matches_brute_force():
    B, H, n, d = 3, 2, 23, 3
    q, k, v, rng = li.qkv(B, H, H, n, d, li.F32, seed=40)
    m = np.stack([li.mask(n, kind, rng=rng) for kind in ("random", "causal", "first")])
    out = oracle.prefix_mask(q, k, v, m)
    for b in range(B):
        want = brute_prefix(q[b:b + 1], k[b:b + 1], v[b:b + 1], mask2d_from_m(m[b]))
        np.testing.assert_allclose(out[b:b + 1], want, rtol=1e-12, atol=1e-12)
    # rows differ, so the outputs differ from the shared-mask form with row 0
    assert not np.allclose(out, oracle.prefix_mask(q, k, v, m[0]))


def test_prefix_mask_per_batch_equal_rows_is_shared():
    B, H, n, d = 2, 3, 31, 4
    q, k, v, rng = li.qkv(B, H, H, n, d, li.F32, seed=41)
    m = li.mask(n, "random", rng=rng)
    np.testing.assert_array_equal(oracle.prefix_mask(q, k, v, np.tile(m, (B, 1))), oracle.prefix_mask(q, k, v, m))


# ---------------------------------------------------------------------------
# A feature map of the caller's choice (LinearTile 1.0.1, "Features": phi
# replaceable at will): given to the oracle as an fp64 function, or applied
# to q and k beforehand ("features").  Pinned by what holds for every
# positive map: equal keys give the mean of V, d = 1 does not depend on Q,
# the pairwise brute force with that map's weights.
# ---------------------------------------------------------------------------
def _softplus(x):
    return np.log1p(np.exp(x))


def _sq1(x):  # 1 + x^2: exact in fp32 on a 2^-4 grid of small values
    return 1.0 + x * x


def brute_normalised_fn(q, k, v, causal, fn):
    q, k, v = (li.to_f32(x).astype(np.float64) for x in (q, k, v))
    B, Hq, n, d = q.shape
    R = Hq // k.shape[1]
    out = np.empty_like(q)
    for b in range(B):
        for h in range(Hq):
            g = h // R
            w = fn(q[b, h]) @ fn(k[b, g]).T
            if causal:
                w = np.tril(w)
            out[b, h] = (w @ v[b, g]) / w.sum(axis=1, keepdims=True)
    return out


@pytest.mark.parametrize("fn", [_softplus, np.exp, _sq1], ids=["softplus", "exp", "sq1"])
@pytest.mark.parametrize("shape", [(1, 1, 1, 17, 1), (2, 4, 2, 23, 3), (1, 2, 2, 19, 6)])
def test_callback_feature_map_matches_brute_force(fn, shape):
    B, Hq, Hkv, n, d = shape
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, li.F32, seed=5, scaled=True)
    assert rel_rows(oracle.forward(q, k, v, phi=fn), brute_normalised_fn(q, k, v, False, fn)) < 1e-12
    assert rel_rows(oracle.causal(q, k, v, phi=fn), brute_normalised_fn(q, k, v, True, fn)) < 1e-12


def test_callback_relu1_equals_the_built_in_map():
    q, k, v, _ = li.qkv(2, 4, 2, 40, 8, li.F32, seed=6)
    assert np.array_equal(oracle.forward(q, k, v, phi=_relu1), oracle.forward(q, k, v))
    assert np.array_equal(oracle.causal(q, k, v, phi=_relu1), oracle.causal(q, k, v))


@pytest.mark.parametrize("fn", [_softplus, np.exp], ids=["softplus", "exp"])
def test_callback_equal_keys_give_mean_of_v(fn):
    """Every key row equal: every key has the same weight phi(Q_i) . phi(k)
    whatever the positive map, so the outputs are the (running) mean of V."""
    B, H, n, d = 1, 2, 30, 4
    q, _, v, rng = li.qkv(B, H, H, n, d, li.F32, seed=7)
    k = np.broadcast_to(rng.standard_normal(d, dtype=np.float32), (B, H, n, d)).copy()
    vf = v.astype(np.float64)
    nc = oracle.forward(q, k, v, phi=fn)
    assert np.allclose(nc, np.broadcast_to(vf.mean(axis=2, keepdims=True), nc.shape), rtol=1e-12, atol=1e-12)
    run = np.cumsum(vf, axis=2) / np.arange(1, n + 1)[None, None, :, None]
    assert np.allclose(oracle.causal(q, k, v, phi=fn), run, rtol=1e-12, atol=1e-12)


def test_callback_d1_output_does_not_depend_on_q():
    """d = 1: phi(q_i) cancels between numerator and denominator."""
    q1, k, v, _ = li.qkv(1, 1, 1, 25, 1, li.F32, seed=8)
    q2 = (q1 * 3.0 + 1.0).astype(np.float32)
    a = oracle.causal(q1, k, v, phi=_softplus)
    b = oracle.causal(q2, k, v, phi=_softplus)
    assert np.allclose(a, b, rtol=1e-13, atol=0)
    pk = _softplus(k[0, 0, :, 0].astype(np.float64))
    want = np.cumsum(pk * v[0, 0, :, 0]) / np.cumsum(pk)
    assert np.allclose(a[0, 0, :, 0], want, rtol=1e-13)


def test_features_mode_equals_the_map_applied_by_the_oracle():
    """q and k mapped beforehand ("features") give what the oracle gives
    applying the same map itself (1 + x^2 on a 2^-4 grid is exact in fp32),
    in every normalised form and the decode step."""
    B, Hq, Hkv, n, d = 2, 4, 2, 21, 5
    rng = np.random.default_rng(9)
    grid = lambda shape: (rng.integers(-24, 25, size=shape) / 16.0).astype(np.float32)
    q, k, v = grid((B, Hq, n, d)), grid((B, Hkv, n, d)), grid((B, Hkv, n, d))
    fq, fk = _sq1(q).astype(np.float32), _sq1(k).astype(np.float32)
    assert np.array_equal(oracle.forward(fq, fk, v, phi="features"), oracle.forward(q, k, v, phi=_sq1))
    o1, S1, z1 = oracle.causal(fq, fk, v, phi="features", want_state=True)
    o2, S2, z2 = oracle.causal(q, k, v, phi=_sq1, want_state=True)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2) and np.array_equal(z1, z2)
    qs, ks, vs = grid((B, Hq, d)), grid((B, Hkv, d)), grid((B, Hkv, d))
    S1c, z1c = S1.copy(), z1.copy()
    a = oracle.decode_step(_sq1(qs).astype(np.float32), _sq1(ks).astype(np.float32), vs, S1, z1, phi="features")
    b = oracle.decode_step(qs, ks, vs, S1c, z1c, phi=_sq1)
    assert np.array_equal(a, b) and np.array_equal(S1, S1c)


def test_callback_decode_steps_continue_the_causal_pass():
    B, Hq, Hkv, n, d, T = 2, 4, 2, 30, 6, 5
    q, k, v, _ = li.qkv(B, Hq, Hkv, n, d, li.F32, seed=10, scaled=True)
    full = oracle.causal(q, k, v, phi=_softplus)
    _, S, z = oracle.causal(q[:, :, : n - T], k[:, :, : n - T], v[:, :, : n - T], want_state=True, phi=_softplus)
    for t in range(n - T, n):
        o = oracle.decode_step(q[:, :, t].copy(), k[:, :, t].copy(), v[:, :, t].copy(), S, z, phi=_softplus)
        assert rel_rows(o, full[:, :, t]) < 1e-12


# ---------------------------------------------------------------------------
# Sliding window (LinearTile 1.0.1, "Features"): query i sees keys
# i - w < j <= i.  Pinned by its special cases: w = 1 returns V_i, w >= i + 1
# is the causal form (the oracle's state recurrence, a different
# computation), equal keys give the window mean of V, d = 1 does not depend
# on Q, and keys outside a query's window do not move its output.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [li.F32, li.BF16])
def test_window_of_one_returns_v(dtype):
    q, k, v, _ = li.qkv(2, 4, 2, 37, 5, dtype, seed=20)
    got = oracle.window(q, k, v, 1)
    want = np.repeat(li.to_f32(v).astype(np.float64), 2, axis=1)
    assert np.allclose(got, want, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("phi", ["relu1", "elu1"])
def test_window_covering_the_prefix_is_the_causal_form(phi):
    q, k, v, _ = li.qkv(2, 4, 2, 41, 6, li.F32, seed=21, scaled=True)
    for w in (41, 50, 1000):
        assert rel_rows(oracle.window(q, k, v, w, phi=phi), oracle.causal(q, k, v, phi=phi)) < 1e-12
    # rows i < w see the whole prefix
    got = oracle.window(q, k, v, 10, phi=phi)
    assert rel_rows(got[:, :, :10], oracle.causal(q, k, v, phi=phi)[:, :, :10]) < 1e-12


def test_window_equal_keys_give_the_window_mean():
    B, H, n, d, w = 1, 2, 50, 4, 7
    q, _, v, rng = li.qkv(B, H, H, n, d, li.F32, seed=22)
    k = np.broadcast_to(rng.standard_normal(d, dtype=np.float32), (B, H, n, d)).copy()
    vf = v.astype(np.float64)
    want = np.stack([vf[:, :, max(0, i - w + 1): i + 1].mean(axis=2) for i in range(n)], axis=2)
    assert np.allclose(oracle.window(q, k, v, w), want, rtol=1e-12, atol=1e-12)


def test_window_d1_output_does_not_depend_on_q():
    q1, k, v, _ = li.qkv(1, 1, 1, 30, 1, li.F32, seed=23)
    q2 = (q1 * -2.0 + 0.5).astype(np.float32)
    w = 6
    a, b = oracle.window(q1, k, v, w), oracle.window(q2, k, v, w)
    assert np.allclose(a, b, rtol=1e-13, atol=0)
    pk = _relu1(k[0, 0, :, 0].astype(np.float64))
    vv = v[0, 0, :, 0].astype(np.float64)
    want = [(pk[max(0, i - w + 1): i + 1] * vv[max(0, i - w + 1): i + 1]).sum() / pk[max(0, i - w + 1): i + 1].sum()
            for i in range(30)]
    assert np.allclose(a[0, 0, :, 0], want, rtol=1e-13)


def test_window_ignores_keys_outside_it():
    """Changing key/value i - w (just outside query i's window) leaves out_i
    unchanged and moves out_{i-1} (whose window holds it)."""
    B, H, n, d, w = 1, 1, 40, 4, 9
    q, k, v, rng = li.qkv(B, H, H, n, d, li.F32, seed=24)
    i = 25
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, i - w] += 1.0
    v2[0, 0, i - w] -= 3.0
    a, b = oracle.window(q, k, v, w), oracle.window(q, k2, v2, w)
    assert np.array_equal(a[0, 0, i], b[0, 0, i])
    assert not np.allclose(a[0, 0, i - 1], b[0, 0, i - 1])


def test_window_gqa_equals_repeated_kv_heads():
    q, k, v, _ = li.qkv(2, 6, 2, 23, 3, li.F32, seed=25)
    rep = lambda x: np.repeat(x, 3, axis=1)
    assert np.array_equal(oracle.window(q, k, v, 5), oracle.window(q, rep(k), rep(v), 5))


# ---------------------------------------------------------------------------
# Gradients of the causal form (LinearTile 1.0.1, "Project Structure" /
# "Run Tests": backward).  Pinned by central finite differences of the
# forward oracle in fp64, by float64 autograd through a plain torch
# transcription of the forward, and by special cases: d = 1 (the output does
# not depend on Q, so dQ = 0), dV does not depend on V, features mode equals
# relu + 1 where phi' = 1, GQA = repeated heads with dK, dV summed.
# ---------------------------------------------------------------------------
def _away_from_zero(rng, shape, lo=0.05):
    x = rng.standard_normal(size=shape)
    return np.where(np.abs(x) < lo, np.sign(x + 1e-12) * lo, x)  # no element at relu's kink


@pytest.mark.parametrize("phi", ["relu1", "elu1"])
@pytest.mark.parametrize("shape", [(1, 1, 1, 6, 3), (1, 2, 1, 5, 2), (2, 2, 2, 4, 4)])
def test_backward_matches_finite_differences(phi, shape):
    B, Hq, Hkv, n, d = shape
    rng = np.random.default_rng(40)
    q = _away_from_zero(rng, (B, Hq, n, d))
    k = _away_from_zero(rng, (B, Hkv, n, d))
    v = rng.standard_normal((B, Hkv, n, d))
    dout = rng.standard_normal((B, Hq, n, d))
    dq, dk, dv = oracle.causal_backward(q, k, v, dout, phi=phi)
    loss = lambda q_, k_, v_: float((oracle.causal(q_, k_, v_, phi=phi) * dout).sum())
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + eps
            lp = loss(q, k, v)
            x[idx] = x0 - eps
            lm = loss(q, k, v)
            x[idx] = x0
            fd[idx] = (lp - lm) / (2 * eps)
        assert np.allclose(g, fd, rtol=1e-6, atol=1e-8), np.abs(g - fd).max()


@pytest.mark.parametrize("phi", ["relu1", "elu1"])
def test_backward_matches_float64_autograd(phi):
    torch = pytest.importorskip("torch")
    B, Hq, Hkv, n, d = 2, 4, 2, 37, 8
    rng = np.random.default_rng(41)
    q, k, v, dout = (rng.standard_normal(s) for s in ((B, Hq, n, d), (B, Hkv, n, d), (B, Hkv, n, d), (B, Hq, n, d)))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    f = (lambda x: torch.relu(x) + 1) if phi == "relu1" else (lambda x: torch.nn.functional.elu(x) + 1)
    R = Hq // Hkv
    kk, vv = tk.repeat_interleave(R, dim=1), tv.repeat_interleave(R, dim=1)
    w = torch.tril(f(tq) @ f(kk).transpose(-1, -2))
    out = (w @ vv) / w.sum(-1, keepdim=True)
    (out * torch.tensor(dout)).sum().backward()
    dq, dk, dv = oracle.causal_backward(q, k, v, dout, phi=phi)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.allclose(mine, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_special_cases():
    rng = np.random.default_rng(42)
    B, Hq, Hkv, n = 1, 2, 1, 20
    # d = 1: phi(q) cancels in the output, so dQ = 0 exactly
    q, k, v, dout = (rng.standard_normal(s) for s in ((B, Hq, n, 1), (B, Hkv, n, 1), (B, Hkv, n, 1), (B, Hq, n, 1)))
    dq, _, _ = oracle.causal_backward(q, k, v, dout)
    assert np.abs(dq).max() < 1e-12
    # dV does not depend on V
    d = 5
    q, k, v, v2, dout = (rng.standard_normal(s) for s in ((B, Hq, n, d), (B, Hkv, n, d), (B, Hkv, n, d),
                                                          (B, Hkv, n, d), (B, Hq, n, d)))
    assert np.allclose(oracle.causal_backward(q, k, v, dout)[2], oracle.causal_backward(q, k, v2, dout)[2],
                       rtol=1e-13, atol=1e-14)
    # features mode on phi(x) = x + 1 (x > 0) equals relu + 1 on x (phi' = 1 there)
    qp, kp = np.abs(q) + 0.1, np.abs(k) + 0.1
    a = oracle.causal_backward(qp, kp, v, dout)
    b = oracle.causal_backward(qp + 1.0, kp + 1.0, v, dout, phi="features")
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=1e-12, atol=1e-13)
    # GQA: repeated key/value heads, dK and dV summed over the repeats
    rep = lambda x: np.repeat(x, 2, axis=1)
    g1 = oracle.causal_backward(q, k, v, dout)
    g2 = oracle.causal_backward(q, rep(k), rep(v), dout)
    assert np.allclose(g1[0], g2[0], rtol=1e-13, atol=1e-14)
    for i in (1, 2):
        assert np.allclose(g1[i], g2[i].reshape(B, Hkv, 2, n, d).sum(axis=2), rtol=1e-12, atol=1e-13)
