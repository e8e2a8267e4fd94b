"""C-ABI checks that need no GPU: the library loads, exports every function
include/la.h declares, sizes workspaces, and rejects every invalid argument
with its status code before anything is launched (the checks run on the host
and return before the first HIP call, so fake device pointers are safe)."""
import ctypes
import os
import re

import pytest

import linear_attention_phi_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la.h")

OK, NULL, SHAPE, DTYPE, UNSUP, WS, ALIGN, ALIAS = range(8)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return la.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == {"la_status_str", "la_workspace_bytes", "la_forward", "la_causal_forward",
                          "la_prefix_mask_forward", "la_decode_step", "la_forward_phi",
                          "la_causal_forward_phi", "la_decode_step_phi", "la_prefix_mask_forward_batched",
                          "la_workspace_init", "la_workspace_status", "la_workspace_set_wait",
                          "la_causal_forward_noalloc", "la_window_forward", "la_causal_forward_strided",
                          "la_causal_backward"}
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in enumerate(la.STATUS_NAMES):
        assert la.la_status_str(code).startswith(name)
    assert la.la_status_str(99) == "unknown la_status"
    # the device-side statuses la_workspace_status returns
    assert la.la_status_str(9).startswith("LA_ERR_TIMEOUT")
    assert la.la_status_str(10).startswith("LA_ERR_RANGE")
    assert la.la_status_str(11).startswith("LA_ERR_DEVICE")
    assert (la.LA_ERR_TIMEOUT, la.LA_ERR_RANGE) == (9, 10)


def test_control_block_calls_reject_bad_workspaces(lib):
    """la_workspace_init / _status / _set_wait check the workspace on the host
    and return before any HIP call when it is NULL, smaller than the 256-byte
    control block or misaligned."""
    for ws, nbytes, want in ((None, 4096, NULL), (WSP, 255, WS), (WSP, 0, WS), (WSP + 8, 4096, ALIGN)):
        assert lib.la_workspace_init(ws, nbytes, None) == want
        assert lib.la_workspace_status(ws, nbytes, None) == want
        assert lib.la_workspace_set_wait(ws, nbytes, 64, 1, None) == want


def test_workspace_bytes_include_the_control_block(lib):
    """Every forward workspace holds the 256-byte control block before its
    data regions: the causal general path's size is that block plus (nseg + 1)
    fp32 state slots per head."""
    f = la.la_workspace_bytes
    # fp32 d = 32 causal, B1 H1 n64 chunk 32: two one-chunk segments -> 3 slots of 32*32 + 32 floats
    assert f(la.LA_OP_CAUSAL, 1, 1, 1, 64, 32, la.LA_F32, 32) == 256 + 3 * 4 * (32 * 32 + 32)
    for op in (la.LA_OP_FORWARD, la.LA_OP_CAUSAL, la.LA_OP_PREFIX_MASK):
        assert f(op, 1, 1, 1, 1, 1, la.LA_F32, 0) > 256


def test_workspace_bytes():
    f = la.la_workspace_bytes
    # causal bf16 B8 H8 n2048 d64: (nseg + 1) fp32 slots of (64*64 + 64) per head
    b = f(la.LA_OP_CAUSAL, 8, 8, 8, 2048, 64, la.LA_BF16, 64)
    assert b > 256 and (b - 256) % (4 * (64 * 64 + 64)) == 0
    assert f(la.LA_OP_CAUSAL, 8, 8, 8, 2048, 64, la.LA_BF16, 0) == b  # default chunk is 64
    assert f(la.LA_OP_FORWARD, 2, 8, 8, 4096, 64, la.LA_F32, 0) > 0
    # prefix form: states plus bucket offsets and the permutation
    p = f(la.LA_OP_PREFIX_MASK, 4, 8, 8, 8192, 64, la.LA_F32, 64)
    assert p > 4 * (8192 + 8192 // 64 + 1)
    # invalid requests size to 0
    assert f(7, 1, 1, 1, 16, 16, la.LA_F32, 0) == 0
    assert f(la.LA_OP_CAUSAL, 1, 3, 2, 16, 16, la.LA_F32, 0) == 0      # Hq % Hkv
    assert f(la.LA_OP_CAUSAL, 1, 1, 1, 16, 129, la.LA_F32, 0) == 0     # d > 128
    assert f(la.LA_OP_CAUSAL, 1, 1, 1, 0, 16, la.LA_F32, 0) == 0       # n = 0
    assert f(la.LA_OP_CAUSAL, 1, 1, 1, 16, 16, 5, 0) == 0              # dtype
    assert f(la.LA_OP_CAUSAL, 1, 1, 1, 16, 16, la.LA_F32, 48) == 0     # chunk
    assert f(la.LA_OP_CAUSAL, 1, 1, 1, 16, 128, la.LA_F32, 64) == 0    # fp32 d=128 chunk 64: LDS
    assert f(la.LA_OP_CAUSAL, 1, 1, 1, 16, 128, la.LA_F32, 32) > 0
    assert f(la.LA_OP_PREFIX_MASK, 1, 2, 1, 16, 16, la.LA_F32, 0) == 0  # prefix needs Hq == Hkv


# Fake, 16-byte aligned "device" addresses far apart; never dereferenced.
Q, K, V, O, WSP, M, S, Z = (0x10000000 * (i + 1) for i in range(8))
BIG = 1 << 30


def fwd(lib, q=Q, k=K, v=V, B=1, Hq=2, Hkv=1, n=16, d=16, dt=0, out=O, ws=WSP, wsb=BIG):
    return lib.la_forward(q, k, v, B, Hq, Hkv, n, d, dt, out, ws, wsb, None)


def causal(lib, q=Q, k=K, v=V, B=1, Hq=2, Hkv=1, n=16, d=16, dt=1, chunk=0, out=O, Sf=None, zf=None,
           ws=WSP, wsb=BIG):
    return lib.la_causal_forward(q, k, v, B, Hq, Hkv, n, d, dt, chunk, out, Sf, zf, ws, wsb, None)


def prefix(lib, q=Q, k=K, v=V, m=M, B=1, H=1, n=16, d=16, dt=0, chunk=0, out=O, ws=WSP, wsb=BIG):
    return lib.la_prefix_mask_forward(q, k, v, m, B, H, n, d, dt, chunk, out, ws, wsb, None)


def decode(lib, q=Q, k=K, v=V, B=1, Hq=2, Hkv=1, d=16, dt=0, S_=S, z=Z, out=O):
    return lib.la_decode_step(q, k, v, B, Hq, Hkv, d, dt, S_, z, out, None)


def test_feature_map_rejections(lib):
    """The *_phi entry points reject an unknown feature map, and run every
    other check of their plain counterparts (each call below fails a check,
    so nothing is launched)."""
    for phi in (3, -1, 7):
        assert lib.la_forward_phi(Q, K, V, 1, 2, 1, 16, 16, 0, phi, O, WSP, BIG, None) == UNSUP
        assert lib.la_causal_forward_phi(Q, K, V, 1, 2, 1, 16, 16, 1, phi, 0, O, None, None, WSP, BIG, None) == UNSUP
        assert lib.la_decode_step_phi(Q, K, V, 1, 2, 1, 16, 0, phi, S, Z, O, None) == UNSUP
    for phi in (la.LA_PHI_RELU1, la.LA_PHI_ELU1, la.LA_PHI_FEATURES):
        assert lib.la_forward_phi(None, K, V, 1, 2, 1, 16, 16, 0, phi, O, WSP, BIG, None) == NULL
        assert lib.la_forward_phi(Q, K, V, 1, 2, 1, 16, 16, 0, phi, K, WSP, BIG, None) == ALIAS
        assert lib.la_forward_phi(Q, K, V, 1, 2, 1, 16, 16, 0, phi, O, WSP, 16, None) == WS
        assert lib.la_causal_forward_phi(Q, K, V, 1, 2, 1, 16, 16, 1, phi, 48, O, None, None, WSP, BIG, None) == UNSUP
        assert lib.la_causal_forward_phi(Q, K, V, 1, 2, 1, 16, 16, 1, phi, 0, O, S + 4, None, WSP, BIG, None) == ALIGN
        assert lib.la_decode_step_phi(Q, K, V, 1, 3, 2, 16, 0, phi, S, Z, O, None) == SHAPE
        assert lib.la_decode_step_phi(Q, K, V, 1, 2, 1, 16, 0, phi, S, Z, S, None) == ALIAS


def test_forward_rejections(lib):
    assert fwd(lib, q=None) == NULL
    assert fwd(lib, out=None) == NULL
    assert fwd(lib, dt=3) == DTYPE
    assert fwd(lib, d=0) == SHAPE
    assert fwd(lib, d=129) == SHAPE
    assert fwd(lib, n=0) == SHAPE
    assert fwd(lib, B=0) == SHAPE
    assert fwd(lib, Hq=3, Hkv=2) == SHAPE
    assert fwd(lib, q=Q + 8) == ALIGN
    assert fwd(lib, out=Q + 64) == ALIAS
    assert fwd(lib, out=K) == ALIAS
    assert fwd(lib, wsb=16) == WS
    assert fwd(lib, ws=None) == WS
    assert fwd(lib, ws=WSP + 4) == ALIGN
    assert fwd(lib, ws=V) == ALIAS


def test_causal_rejections(lib):
    assert causal(lib, k=None) == NULL
    assert causal(lib, q=None) == NULL                 # q without out
    assert causal(lib, out=None) == NULL               # out without q
    assert causal(lib, q=None, out=None) == NULL       # state-only needs S_final or z_final
    assert causal(lib, chunk=48) == UNSUP
    assert causal(lib, chunk=16) == UNSUP
    assert causal(lib, d=128, dt=0, chunk=128) == UNSUP
    assert causal(lib, Sf=S + 4) == ALIGN
    assert causal(lib, Sf=Q) == ALIAS
    assert causal(lib, Sf=S, zf=S + 16) == ALIAS
    assert causal(lib, wsb=100) == WS
    assert causal(lib, ws=O) == ALIAS
    assert causal(lib, n=(1 << 31)) == SHAPE


def test_batched_prefix_workspace_and_rejections(lib):
    """A sort per batch: the workspace grows by B - 1 bucket arrays; the
    checks are those of the shared-mask form, the mask spanning B rows."""
    f = la.la_workspace_bytes
    one = f(la.LA_OP_PREFIX_MASK, 4, 8, 8, 8192, 64, la.LA_F32, 64)
    four = f(la.LA_OP_PREFIX_MASK_BATCHED, 4, 8, 8, 8192, 64, la.LA_F32, 64)
    assert four - one == 3 * 4 * (8192 // 64 + 1 + 8192)
    assert f(la.LA_OP_PREFIX_MASK_BATCHED, 1, 2, 1, 16, 16, la.LA_F32, 0) == 0
    call = lib.la_prefix_mask_forward_batched
    assert call(Q, K, V, None, 2, 1, 16, 16, 0, 0, O, WSP, BIG, None) == NULL
    assert call(Q, K, V, M + 8, 2, 1, 16, 16, 0, 0, O, WSP, BIG, None) == ALIGN
    assert call(Q, K, V, M, 2, 1, 16, 16, 0, 100, O, WSP, BIG, None) == UNSUP
    assert call(Q, K, V, M, 2, 1, 16, 16, 0, 0, O, WSP, 8, None) == WS
    # out overlapping the second batch's mask row
    assert call(Q, K, V, M, 2, 1, 16, 16, 0, 0, M + 16 * 8, WSP, BIG, None) == ALIAS


def test_prefix_rejections(lib):
    assert prefix(lib, m=None) == NULL
    assert prefix(lib, m=M + 8) == ALIGN
    assert prefix(lib, out=M) == ALIAS
    assert prefix(lib, n=64 * 16384) == UNSUP   # too many buckets
    assert prefix(lib, chunk=100) == UNSUP
    assert prefix(lib, wsb=8) == WS


def test_decode_rejections(lib):
    assert decode(lib, S_=None) == NULL
    assert decode(lib, z=None) == NULL
    assert decode(lib, d=200) == SHAPE
    assert decode(lib, Hq=3, Hkv=2) == SHAPE
    assert decode(lib, dt=2) == DTYPE
    assert decode(lib, out=S) == ALIAS
    assert decode(lib, z=S + 256) == ALIAS
    assert decode(lib, q=Q + 2) == ALIGN


def test_binding_checks_shapes_before_calling():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 2, 8, 4)
    k = torch.zeros(1, 1, 8, 4)
    with pytest.raises(ValueError):
        la.la_forward(q, k, torch.zeros(1, 1, 8, 5))           # v shape
    with pytest.raises(ValueError):
        la.la_forward(q, k.to(torch.bfloat16), k)              # dtype mismatch
    with pytest.raises(ValueError):
        la.la_forward(torch.zeros(1, 3, 8, 4), torch.zeros(1, 2, 8, 4), torch.zeros(1, 2, 8, 4))
    with pytest.raises(TypeError):
        la.la_forward(q.double(), k.double(), k.double())
    with pytest.raises(ValueError):  # CPU tensors are refused (no host fallback)
        la.la_forward(q, k, k)
    with pytest.raises(ValueError, match="phi"):  # an unknown feature map, before anything else
        la.la_forward(q, k, k, phi="softmax")
    with pytest.raises(ValueError, match="phi"):
        la.la_causal_forward(q, k, k, phi="elu")
    with pytest.raises(ValueError, match="phi"):
        la.la_decode_step(q[:, :, 0], k[:, :, 0], k[:, :, 0], torch.zeros(1, 1, 4, 4), torch.zeros(1, 1, 4),
                          phi="")
    q4 = torch.zeros(2, 1, 8, 4)
    with pytest.raises(ValueError, match="m must"):  # a mask neither [n] nor [B, n]
        la.la_prefix_mask_forward(q4, q4, q4, torch.zeros(3, 8, dtype=torch.int64))


def test_noalloc_rejections(lib):
    """la_causal_forward_noalloc checks its arguments as la_causal_forward does,
    and refuses a size whose workspace exceeds its 64 MiB static array, all
    before any HIP call."""
    f = lambda **kw: lib.la_causal_forward_noalloc(*[kw.get(x, dflt) for x, dflt in (
        ("q", Q), ("k", K), ("v", V), ("B", 1), ("Hq", 2), ("Hkv", 1), ("n", 16), ("d", 16), ("dt", 1),
        ("chunk", 0), ("out", O), ("Sf", None), ("zf", None))], None)
    assert f(q=None) == NULL
    assert f(Hq=3, Hkv=2) == SHAPE
    assert f(dt=7) == DTYPE
    assert f(chunk=48) == UNSUP
    assert f(q=Q + 8) == ALIGN
    assert f(out=K) == ALIAS
    # B16 H64 n4096 d128 fp32: 1024 heads of two 66 KB state slots, more than 64 MiB
    assert la.la_workspace_bytes(la.LA_OP_CAUSAL, 16, 64, 64, 4096, 128, la.LA_F32, 0) > 64 << 20
    far = [(i + 1) << 40 for i in range(4)]  # fake addresses 1 TiB apart: the 2 GiB tensors do not overlap
    assert f(q=far[0], k=far[1], v=far[2], out=far[3], B=16, Hq=64, Hkv=64, n=4096, d=128, dt=0) == WS


def test_window_rejections(lib):
    """la_window_forward: every check on the host, nothing launched."""
    f = lambda **kw: lib.la_window_forward(*[kw.get(x, dflt) for x, dflt in (
        ("q", Q), ("k", K), ("v", V), ("B", 1), ("Hq", 2), ("Hkv", 1), ("n", 16), ("d", 16), ("dt", 1),
        ("phi", 0), ("w", 4), ("out", O))], None)
    assert f(q=None) == NULL
    assert f(out=None) == NULL
    assert f(w=0) == SHAPE
    assert f(w=-3) == SHAPE
    assert f(Hq=3, Hkv=2) == SHAPE
    assert f(dt=9) == DTYPE
    assert f(phi=5) == UNSUP
    assert f(dt=0, d=128) == UNSUP        # fp32 with d > 64: the tiles do not fit in LDS
    assert f(k=K + 4) == ALIGN
    assert f(out=V) == ALIAS


def test_strided_rejections(lib):
    """la_causal_forward_strided: every check on the host, nothing launched."""
    I3 = ctypes.c_int64 * 3
    B, H, n, d = 2, 2, 64, 16
    bnhd = I3(n * H * d, d, H * d)  # [B, n, H, d]

    def f(**kw):
        a = dict(q=Q, k=K, v=V, cu=None, nseq=B, max_len=n, total=0, Hq=H, Hkv=H, d=d, qs=bnhd, ks=bnhd, dt=1,
                 phi=0, w=0, out=O, Sf=None, zf=None, ws=WSP, wsb=BIG)
        a.update(kw)
        return lib.la_causal_forward_strided(a["q"], a["k"], a["v"], a["cu"], a["nseq"], a["max_len"], a["total"],
                                             a["Hq"], a["Hkv"], a["d"], a["qs"], a["ks"], a["dt"], a["phi"], a["w"],
                                             a["out"], a["Sf"], a["zf"], a["ws"], a["wsb"], None)
    assert f(k=None) == NULL
    assert f(qs=None) == NULL
    assert f(q=None) == NULL                      # q without out
    assert f(q=None, out=None) == NULL            # state only needs S_final or z_final
    assert f(q=None, out=None, w=5, Sf=S) == NULL or f(q=None, out=None, w=5, Sf=S) == UNSUP
    assert f(w=-1) == SHAPE
    assert f(w=4, Sf=S) == UNSUP                   # a window hands on no state
    assert f(qs=I3(n * H * d, d, -H * d)) == SHAPE  # negative stride
    assert f(qs=I3(n * H * d, 4, H * d)) == SHAPE   # heads of a row overlap
    assert f(cu=M) == SHAPE                       # packed with a nonzero sequence stride
    assert f(cu=M, qs=I3(0, d, H * d), ks=I3(0, d, H * d), total=-1) == SHAPE
    assert f(cu=M + 8, qs=I3(0, d, H * d), ks=I3(0, d, H * d), total=100) == ALIGN
    assert f(dt=0, d=128, w=3, qs=I3(n * H * 128, 128, H * 128), ks=I3(n * H * 128, 128, H * 128)) == UNSUP
    assert f(out=K) == ALIAS
    assert f(wsb=100) == WS
    assert f(phi=7) == UNSUP
    need = la.la_workspace_bytes(la.LA_OP_SEQS, B, H, H, n, d, la.LA_BF16, 0)
    assert need > 256
    assert f(wsb=need - 1) == WS


def test_backward_rejections(lib):
    """la_causal_backward: every check on the host, nothing launched."""
    DQ, DK, DV, DO = (0x10000000 * (i + 20) for i in range(4))

    def f(**kw):
        a = dict(q=Q, k=K, v=V, do=DO, B=1, Hq=2, Hkv=1, n=16, d=16, dt=1, phi=0, dq=DQ, dk=DK, dv=DV, ws=WSP,
                 wsb=BIG)
        a.update(kw)
        return lib.la_causal_backward(a["q"], a["k"], a["v"], a["do"], a["B"], a["Hq"], a["Hkv"], a["n"], a["d"],
                                      a["dt"], a["phi"], a["dq"], a["dk"], a["dv"], a["ws"], a["wsb"], None)
    assert f(do=None) == NULL
    assert f(dv=None) == NULL
    assert f(d=128) == UNSUP          # d > 64
    assert f(phi=4) == UNSUP
    assert f(Hq=3, Hkv=2) == SHAPE
    assert f(dq=Q) == ALIAS
    assert f(dk=DV) == ALIAS
    assert f(dk=K + 8) == ALIGN
    assert f(wsb=64) == WS
    assert la.la_workspace_bytes(la.LA_OP_CAUSAL_BACKWARD, 8, 8, 8, 2048, 64, la.LA_BF16, 0) > 256
    assert la.la_workspace_bytes(la.LA_OP_CAUSAL_BACKWARD, 1, 1, 1, 16, 128, la.LA_BF16, 0) == 0
