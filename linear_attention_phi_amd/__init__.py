"""Python binding of liblaphi.so, the MI355X (gfx950) kernelized
linear-attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/la.h).  PyTorch supplies device memory and
the current stream.  There is no fallback: if the library is missing or a
call fails, an exception is raised.

Functions carry the C names:
  la_forward(q, k, v)                        non-causal
  la_causal_forward(q, k, v, chunk=0)        causal (optionally the final state)
  la_prefix_mask_forward(q, k, v, m)         unnormalised Q K^T V, prefix mask m [n]
                                             (or [B, n]: la_prefix_mask_forward_batched)
  la_decode_step(q, k, v, S, z)              one recurrent step (S, z in place)
  la_window_forward(q, k, v, window)         sliding window: keys i - window < j <= i
  la_causal_forward_noalloc(q, k, v)         la_causal_forward on the static scratch
  la_causal_forward_strided(q, k, v, ...)    causal / window form on strided or packed sequences
  la_causal_backward(q, k, v, dout)          gradients of the causal form
  (la_forward, la_causal_forward and la_decode_step take phi="relu1",
  phi="elu1" or phi="features" -- q and k then hold phi(Q) and phi(K) of a
  positive map the caller applied; the last two call la_forward_phi /
  la_causal_forward_phi / la_decode_step_phi with LA_PHI_ELU1 or
  LA_PHI_FEATURES)
  la_workspace_bytes(op, B, Hq, Hkv, n, d, dtype, chunk)
  la_workspace_init(ws) / la_workspace_status(ws) / la_workspace_set_wait(ws, limit, skew)
  la_status_str(code)
Tensors are contiguous [B, H, n, d] (q, out: H = Hq; k, v: H = Hkv) in
float32 or bfloat16 on one GPU; states are float32.

Workspaces: unless a call is given ws=, it uses one cached per (device,
stream), so calls on different streams never share one (calls on one stream
run in order).  A cached workspace starts zero-filled, as the control block
in its first 256 bytes must.  Under HIP graph capture a call must be given
ws= (a workspace allocated and zero-filled before the capture), because a
workspace allocated during capture would be re-zeroed by every replay.
With the environment variable LA_DEBUG_CHECKS=1, every forward call
synchronises its stream afterwards and raises LAError for the errors only the
device sees (a bounded wait that gave up, a mask value out of range).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# LA_LIBRARY names another build of the same library to load instead (the
# host-sanitizer build the CPU tests make); by default the in-tree one.
LIB_PATH = os.environ.get("LA_LIBRARY") or os.path.join(_HERE, "liblaphi.so")

LA_F32, LA_BF16 = 0, 1
LA_OP_FORWARD, LA_OP_CAUSAL, LA_OP_PREFIX_MASK, LA_OP_PREFIX_MASK_BATCHED, LA_OP_SEQS = 0, 1, 2, 3, 4
LA_OP_CAUSAL_BACKWARD = 5
LA_PHI_RELU1, LA_PHI_ELU1, LA_PHI_FEATURES = 0, 1, 2
_PHI = {"relu1": LA_PHI_RELU1, "elu1": LA_PHI_ELU1, "features": LA_PHI_FEATURES}


def _phi(phi):
    if phi not in _PHI:
        raise ValueError(f"phi must be one of {sorted(_PHI)}")
    return _PHI[phi]
STATUS_NAMES = ["LA_OK", "LA_ERR_NULL", "LA_ERR_SHAPE", "LA_ERR_DTYPE", "LA_ERR_UNSUPPORTED",
                "LA_ERR_WORKSPACE", "LA_ERR_ALIGN", "LA_ERR_ALIAS", "LA_ERR_LAUNCH", "LA_ERR_TIMEOUT",
                "LA_ERR_RANGE", "LA_ERR_DEVICE"]
LA_ERR_TIMEOUT, LA_ERR_RANGE = 9, 10
CTL_BYTES = 256  # the workspace's control block

_lib = None


class LAError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {la_status_str(code)}")


def load():
    """Load liblaphi.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m linear_attention_phi_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        lib.la_status_str.argtypes = [I32]
        lib.la_status_str.restype = ctypes.c_char_p
        lib.la_workspace_bytes.argtypes = [I32, I64, I64, I64, I64, I64, I32, I32]
        lib.la_workspace_bytes.restype = SZ
        lib.la_forward.argtypes = [P, P, P, I64, I64, I64, I64, I64, I32, P, P, SZ, P]
        lib.la_causal_forward.argtypes = [P, P, P, I64, I64, I64, I64, I64, I32, I32, P, P, P, P, SZ, P]
        lib.la_prefix_mask_forward.argtypes = [P, P, P, P, I64, I64, I64, I64, I32, I32, P, P, SZ, P]
        lib.la_prefix_mask_forward_batched.argtypes = [P, P, P, P, I64, I64, I64, I64, I32, I32, P, P, SZ, P]
        lib.la_decode_step.argtypes = [P, P, P, I64, I64, I64, I64, I32, P, P, P, P]
        lib.la_forward_phi.argtypes = [P, P, P, I64, I64, I64, I64, I64, I32, I32, P, P, SZ, P]
        lib.la_causal_forward_phi.argtypes = [P, P, P, I64, I64, I64, I64, I64, I32, I32, I32, P, P, P, P, SZ, P]
        lib.la_decode_step_phi.argtypes = [P, P, P, I64, I64, I64, I64, I32, I32, P, P, P, P]
        U32 = ctypes.c_uint32
        lib.la_workspace_init.argtypes = [P, SZ, P]
        lib.la_workspace_status.argtypes = [P, SZ, P]
        lib.la_workspace_set_wait.argtypes = [P, SZ, U32, U32, P]
        lib.la_causal_forward_noalloc.argtypes = [P, P, P, I64, I64, I64, I64, I64, I32, I32, P, P, P, P]
        lib.la_window_forward.argtypes = [P, P, P, I64, I64, I64, I64, I64, I32, I32, I64, P, P]
        lib.la_causal_forward_strided.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I64, P, P, I32, I32, I64,
                                                  P, P, P, P, SZ, P]
        lib.la_causal_backward.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I32, I32, P, P, P, P, SZ, P]
        for f in ("la_forward", "la_causal_forward", "la_prefix_mask_forward", "la_decode_step",
                  "la_forward_phi", "la_causal_forward_phi", "la_decode_step_phi", "la_prefix_mask_forward_batched",
                  "la_workspace_init", "la_workspace_status", "la_workspace_set_wait",
                  "la_causal_forward_noalloc", "la_window_forward", "la_causal_forward_strided",
                  "la_causal_backward"):
            getattr(lib, f).restype = I32
        _lib = lib
    return _lib


def la_status_str(code: int) -> str:
    return load().la_status_str(int(code)).decode()


def la_workspace_bytes(op, B, Hq, Hkv, n, d, dtype, chunk=0) -> int:
    return int(load().la_workspace_bytes(op, B, Hq, Hkv, n, d, dtype, chunk))


# ----------------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return LA_F32
    if t.dtype == torch.bfloat16:
        return LA_BF16
    raise TypeError(f"dtype {t.dtype} not supported (float32 or bfloat16)")


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dev_any(t):
    """A GPU tensor's data pointer, whatever its strides (the caller passes them)."""
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


_ws_cache: dict = {}


def workspace(nbytes: int, device):
    """A device workspace of at least nbytes, cached per (device, current
    stream) and shared by the calls on that stream, which run in order.  It is
    allocated zero-filled on that stream (the control block must start at
    zero) and only ever used there.  Raises under graph capture if no cached
    workspace is large enough (pass ws= then)."""
    torch = _torch()
    if device.type != "cuda":
        raise ValueError("inputs must be GPU tensors (there is no host path)")
    stream = torch.cuda.current_stream(device)
    key = (device.index, stream.cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("a linear-attention call under graph capture needs ws= (a workspace "
                               "allocated and zero-filled before the capture)")
        buf = torch.zeros(max(nbytes, CTL_BYTES), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def new_workspace(nbytes: int, device):
    """A zero-filled workspace of at least nbytes for the caller to keep (for
    graph capture, or calls on several streams at once)."""
    torch = _torch()
    return torch.zeros(max(int(nbytes), CTL_BYTES), dtype=torch.uint8, device=device)


def la_workspace_init(ws):
    """Zero the control block of ws on the current stream."""
    _call(load().la_workspace_init(_dev(ws, "ws"), ws.numel(), _stream(ws)), "la_workspace_init")


def la_workspace_status(ws) -> int:
    """Synchronise the current stream, then return (and clear) the status the
    device recorded in ws since the last check: 0, LA_ERR_TIMEOUT or LA_ERR_RANGE."""
    return int(load().la_workspace_status(_dev(ws, "ws"), ws.numel(), _stream(ws)))


def la_workspace_set_wait(ws, limit=0, skew=0):
    """Diagnostics: polls before a bounded wait gives up (0: default) and a skew
    added to the epoch the waits expect (non-zero: every wait gives up)."""
    _call(load().la_workspace_set_wait(_dev(ws, "ws"), ws.numel(), int(limit), int(skew), _stream(ws)),
          "la_workspace_set_wait")


def _debug_check(ws, what):
    if os.environ.get("LA_DEBUG_CHECKS") == "1" and not _torch().cuda.is_current_stream_capturing():
        _call(la_workspace_status(ws), what)


def _expect(t, shape, dtype, name):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected shape {tuple(shape)} dtype {dtype}, "
                         f"got {tuple(t.shape)} {t.dtype}")


def _qkv(q, k, v):
    """Check q [B,Hq,n,d] and k, v [B,Hkv,n,d] of one dtype; return the sizes."""
    if k.dim() != 4:
        raise ValueError("k must be [B, Hkv, n, d]")
    B, Hkv, n, d = k.shape
    _expect(v, k.shape, k.dtype, "v")
    Hq = Hkv
    if q is not None:
        if q.dim() != 4:
            raise ValueError("q must be [B, Hq, n, d]")
        Hq = q.shape[1]
        _expect(q, (B, Hq, n, d), k.dtype, "q")
        if Hq % Hkv:
            raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    return B, Hq, Hkv, n, d


def _call(rc, what):
    if rc != 0:
        raise LAError(rc, what)


def la_forward(q, k, v, out=None, ws=None, phi="relu1"):
    """Non-causal normalised linear attention; returns out (q's shape and dtype).
    phi: "relu1" (relu(x) + 1, la_forward) or "elu1" (ELU(x) + 1, la_forward_phi)."""
    phi_code = _phi(phi)
    torch = _torch()
    B, Hq, Hkv, n, d = _qkv(q, k, v)
    dt = _dtype_code(q)
    out = torch.empty_like(q) if out is None else out
    _expect(out, q.shape, q.dtype, "out")
    need = la_workspace_bytes(LA_OP_FORWARD, B, Hq, Hkv, n, d, dt, 0)
    ws = workspace(need, q.device) if ws is None else ws
    if phi == "relu1":
        _call(load().la_forward(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), B, Hq, Hkv, n, d, dt,
                                _dev(out, "out"), _dev(ws, "ws"), ws.numel(), _stream(q)), "la_forward")
    else:
        _call(load().la_forward_phi(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), B, Hq, Hkv, n, d, dt, phi_code,
                                    _dev(out, "out"), _dev(ws, "ws"), ws.numel(), _stream(q)), "la_forward_phi")
    _debug_check(ws, "la_forward")
    return out


def la_causal_forward(q, k, v, chunk=0, out=None, want_state=False, S_final=None, z_final=None,
                      ws=None, Hq=None, phi="relu1"):
    """Causal normalised linear attention (phi: "relu1" or "elu1", as la_forward).

    q may be None for a state-only pass (pass Hq, default Hkv); then the
    final state is returned.  With want_state, returns (out, S_final, z_final).
    """
    phi_code = _phi(phi)
    torch = _torch()
    B, Hq_, Hkv, n, d = _qkv(q, k, v)
    dt = _dtype_code(k)
    if q is not None:
        Hq = Hq_
        out = torch.empty_like(q) if out is None else out
        _expect(out, q.shape, q.dtype, "out")
    else:
        Hq = Hq or Hkv
        want_state = True
    if want_state:
        S_final = torch.empty((B, Hkv, d, d), dtype=torch.float32, device=k.device) if S_final is None else S_final
        z_final = torch.empty((B, Hkv, d), dtype=torch.float32, device=k.device) if z_final is None else z_final
        _expect(S_final, (B, Hkv, d, d), torch.float32, "S_final")
        _expect(z_final, (B, Hkv, d), torch.float32, "z_final")
    need = la_workspace_bytes(LA_OP_CAUSAL, B, Hq, Hkv, n, d, dt, chunk)
    if need == 0:
        raise LAError(4, f"la_causal_forward (chunk={chunk}, d={d}, dtype={k.dtype})")
    ws = workspace(need, k.device) if ws is None else ws
    if phi == "relu1":
        _call(load().la_causal_forward(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), B, Hq, Hkv, n, d, dt, chunk,
                                       _dev(out, "out"), _dev(S_final, "S_final"), _dev(z_final, "z_final"),
                                       _dev(ws, "ws"), ws.numel(), _stream(k)), "la_causal_forward")
    else:
        _call(load().la_causal_forward_phi(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), B, Hq, Hkv, n, d, dt,
                                           phi_code, chunk, _dev(out, "out"), _dev(S_final, "S_final"),
                                           _dev(z_final, "z_final"), _dev(ws, "ws"), ws.numel(), _stream(k)),
              "la_causal_forward_phi")
    _debug_check(ws, "la_causal_forward")
    if q is None:
        return S_final, z_final
    if want_state:
        return out, S_final, z_final
    return out


def la_causal_forward_noalloc(q, k, v, chunk=0, out=None, want_state=False):
    """la_causal_forward (relu + 1) through la_causal_forward_noalloc, whose
    workspace is the library's static per-GPU array: no workspace is
    allocated.  out (and the final state, with want_state) are allocated here
    unless given."""
    torch = _torch()
    B, Hq, Hkv, n, d = _qkv(q, k, v)
    dt = _dtype_code(q)
    out = torch.empty_like(q) if out is None else out
    _expect(out, q.shape, q.dtype, "out")
    S_final = z_final = None
    if want_state:
        S_final = torch.empty((B, Hkv, d, d), dtype=torch.float32, device=k.device)
        z_final = torch.empty((B, Hkv, d), dtype=torch.float32, device=k.device)
    _call(load().la_causal_forward_noalloc(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), B, Hq, Hkv, n, d, dt, chunk,
                                           _dev(out, "out"), _dev(S_final, "S_final"), _dev(z_final, "z_final"),
                                           _stream(q)), "la_causal_forward_noalloc")
    return (out, S_final, z_final) if want_state else out


def la_window_forward(q, k, v, window, out=None, phi="relu1"):
    """Sliding-window causal normalised linear attention: query i sees keys
    max(0, i - window + 1) .. i.  phi as la_forward.  No workspace."""
    phi_code = _phi(phi)
    torch = _torch()
    B, Hq, Hkv, n, d = _qkv(q, k, v)
    dt = _dtype_code(q)
    out = torch.empty_like(q) if out is None else out
    _expect(out, q.shape, q.dtype, "out")
    _call(load().la_window_forward(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), B, Hq, Hkv, n, d, dt, phi_code,
                                   int(window), _dev(out, "out"), _stream(q)), "la_window_forward")
    return out


def la_causal_forward_strided(q, k, v, cu_seqlens=None, max_len=None, window=0, out=None, want_state=False,
                              ws=None, phi="relu1", Hq=None):
    """The causal (window=0) or sliding-window form over sequences of any layout.

    cu_seqlens None: q [B, Hq, n, d], k, v [B, Hkv, n, d] as views with any
    strides (the last one 1), e.g. x.view(B, n, H, d).transpose(1, 2) for a
    [batch, seq, H, d] buffer.  cu_seqlens given (int64 [nseq + 1] on the
    GPU): packed q [total, Hq, d], k, v [total, Hkv, d] (any strides, the last
    one 1); sequence s is rows cu[s] .. cu[s+1] - 1; max_len bounds the lengths
    (computed from cu_seqlens, with a host synchronisation, when None).  out
    takes q's layout (allocated like q unless given).  q may be None for a
    state-only causal pass (pass Hq).  With want_state (causal form) returns
    (out, S_final [nseq, Hkv, d, d], z_final [nseq, Hkv, d])."""
    phi_code = _phi(phi)
    torch = _torch()
    packed = cu_seqlens is not None
    dims = 3 if packed else 4
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        if t is None:
            continue
        if t.dim() != dims or t.stride(-1) != 1 or not t.is_cuda:
            raise ValueError(f"{name} must be a {dims}-D GPU tensor whose last dimension is contiguous")
    if k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("k and v must share shape and dtype")
    if packed:
        total, Hkv, d = k.shape
        if cu_seqlens.dtype != torch.int64 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
            raise ValueError("cu_seqlens must be a contiguous int64 vector [nseq + 1]")
        nseq = cu_seqlens.numel() - 1
        if max_len is None:
            max_len = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if nseq > 0 else 0
        kvs = (0, k.stride(1), k.stride(0))
        seq_dim, head_dim = None, 1
    else:
        nseq, Hkv, max_len, d = k.shape
        total = nseq * max_len
        kvs = (k.stride(0), k.stride(1), k.stride(2))
    if v.stride() != k.stride():
        raise ValueError("k and v must share strides")
    if q is not None:
        Hq = q.shape[1]
        if q.dtype != k.dtype or (packed and tuple(q.shape) != (total, Hq, d)) or (
                not packed and tuple(q.shape) != (nseq, Hq, max_len, d)):
            raise ValueError("q must match k's sizes (with its own head count) and dtype")
        out = torch.empty_like(q) if out is None else out
        if out.shape != q.shape or out.stride() != q.stride() or out.dtype != q.dtype:
            raise ValueError("out must have q's shape, strides and dtype")
        qs = (0, q.stride(1), q.stride(0)) if packed else (q.stride(0), q.stride(1), q.stride(2))
    else:
        Hq = Hq or Hkv
        want_state = True
        qs = (0, d, Hq * d) if packed else (Hq * max_len * d, max_len * d, d)
    if Hq % Hkv:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    dt = _dtype_code(k)
    S_final = z_final = None
    if want_state:
        if window:
            raise ValueError("the window form hands on no state")
        S_final = torch.empty((nseq, Hkv, d, d), dtype=torch.float32, device=k.device)
        z_final = torch.empty((nseq, Hkv, d), dtype=torch.float32, device=k.device)
    need = la_workspace_bytes(LA_OP_SEQS, max(nseq, 1), Hq, Hkv, max(max_len, 1), d, dt, 0)
    ws = workspace(need, k.device) if ws is None else ws
    qa = (ctypes.c_int64 * 3)(*qs)
    ka = (ctypes.c_int64 * 3)(*kvs)
    _call(load().la_causal_forward_strided(_dev_any(q) if q is not None else None, _dev_any(k), _dev_any(v),
                                           _dev(cu_seqlens, "cu_seqlens") if packed else None, nseq, max_len,
                                           total, Hq, Hkv, d, qa, ka, dt, phi_code, int(window),
                                           _dev_any(out) if out is not None else None, _dev(S_final, "S_final"),
                                           _dev(z_final, "z_final"), _dev(ws, "ws"), ws.numel(), _stream(k)),
          "la_causal_forward_strided")
    _debug_check(ws, "la_causal_forward_strided")
    if q is None:
        return S_final, z_final
    return (out, S_final, z_final) if want_state else out


def la_causal_backward(q, k, v, dout, ws=None, phi="relu1"):
    """Gradients (dq, dk, dv) of sum(dout * la_causal_forward(q, k, v, phi=phi));
    the forward is recomputed.  Contiguous [B, H, n, d] tensors, d <= 64."""
    phi_code = _phi(phi)
    torch = _torch()
    B, Hq, Hkv, n, d = _qkv(q, k, v)
    _expect(dout, q.shape, q.dtype, "dout")
    dt = _dtype_code(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    need = la_workspace_bytes(LA_OP_CAUSAL_BACKWARD, B, Hq, Hkv, n, d, dt, 0)
    if need == 0:
        raise LAError(4, f"la_causal_backward (d={d}, dtype={q.dtype})")
    ws = workspace(need, q.device) if ws is None else ws
    _call(load().la_causal_backward(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(dout, "dout"), B, Hq, Hkv, n, d,
                                    dt, phi_code, _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv"), _dev(ws, "ws"),
                                    ws.numel(), _stream(q)), "la_causal_backward")
    _debug_check(ws, "la_causal_backward")
    return dq, dk, dv


def la_prefix_mask_forward(q, k, v, m, chunk=0, out=None, ws=None):
    """Unnormalised Q K^T V where query i sees keys 0..m[i] (m: int64 [n] on the
    GPU, shared by the batches), or query i of batch b keys 0..m[b, i] (m:
    int64 [B, n], la_prefix_mask_forward_batched)."""
    torch = _torch()
    B, H, Hkv, n, d = _qkv(q, k, v)
    if Hkv != H:
        raise ValueError("the prefix-mask form needs as many key/value heads as query heads")
    dt = _dtype_code(q)
    if m.dtype != torch.int64 or tuple(m.shape) not in ((n,), (B, n)) or not m.is_contiguous():
        raise ValueError("m must be a contiguous int64 tensor of shape (n,) or (B, n)")
    batched = m.dim() == 2
    out = torch.empty_like(q) if out is None else out
    _expect(out, q.shape, q.dtype, "out")
    need = la_workspace_bytes(LA_OP_PREFIX_MASK_BATCHED if batched else LA_OP_PREFIX_MASK, B, H, H, n, d, dt, chunk)
    if need == 0:
        raise LAError(4, f"la_prefix_mask_forward (chunk={chunk}, n={n}, d={d}, dtype={q.dtype})")
    ws = workspace(need, q.device) if ws is None else ws
    fn = "la_prefix_mask_forward_batched" if batched else "la_prefix_mask_forward"
    _call(getattr(load(), fn)(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(m, "m"), B, H, n, d,
                              dt, chunk, _dev(out, "out"), _dev(ws, "ws"), ws.numel(), _stream(q)), fn)
    _debug_check(ws, fn)
    return out


def la_decode_step(q, k, v, S, z, out=None, phi="relu1"):
    """One decode step: q [B,Hq,d], k/v [B,Hkv,d]; S [B,Hkv,d,d], z [B,Hkv,d]
    (float32) are updated in place.  Returns out [B,Hq,d].  phi as la_forward
    (the map the state was built with)."""
    phi_code = _phi(phi)
    torch = _torch()
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    dt = _dtype_code(q)
    _expect(k, (B, Hkv, d), q.dtype, "k")
    _expect(v, (B, Hkv, d), q.dtype, "v")
    if Hq % Hkv:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    _expect(S, (B, Hkv, d, d), torch.float32, "S")
    _expect(z, (B, Hkv, d), torch.float32, "z")
    out = torch.empty_like(q) if out is None else out
    _expect(out, q.shape, q.dtype, "out")
    if phi == "relu1":
        _call(load().la_decode_step(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), B, Hq, Hkv, d, dt,
                                    _dev(S, "S"), _dev(z, "z"), _dev(out, "out"), _stream(q)), "la_decode_step")
    else:
        _call(load().la_decode_step_phi(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), B, Hq, Hkv, d, dt, phi_code,
                                        _dev(S, "S"), _dev(z, "z"), _dev(out, "out"), _stream(q)),
              "la_decode_step_phi")
    return out
