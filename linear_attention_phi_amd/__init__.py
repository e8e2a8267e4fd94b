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
  (la_forward, la_causal_forward and la_decode_step take phi="relu1" or
  phi="elu1"; the latter calls la_forward_phi / la_causal_forward_phi /
  la_decode_step_phi with LA_PHI_ELU1)
  la_workspace_bytes(op, B, Hq, Hkv, n, d, dtype, chunk)
  la_status_str(code)
Tensors are contiguous [B, H, n, d] (q, out: H = Hq; k, v: H = Hkv) in
float32 or bfloat16 on one GPU; states are float32.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblaphi.so")

LA_F32, LA_BF16 = 0, 1
LA_OP_FORWARD, LA_OP_CAUSAL, LA_OP_PREFIX_MASK, LA_OP_PREFIX_MASK_BATCHED = 0, 1, 2, 3
LA_PHI_RELU1, LA_PHI_ELU1 = 0, 1
_PHI = {"relu1": LA_PHI_RELU1, "elu1": LA_PHI_ELU1}


def _phi(phi):
    if phi not in _PHI:
        raise ValueError(f"phi must be one of {sorted(_PHI)}")
    return _PHI[phi]
STATUS_NAMES = ["LA_OK", "LA_ERR_NULL", "LA_ERR_SHAPE", "LA_ERR_DTYPE", "LA_ERR_UNSUPPORTED",
                "LA_ERR_WORKSPACE", "LA_ERR_ALIGN", "LA_ERR_ALIAS", "LA_ERR_LAUNCH"]

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
        for f in ("la_forward", "la_causal_forward", "la_prefix_mask_forward", "la_decode_step",
                  "la_forward_phi", "la_causal_forward_phi", "la_decode_step_phi", "la_prefix_mask_forward_batched"):
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


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


_ws_cache: dict = {}


def workspace(nbytes: int, device):
    """A device workspace of at least nbytes, cached per device and shared by
    every call on that device (its contents before a call do not matter)."""
    torch = _torch()
    key = (device.type, device.index)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


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
    if q is None:
        return S_final, z_final
    if want_state:
        return out, S_final, z_final
    return out


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
