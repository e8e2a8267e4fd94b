"""fp64 CPU oracle for kernelized linear attention (TEST INFRASTRUCTURE).

Only tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never imports, links or calls it, and it imports nothing from
the product.

The arithmetic lives in ``la_oracle.c`` (plain fp64 loops, OpenMP over
batch x head).  This module only builds that file with gcc and marshals
numpy arrays into it.  Inputs are fp32 arrays, or bf16 values passed as their
raw ``uint16`` bit patterns (widened exactly inside the C code).

What each function computes, and the web pages it follows, is stated in
``la_oracle.h`` / ``la_oracle.c``.  Every function is pinned by
``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
LIB_PATH = os.path.join(_HERE, "liblaoracle.so")
# LAO_LIBRARY names another build of la_oracle.c to load as it is (the
# host-sanitizer build the CPU tests make); by default the in-tree one,
# rebuilt when older than its source.
_OVERRIDE = os.environ.get("LAO_LIBRARY")

F32, BF16 = 0, 1

_lib = None


def build_sanitized(out: str) -> str:
    """Compile la_oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer
    (clang, shared ASan runtime, no OpenMP) into out, for the CPU tests that
    run the oracle's pins under the sanitizers."""
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
    cmd = [clang, "-O1", "-g", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-shared-libasan", _SRC, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def build(verbose: bool = False) -> str:
    """Compile la_oracle.c into liblaoracle.so (gcc -O2 -fopenmp, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", _SRC, "-o", LIB_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    global _lib
    _lib = None
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if _OVERRIDE:
            lib = ctypes.CDLL(_OVERRIDE)
        else:
            if not os.path.exists(LIB_PATH) or (
                    os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC)):
                build()
            lib = ctypes.CDLL(LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.lao_num_threads.restype = I
        lib.lao_forward.argtypes = [P, P, P, I, I, I64, I64, I64, I64, I64, P, I64, P]
        lib.lao_causal.argtypes = [P, P, P, I, I, I64, I64, I64, I64, I64, P, I64, P, P, P]
        lib.lao_prefix_mask.argtypes = [P, P, P, I, P, I64, I64, I64, I64, I64, P, I64, P]
        lib.lao_window.argtypes = [P, P, P, I, I, I64, I64, I64, I64, I64, I64, P, I64, P]
        lib.lao_window.restype = None
        lib.lao_causal_backward.argtypes = [P, P, P, P, I, I, I64, I64, I64, I64, I64, P, P, P]
        lib.lao_causal_backward.restype = None
        lib.lao_decode_step.argtypes = [P, P, P, I, I, I64, I64, I64, I64, P, P, P]
        for f in ("lao_forward", "lao_causal", "lao_prefix_mask", "lao_decode_step"):
            getattr(lib, f).restype = None

        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().lao_num_threads())


def _inp(x):
    """Return (contiguous array, dtype code) for an fp32, bf16-bits or fp64 input."""
    if x is None:
        return None, F32
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.float64:
        return x, 2
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError(f"oracle inputs must be float32 or uint16 (bf16 bits), got {x.dtype}")


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _rows(rows, n):
    if rows is None:
        return None, n
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if r.ndim != 1 or (r.size and (r.min() < 0 or r.max() >= n or np.any(np.diff(r) <= 0))):
        raise ValueError("rows must be strictly ascending indices in [0, n)")
    return r, r.size


def _check_gqa(qs, ks, vs):
    if (len(qs) != 4 or ks != vs or qs[0] != ks[0] or qs[2:] != ks[2:]
            or ks[1] < 1 or qs[1] % ks[1] != 0):
        raise ValueError(f"bad shapes q{qs} k{ks} v{vs}: need q [B,Hq,n,d], "
                         "k = v [B,Hkv,n,d], Hq a multiple of Hkv")


def _same_dtype(*codes):
    if len(set(c for c in codes)) != 1:
        raise TypeError("q, k and v must share one dtype")
    return codes[0]


_PHI = {"relu1": 0, "elu1": 1, "features": 2}
F64 = 2


def _phi(phi):
    """Feature-map code: "relu1", "elu1" or "features" (q and k hold phi(Q)
    and phi(K) already)."""
    if phi not in _PHI:
        raise ValueError(f"phi must be one of {sorted(_PHI)} or a function")
    return _PHI[phi]


def _mapped(x, phi):
    """A test's own feature map (a numpy function, applied elementwise)
    evaluated in fp64 on the stored values, as fp64 "features"."""
    if x is None:
        return None
    xf = (x.astype(np.uint32) << 16).view(np.float32) if x.dtype == np.uint16 else x
    return np.ascontiguousarray(phi(np.asarray(xf, dtype=np.float64)), dtype=np.float64)


def _with_map(q, k, v, phi):
    """(q, k, v, phi) with a callable phi applied here in fp64 to q and k (then
    "features"; v widened to fp64 too, so that the three share a dtype)."""
    if callable(phi):
        return _mapped(q, phi), _mapped(k, phi), _mapped(v, lambda x: x), "features"
    return q, k, v, phi


def forward(q, k, v, rows=None, phi="relu1"):
    """Non-causal normalised linear attention; q [B,Hq,n,d], k/v [B,Hkv,n,d].
    phi: "relu1" (relu(x) + 1), "elu1" (ELU(x) + 1), "features" (q and k hold
    phi(Q), phi(K) already) or a numpy function applied elementwise in fp64
    (a map of the caller's choice)."""
    q, k, v, phi = _with_map(q, k, v, phi)
    q, cq = _inp(q); k, ck = _inp(k); v, cv = _inp(v)
    dt = _same_dtype(cq, ck, cv)
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    _check_gqa(q.shape, k.shape, v.shape)
    r, nr = _rows(rows, n)
    out = np.empty((B, Hq, nr, d), dtype=np.float64)
    _load().lao_forward(_ptr(q), _ptr(k), _ptr(v), dt, _phi(phi), B, Hq, Hkv, n, d,
                        _ptr(r), nr, _ptr(out))
    return out


def causal(q, k, v, rows=None, want_state=False, Hq=None, phi="relu1"):
    """Causal normalised linear attention (query i sees keys 0..i).

    q may be None for a state-only pass (then pass Hq for the head count, or
    it defaults to Hkv).  With want_state the final (S [B,Hkv,d,d],
    z [B,Hkv,d]) are returned as well.
    """
    q, k, v, phi = _with_map(q, k, v, phi)
    k, ck = _inp(k); v, cv = _inp(v)
    B, Hkv, n, d = k.shape
    if q is not None:
        q, cq = _inp(q)
        dt = _same_dtype(cq, ck, cv)
        Hq = q.shape[1]
        _check_gqa(q.shape, k.shape, v.shape)
    else:
        dt = _same_dtype(ck, cv)
        Hq = Hq or Hkv
    r, nr = _rows(rows, n)
    out = None if q is None else np.empty((B, Hq, nr, d), dtype=np.float64)
    S = np.empty((B, Hkv, d, d), dtype=np.float64) if want_state else None
    z = np.empty((B, Hkv, d), dtype=np.float64) if want_state else None
    _load().lao_causal(_ptr(q), _ptr(k), _ptr(v), dt, _phi(phi), B, Hq, Hkv, n, d,
                       _ptr(r), nr, _ptr(out), _ptr(S), _ptr(z))
    if want_state:
        return out, S, z
    return out


def window(q, k, v, w, rows=None, phi="relu1"):
    """Sliding-window normalised linear attention: query i sees keys
    max(0, i - w + 1) .. i.  q [B,Hq,n,d], k/v [B,Hkv,n,d]; phi as forward."""
    q, k, v, phi = _with_map(q, k, v, phi)
    q, cq = _inp(q); k, ck = _inp(k); v, cv = _inp(v)
    dt = _same_dtype(cq, ck, cv)
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    _check_gqa(q.shape, k.shape, v.shape)
    if int(w) < 1:
        raise ValueError("the window must hold at least one key")
    r, nr = _rows(rows, n)
    out = np.empty((B, Hq, nr, d), dtype=np.float64)
    code = _phi(phi)
    _load().lao_window(_ptr(q), _ptr(k), _ptr(v), dt, code, B, Hq, Hkv, n, d, int(w), _ptr(r), nr, _ptr(out))
    return out


def causal_backward(q, k, v, dout, phi="relu1"):
    """Gradients (dq [B,Hq,n,d], dk, dv [B,Hkv,n,d], fp64) of the loss
    sum(dout * out) of the causal normalised form.  phi: "relu1", "elu1" or
    "features" (gradients with respect to the features themselves)."""
    q, cq = _inp(q); k, ck = _inp(k); v, cv = _inp(v); dout, co = _inp(dout)
    dt = _same_dtype(cq, ck, cv, co)
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    _check_gqa(q.shape, k.shape, v.shape)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(k.shape, dtype=np.float64)
    dv = np.empty(v.shape, dtype=np.float64)
    _load().lao_causal_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), dt, _phi(phi), B, Hq, Hkv, n, d,
                                _ptr(dq), _ptr(dk), _ptr(dv))
    return dq, dk, dv


def prefix_mask(q, k, v, m, rows=None):
    """Unnormalised Q K^T V with prefix mask m: query i of batch b sees keys
    0..m[i] (m of shape (n,), shared by the batches) or 0..m[b, i] (m of
    shape (B, n), one mask per batch)."""
    q, cq = _inp(q); k, ck = _inp(k); v, cv = _inp(v)
    dt = _same_dtype(cq, ck, cv)
    B, H, n, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("prefix_mask needs q, k and v of one shape [B,H,n,d]")
    m = np.ascontiguousarray(np.asarray(m, dtype=np.int64))
    if m.shape not in ((n,), (B, n)) or (n and (m.min() < 0 or m.max() >= n)):
        raise ValueError("m must have shape (n,) or (B, n) with values in [0, n)")
    r, nr = _rows(rows, n)
    out = np.empty((B, H, nr, d), dtype=np.float64)
    _load().lao_prefix_mask(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(m), 0 if m.ndim == 1 else n,
                            B, H, n, d, _ptr(r), nr, _ptr(out))
    return out


def decode_step(q, k, v, S, z, phi="relu1"):
    """One decode step: S [B,Hkv,d,d] and z [B,Hkv,d] (float64) update in place."""
    q, k, v, phi = _with_map(q, k, v, phi)
    q, cq = _inp(q); k, ck = _inp(k); v, cv = _inp(v)
    dt = _same_dtype(cq, ck, cv)
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    if (k.shape != v.shape or k.shape[0] != B or k.shape[2] != d or Hq % Hkv
            or S.shape != (B, Hkv, d, d) or z.shape != (B, Hkv, d)):
        raise ValueError("decode_step shapes: q [B,Hq,d], k = v [B,Hkv,d], "
                         "S [B,Hkv,d,d], z [B,Hkv,d]")
    if S.dtype != np.float64 or z.dtype != np.float64 or not (
            S.flags.c_contiguous and z.flags.c_contiguous):
        raise TypeError("S and z must be C-contiguous float64 arrays")
    out = np.empty((B, Hq, d), dtype=np.float64)
    _load().lao_decode_step(_ptr(q), _ptr(k), _ptr(v), dt, _phi(phi), B, Hq, Hkv, d,
                            _ptr(S), _ptr(z), _ptr(out))
    return out
