"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle for the attention forward.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package.  The product path (the HIP library and its binding) never imports, links or runs
anything here, and this package imports nothing from the product path.

`attn_oracle.c` is the plain definition (see its header for the passages it follows);
this module only builds it with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "attn_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

_CODES = {"f32": 0, "f16": 1, "bf16": 2}


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle (gcc, fp64, OpenMP, no fast-math, no FMA contraction)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """ctypes view of one compiled copy of the oracle (the default one, or a test's own build)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_attn_rows_window.restype = ctypes.c_int
        lib.oracle_attn_rows_window.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.oracle_attn_bwd.restype = ctypes.c_int
        lib.oracle_attn_bwd.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.oracle_decode.restype = ctypes.c_double
        lib.oracle_decode.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64]
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        self.lib = lib
        self.path = path

    def attn_rows(self, q, k, v, dtype: str, scale, causal: bool = False, key_lens=None,
                  rows=None, nthreads: int = 0, window=None):
        """Reference O (fp64 [n, D]) and LSE (fp64 [n]) for flat row ids ((b*H+h)*Nq+i).

        q: [B,H,Nq,D]; k, v: [B,H,Nk,D] in storage form (bf16 as uint16 bits).
        `scale` is used exactly as given (pass the float32 value the GPU path receives).
        rows=None computes every row in order.  window=w keeps only keys with |i - j| <= w
        (None: no window).  causal: False/0, True/1 (top-left, j <= i) or 2 (bottom-right,
        j <= i + L_b - Nq: the queries are the last Nq positions of the key sequence).
        """
        q = _as_storage(q, dtype)
        k = _as_storage(k, dtype)
        v = _as_storage(v, dtype)
        B, H, Nq, D = q.shape
        Nk = k.shape[2]
        if k.shape != (B, H, Nk, D) or v.shape != (B, H, Nk, D):
            raise ValueError("k and v must be [B,H,Nk,D] matching q")
        kl = None
        if key_lens is not None:
            kl = np.ascontiguousarray(key_lens, dtype=np.int32)
            if kl.shape != (B,):
                raise ValueError("key_lens must be int32[B]")
        if rows is None:
            r = None
            n = B * H * Nq
        else:
            r = np.ascontiguousarray(rows, dtype=np.int64)
            n = r.size
        o = np.empty((n, D), dtype=np.float64)
        lse = np.empty(n, dtype=np.float64)
        w = -1 if window is None else int(window)
        if w < -1:
            raise ValueError("window must be None or >= 0")
        if int(causal) not in (0, 1, 2):
            raise ValueError("causal must be 0, 1 or 2")
        rc = self.lib.oracle_attn_rows_window(_ptr(q), _ptr(k), _ptr(v), _CODES[dtype], B, H, Nq,
                                              Nk, D, float(scale), int(causal), w, _ptr(kl),
                                              _ptr(r), n, _ptr(o), _ptr(lse), int(nthreads))
        if rc != 0:
            raise ValueError(f"oracle_attn_rows failed with {rc}")
        return o, lse

    def attn(self, q, k, v, dtype: str, scale, causal: bool = False, key_lens=None,
             nthreads: int = 0, window=None):
        """Reference O (fp64 [B,H,Nq,D]) and LSE (fp64 [B,H,Nq]) for every row."""
        B, H, Nq, D = q.shape
        o, lse = self.attn_rows(q, k, v, dtype, scale, causal, key_lens, None, nthreads, window)
        return o.reshape(B, H, Nq, D), lse.reshape(B, H, Nq)

    def attn_bwd(self, q, k, v, do, dtype: str, scale, causal: bool = False, key_lens=None,
                 dlse=None, bh=None, nthreads: int = 0, window=None):
        """Reference gradients dQ, dK, dV (fp64) of the attention forward.

        q, do: [B,H,Nq,D]; k, v: [B,H,Nk,D] in storage form (bf16 as uint16 bits); do is the
        gradient of the loss with respect to O.  dlse: float32 [B,H,Nq] gradient with respect
        to the LSE output, or None (zero).  causal: False/True (top-left).  bh: slice ids
        b*H + h to compute, or None for all.  window=w keeps only keys with |i - j| <= w (None:
        no band).  Returns dq [n,Nq,D], dk [n,Nk,D], dv [n,Nk,D] for the n selected slices,
        reshaped to [B,H,...] when bh is None.
        """
        q = _as_storage(q, dtype)
        k = _as_storage(k, dtype)
        v = _as_storage(v, dtype)
        do = _as_storage(do, dtype)
        B, H, Nq, D = q.shape
        Nk = k.shape[2]
        if k.shape != (B, H, Nk, D) or v.shape != (B, H, Nk, D) or do.shape != q.shape:
            raise ValueError("k, v must be [B,H,Nk,D] and do like q")
        if int(causal) not in (0, 1):
            raise ValueError("causal must be 0 or 1")
        kl = None if key_lens is None else np.ascontiguousarray(key_lens, dtype=np.int32)
        if kl is not None and kl.shape != (B,):
            raise ValueError("key_lens must be int32[B]")
        g = None if dlse is None else np.ascontiguousarray(dlse, dtype=np.float32)
        if g is not None and g.shape != (B, H, Nq):
            raise ValueError("dlse must be float32[B,H,Nq]")
        sel = None if bh is None else np.ascontiguousarray(bh, dtype=np.int64).reshape(-1)
        n = B * H if sel is None else sel.size
        dq = np.empty((n, Nq, D), np.float64)
        dk = np.empty((n, Nk, D), np.float64)
        dv = np.empty((n, Nk, D), np.float64)
        w = -1 if window is None else int(window)
        if w < -1:
            raise ValueError("window must be None or >= 0")
        rc = self.lib.oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(g), _CODES[dtype],
                                      B, H, Nq, Nk, D, float(scale), int(causal), w, _ptr(kl),
                                      _ptr(sel), n, _ptr(dq), _ptr(dk), _ptr(dv), int(nthreads))
        if rc != 0:
            raise ValueError(f"oracle_attn_bwd failed with {rc}")
        if sel is None:
            return dq.reshape(B, H, Nq, D), dk.reshape(B, H, Nk, D), dv.reshape(B, H, Nk, D)
        return dq, dk, dv

    def decode(self, a: np.ndarray, dtype: str) -> np.ndarray:
        """The oracle's own widening of stored values to fp64 (element by element)."""
        a = _as_storage(a, dtype)
        flat = a.reshape(-1)
        return np.array([self.lib.oracle_decode(_ptr(flat), _CODES[dtype], i)
                         for i in range(flat.size)])

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIB):
            build()
        _default = Oracle(LIB)
    return _default


def _ptr(a):
    return None if a is None else a.ctypes.data


def _as_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    want = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]
    if a.dtype != want:
        raise TypeError(f"{dtype} data must be stored as {np.dtype(want)}, got {a.dtype}")
    return np.ascontiguousarray(a)


def attn_rows(*a, **kw):
    return default().attn_rows(*a, **kw)


def attn(*a, **kw):
    return default().attn(*a, **kw)


def attn_bwd(*a, **kw):
    return default().attn_bwd(*a, **kw)


def decode(a, dtype):
    return default().decode(a, dtype)


def max_threads() -> int:
    return default().max_threads()
