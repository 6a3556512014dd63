"""Python access to the fp64 CPU oracle in ``gdn_oracle.c``.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the benchmark's
CPU-baseline leg are the only callers. The product library never imports this package.

The wrapper only marshals numpy arrays (float64, C-contiguous) into the C entry points; every
step of the arithmetic is in ``gdn_oracle.c``. See that file for the definitions and their
sources ("GDN tuning limits on Kunlun XPU", section 二 背景; the sliding-window low-rank state,
section 三.3).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "gdn_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add, every operation rounds as written in the source.
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc and return the path of the shared library."""
    cmd = ["gcc", *CFLAGS, "-o", output, source, "-lm"]
    subprocess.run(cmd, check=True)
    return output


_lib = None


def load(path: str | None = None):
    """Load (building first if absent) the oracle library; a path selects another build."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIBRARY):
            build()
        _lib = _declare(ctypes.CDLL(LIBRARY))
    return _lib


def _declare(lib):
    P = ctypes.c_void_p
    i64, i32, f64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    lib.oracle_gdn_decode.argtypes = [i64, i32, i32, i32, i32, P, P, P, P, P, P, P, f64]
    lib.oracle_gdn_decode.restype = ctypes.c_int
    lib.oracle_conv_gate.argtypes = [i64, i32, i32, i32, i32, P, P, P, P, P, P, f64,
                                     P, P, P, P, P]
    lib.oracle_conv_gate.restype = ctypes.c_int
    lib.oracle_gdn_conv_gate_decode.argtypes = [i64, i32, i32, i32, i32, P, P, P, P, P, P,
                                                P, P, f64, f64]
    lib.oracle_gdn_conv_gate_decode.restype = ctypes.c_int
    lib.oracle_gdn_lowrank_decode.argtypes = [i64, i32, i32, i32, i32, i32, P, P, P, P, P,
                                              P, P, P, P, P, f64]
    lib.oracle_gdn_lowrank_decode.restype = ctypes.c_int
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def gdn_decode(q, k, v, alpha, beta, state, scale: float = 1.0, lib=None):
    """Run T recurrent steps. Shapes: q,k [B,T,H,dk]; v [B,T,H,dv]; alpha,beta [B,T,H];
    state [B,H,dv,dk]. Returns (new_state, o [B,T,H,dv]) as new float64 arrays."""
    lib = lib or load()
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    S = _f64(state).copy()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape == (B, T, H, dv)
    assert alpha.shape == (B, T, H) and beta.shape == (B, T, H) and S.shape == (B, H, dv, dk)
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    rc = lib.oracle_gdn_decode(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                               _ptr(beta), _ptr(S), _ptr(o), float(scale))
    if rc != 0:
        raise ValueError("oracle_gdn_decode rejected its arguments")
    return S, o


def conv_gate(x, conv_state, conv_w, conv_b, a_logit, b_logit, H: int, dk: int, dv: int,
              l2_eps: float = 1e-6, lib=None):
    """The fused prologue alone. x [B,T,C]; conv_state [B,C,3]; conv_w [C,4]; conv_b [C] or
    None; logits [B,T,H]. Returns (q, k, v, alpha, beta, new_conv_state)."""
    lib = lib or load()
    x, a_logit, b_logit, conv_w = map(_f64, (x, a_logit, b_logit, conv_w))
    cb = None if conv_b is None else _f64(conv_b)
    cs = _f64(conv_state).copy()
    B, T, C = x.shape
    assert C == H * (2 * dk + dv) and cs.shape == (B, C, 3) and conv_w.shape == (C, 4)
    q = np.zeros((B, T, H, dk)); k = np.zeros((B, T, H, dk)); v = np.zeros((B, T, H, dv))
    al = np.zeros((B, T, H)); be = np.zeros((B, T, H))
    rc = lib.oracle_conv_gate(B, T, H, dk, dv, _ptr(x), _ptr(cs), _ptr(conv_w), _ptr(cb),
                              _ptr(a_logit), _ptr(b_logit), float(l2_eps),
                              _ptr(q), _ptr(k), _ptr(v), _ptr(al), _ptr(be))
    if rc != 0:
        raise ValueError("oracle_conv_gate rejected its arguments")
    return q, k, v, al, be, cs


def gdn_conv_gate_decode(x, conv_state, conv_w, conv_b, a_logit, b_logit, state, H: int,
                         dk: int, dv: int, scale: float = 1.0, l2_eps: float = 1e-6, lib=None):
    """The whole fused layer step. Returns (new_state, o, new_conv_state)."""
    lib = lib or load()
    x, a_logit, b_logit, conv_w = map(_f64, (x, a_logit, b_logit, conv_w))
    cb = None if conv_b is None else _f64(conv_b)
    cs = _f64(conv_state).copy()
    S = _f64(state).copy()
    B, T, C = x.shape
    assert C == H * (2 * dk + dv) and S.shape == (B, H, dv, dk)
    o = np.zeros((B, T, H, dv))
    rc = lib.oracle_gdn_conv_gate_decode(B, T, H, dk, dv, _ptr(x), _ptr(cs), _ptr(conv_w),
                                         _ptr(cb), _ptr(a_logit), _ptr(b_logit), _ptr(S),
                                         _ptr(o), float(scale), float(l2_eps))
    if rc != 0:
        raise ValueError("oracle_gdn_conv_gate_decode rejected its arguments")
    return S, o, cs


def gdn_lowrank_decode(q, k, v, alpha, beta, U, K, c, pos, scale: float = 1.0, lib=None):
    """T tokens on the sliding-window low-rank state. Shapes: q,k [B,T,H,dk]; v [B,T,H,dv];
    alpha,beta [B,T,H]; U [B,H,r,dv]; K [B,H,r,dk]; c [B,H,r]; pos [B,H] (int). Returns
    (U, K, c, pos, o [B,T,H,dv]) as new arrays (pos int32, the rest float64)."""
    lib = lib or load()
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    U, K, c = (_f64(a).copy() for a in (U, K, c))
    P = np.ascontiguousarray(np.asarray(pos, dtype=np.int32)).copy()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    r = U.shape[2]
    assert k.shape == q.shape and v.shape == (B, T, H, dv)
    assert alpha.shape == (B, T, H) and beta.shape == (B, T, H)
    assert U.shape == (B, H, r, dv) and K.shape == (B, H, r, dk) and c.shape == (B, H, r)
    assert P.shape == (B, H)
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    rc = lib.oracle_gdn_lowrank_decode(B, T, H, dk, dv, r, _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(alpha), _ptr(beta), _ptr(U), _ptr(K), _ptr(c),
                                       _ptr(P), _ptr(o), float(scale))
    if rc != 0:
        raise ValueError("oracle_gdn_lowrank_decode rejected its arguments")
    return U, K, c, P, o
