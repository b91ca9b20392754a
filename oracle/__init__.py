"""fp64 CPU oracle for the equivariant linear layers.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library.  It shares no code with the
GPU path.  The arithmetic lives in eqref.c (plain C loops, fp64); this module
builds it with gcc when needed and wraps it for numpy arrays.

What each function computes, and the passage it follows, is stated in eqref.c.
Counting helpers at the bottom restate the pages' operation counts
("Flash EQ-Linear", Algorithmic Approach and Specialization for p4;
"Quick ViTs", key design 2).

Parity status: every function here is pinned by tests/test_oracle.py against
library routines (numpy FFT, scipy circulant matrices, plain matmul), closed
forms, hand-derived examples and invariants.  No function is parity unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "eqref.c")
_LIB = os.path.join(_HERE, "libeqref.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False, sanitize: bool = False, out: str | None = None) -> str:
    """Compile eqref.c into a shared library with gcc (OpenMP, fp64, no fast-math)."""
    out = out or _LIB
    if not force and not sanitize and os.path.exists(out) and \
            os.path.getmtime(out) >= os.path.getmtime(_SRC):
        return out
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off"]
    if sanitize:
        cmd += ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    tmp = out + ".tmp%d" % os.getpid()
    cmd += [_SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = build()
        lib = ctypes.CDLL(path)
        d, i, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.eqref_num_threads.restype = i
        lib.eqref_cn_expand.argtypes = [i, i, i, d, d]
        lib.eqref_cn_expand.restype = None
        lib.eqref_apply_dense.argtypes = [i64, i64, i64, d, d, d]
        lib.eqref_apply_dense.restype = None
        lib.eqref_cn_dense.argtypes = [i, i, i, i64, d, d, d]
        lib.eqref_cn_dense.restype = i
        lib.eqref_cn_direct.argtypes = [i, i, i, i64, d, d, d]
        lib.eqref_cn_direct.restype = None
        lib.eqref_apply_dense_t.argtypes = [i64, i64, i64, d, d, d]
        lib.eqref_apply_dense_t.restype = None
        lib.eqref_cn_backward_data.argtypes = [i, i, i, i64, d, d, d]
        lib.eqref_cn_backward_data.restype = None
        lib.eqref_cn_backward_weight.argtypes = [i, i, i, i64, d, d, d]
        lib.eqref_cn_backward_weight.restype = None
        lib.eqref_bias_act.argtypes = [i64, i, i, d, i, d]
        lib.eqref_bias_act.restype = None
        lib.eqref_d8_fourier_matrix.argtypes = [d]
        lib.eqref_d8_fourier_matrix.restype = None
        lib.eqref_d8_to_regular.argtypes = [i64, i, d, d]
        lib.eqref_d8_to_regular.restype = None
        lib.eqref_d8_to_fourier.argtypes = [i64, i, d, d]
        lib.eqref_d8_to_fourier.restype = None
        lib.eqref_d8_bias_act.argtypes = [i64, i, d, i, d]
        lib.eqref_d8_bias_act.restype = None
        lib.eqref_dn_expand.argtypes = [i, i, i, d, d]
        lib.eqref_dn_expand.restype = None
        lib.eqref_dn_dense.argtypes = [i, i, i, i64, d, d, d]
        lib.eqref_dn_dense.restype = i
        lib.eqref_dn_fourier_matrix.argtypes = [i, d]
        lib.eqref_dn_fourier_matrix.restype = None
        lib.eqref_dn_to_regular.argtypes = [i, i64, i, d, d]
        lib.eqref_dn_to_regular.restype = None
        lib.eqref_dn_to_fourier.argtypes = [i, i64, i, d, d]
        lib.eqref_dn_to_fourier.restype = None
        lib.eqref_dn_bias_act.argtypes = [i, i64, i, d, i, d]
        lib.eqref_dn_bias_act.restype = None
        lib.eqref_cn_weight_dft.argtypes = [i, i, i, d, d]
        lib.eqref_cn_weight_dft.restype = None
        lib.eqref_d8_expand.argtypes = [i, i, d, d]
        lib.eqref_d8_expand.restype = None
        lib.eqref_d8_dense.argtypes = [i, i, i64, d, d, d]
        lib.eqref_d8_dense.restype = i
        _lib = lib
        return lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().eqref_num_threads())


def cn_expand(w):
    """Dense group-circulant matrix [(N*C_out), (N*C_in)] from w[C_out][C_in][N]."""
    w = _f64(w)
    C_out, C_in, N = w.shape
    W = np.empty((N * C_out, N * C_in), dtype=np.float64)
    _load().eqref_cn_expand(N, C_in, C_out, _p(w), _p(W))
    return W


def apply_dense(W, x2d):
    """y[t] = W @ x[t] for x2d[T][cols]."""
    W, x2d = _f64(W), _f64(x2d)
    T, cols = x2d.shape
    rows = W.shape[0]
    assert W.shape[1] == cols
    y = np.empty((T, rows), dtype=np.float64)
    _load().eqref_apply_dense(T, rows, cols, _p(W), _p(x2d), _p(y))
    return y


def cn_dense(x, w):
    """C_N layer by replicate-and-multiply; x[T][C_in][N], w[C_out][C_in][N]."""
    x, w = _f64(x), _f64(w)
    T, C_in, N = x.shape
    C_out = w.shape[0]
    assert w.shape == (C_out, C_in, N)
    y = np.empty((T, C_out, N), dtype=np.float64)
    if _load().eqref_cn_dense(N, C_in, C_out, T, _p(x), _p(w), _p(y)) != 0:
        raise MemoryError("oracle: cannot allocate the dense matrix")
    return y


def cn_direct(x, w):
    """C_N layer as the direct circular-convolution sum."""
    x, w = _f64(x), _f64(w)
    T, C_in, N = x.shape
    C_out = w.shape[0]
    assert w.shape == (C_out, C_in, N)
    y = np.empty((T, C_out, N), dtype=np.float64)
    _load().eqref_cn_direct(N, C_in, C_out, T, _p(x), _p(w), _p(y))
    return y


def apply_dense_t(W, dy2d):
    """dx[t] = W^T @ dy[t] for dy2d[T][rows]."""
    W, dy2d = _f64(W), _f64(dy2d)
    T, rows = dy2d.shape
    cols = W.shape[1]
    assert W.shape[0] == rows
    dx = np.empty((T, cols), dtype=np.float64)
    _load().eqref_apply_dense_t(T, rows, cols, _p(W), _p(dy2d), _p(dx))
    return dx


def cn_backward_data_dense(dy, w):
    """Input gradient of the C_N layer as W_dense^T dy; dy[T][C_out][N]."""
    dy = _f64(dy)
    T, C_out, N = dy.shape
    C_in = w.shape[1]
    assert w.shape == (C_out, C_in, N)
    dx = apply_dense_t(cn_expand(w), dy.reshape(T, C_out * N))
    return dx.reshape(T, C_in, N)


def cn_backward_data(dy, w):
    """Input gradient of the C_N layer, direct sum; dy[T][C_out][N] -> dx[T][C_in][N]."""
    dy, w = _f64(dy), _f64(w)
    T, C_out, N = dy.shape
    C_in = w.shape[1]
    assert w.shape == (C_out, C_in, N)
    dx = np.empty((T, C_in, N), dtype=np.float64)
    _load().eqref_cn_backward_data(N, C_in, C_out, T, _p(dy), _p(w), _p(dx))
    return dx


def cn_backward_weight(x, dy):
    """Weight gradient of the C_N layer; x[T][C_in][N], dy[T][C_out][N] -> dw[C_out][C_in][N]."""
    x, dy = _f64(x), _f64(dy)
    T, C_in, N = x.shape
    C_out = dy.shape[1]
    assert dy.shape == (T, C_out, N)
    dw = np.empty((C_out, C_in, N), dtype=np.float64)
    _load().eqref_cn_backward_weight(N, C_in, C_out, T, _p(x), _p(dy), _p(dw))
    return dw


def bias_act(y, bias=None, act=0):
    """act(y + bias[o]) along [T][C_out][N] (act 0: identity, 1: GELU, erf form); returns a copy."""
    y = np.array(y, dtype=np.float64, copy=True, order="C")
    T, C_out, N = y.shape
    b = None if bias is None else _f64(bias)
    if b is not None:
        assert b.shape == (C_out,)
    _load().eqref_bias_act(T, C_out, N, None if b is None else _p(b), int(act), _p(y))
    return y


def cn_dense_bias_act(x, w, bias=None, act=0):
    """The C_N layer followed by the fused neighbours: act(y + bias)."""
    return bias_act(cn_dense(x, w), bias, act)


def cn_weight_dft(w):
    """Packed real-DFT planes [N][C_out][C_in] of w[C_out][C_in][N]."""
    w = _f64(w)
    C_out, C_in, N = w.shape
    P = np.empty((N, C_out, C_in), dtype=np.float64)
    _load().eqref_cn_weight_dft(N, C_out, C_in, _p(w), _p(P))
    return P


def d8_fourier_matrix():
    """The orthonormal D8 Fourier matrix F[p][q] (coefficient p, group element q = a + 4b)."""
    F = np.empty((8, 8), dtype=np.float64)
    _load().eqref_d8_fourier_matrix(_p(F))
    return F


def d8_to_regular(v):
    """Fourier layout [T][8m] -> regular layout [T][m][8]."""
    v = _f64(v)
    T, C = v.shape
    assert C % 8 == 0
    f = np.empty((T, C // 8, 8), dtype=np.float64)
    _load().eqref_d8_to_regular(T, C // 8, _p(v), _p(f))
    return f


def d8_to_fourier(f):
    """Regular layout [T][m][8] -> Fourier layout [T][8m]."""
    f = _f64(f)
    T, m, e = f.shape
    assert e == 8
    v = np.empty((T, 8 * m), dtype=np.float64)
    _load().eqref_d8_to_fourier(T, m, _p(f), _p(v))
    return v


def d8_bias_act(y, bias=None, act=0):
    """The D8 round trip on Fourier features y[T][8m]: regular domain, act(f + bias[j]), back; a copy."""
    y = np.array(y, dtype=np.float64, copy=True, order="C")
    T, C = y.shape
    assert C % 8 == 0
    b = None if bias is None else _f64(bias)
    if b is not None:
        assert b.shape == (C // 8,)
    _load().eqref_d8_bias_act(T, C // 8, None if b is None else _p(b), int(act), _p(y))
    return y


def d8_dense_bias_act(x, wb, C_out, bias=None, act=0):
    """The D8 layer followed by its fused neighbours in the regular domain."""
    return d8_bias_act(d8_dense(x, wb, C_out), bias, act)


def dn_one_dim(n: int) -> int:
    return 4 if n % 2 == 0 else 2


def dn_two_dim(n: int) -> int:
    return n // 2 - 1 if n % 2 == 0 else (n - 1) // 2


def dn_params(n: int, C_in: int, C_out: int) -> int:
    """Parameters of the D_n layer: one square block per 1-D irrep, one 2m x 2m per E_k."""
    mi, mo = C_in // (2 * n), C_out // (2 * n)
    return dn_one_dim(n) * mi * mo + dn_two_dim(n) * (2 * mi) * (2 * mo)


def dn_expand(n, wb, C_in, C_out):
    wb = _f64(wb)
    assert C_in % (2 * n) == 0 and C_out % (2 * n) == 0 and wb.size == dn_params(n, C_in, C_out)
    W = np.empty((C_out, C_in), dtype=np.float64)
    _load().eqref_dn_expand(n, C_in, C_out, _p(wb), _p(W))
    return W


def dn_dense(n, x, wb, C_out):
    """D_n Fourier-domain layer on x[T][C_in] (the D8 layout generalised)."""
    x, wb = _f64(x), _f64(wb)
    T, C_in = x.shape
    assert wb.size == dn_params(n, C_in, C_out)
    y = np.empty((T, C_out), dtype=np.float64)
    if _load().eqref_dn_dense(n, C_in, C_out, T, _p(x), _p(wb), _p(y)) != 0:
        raise MemoryError("oracle: cannot allocate the dense matrix")
    return y


def dn_fourier_matrix(n):
    F = np.empty((2 * n, 2 * n), dtype=np.float64)
    _load().eqref_dn_fourier_matrix(n, _p(F))
    return F


def dn_to_regular(n, v):
    v = _f64(v)
    T, C = v.shape
    assert C % (2 * n) == 0
    f = np.empty((T, C // (2 * n), 2 * n), dtype=np.float64)
    _load().eqref_dn_to_regular(n, T, C // (2 * n), _p(v), _p(f))
    return f


def dn_to_fourier(n, f):
    f = _f64(f)
    T, m, g = f.shape
    assert g == 2 * n
    v = np.empty((T, g * m), dtype=np.float64)
    _load().eqref_dn_to_fourier(n, T, m, _p(f), _p(v))
    return v


def dn_bias_act(n, y, bias=None, act=0):
    y = np.array(y, dtype=np.float64, copy=True, order="C")
    T, C = y.shape
    assert C % (2 * n) == 0
    b = None if bias is None else _f64(bias)
    if b is not None:
        assert b.shape == (C // (2 * n),)
    _load().eqref_dn_bias_act(n, T, C // (2 * n), None if b is None else _p(b), int(act), _p(y))
    return y


def dn_dense_bias_act(n, x, wb, C_out, bias=None, act=0):
    return dn_bias_act(n, dn_dense(n, x, wb, C_out), bias, act)


def d8_expand(wb, C_in, C_out):
    wb = _f64(wb)
    assert wb.size == C_in * C_out // 8
    W = np.empty((C_out, C_in), dtype=np.float64)
    _load().eqref_d8_expand(C_in, C_out, _p(wb), _p(W))
    return W


def d8_dense(x, wb, C_out):
    """D8 Fourier-domain layer; x[T][C_in], wb packed [A1|A2|B1|B2|E]."""
    x, wb = _f64(x), _f64(wb)
    T, C_in = x.shape
    assert wb.size == C_in * C_out // 8
    y = np.empty((T, C_out), dtype=np.float64)
    if _load().eqref_d8_dense(C_in, C_out, T, _p(x), _p(wb), _p(y)) != 0:
        raise MemoryError("oracle: cannot allocate the dense matrix")
    return y


# --- counts -----------------------------------------------------------------
# Real GEMMs of size T x C_in x C_out in the half-spectrum method: the DC bin
# (and the Nyquist bin for even N) are real products; every other kept bin is
# a complex product = four real products.

def cn_kept_bins(N: int) -> int:
    return N // 2 + 1


def cn_real_gemms(N: int) -> int:
    complex_bins = (N - 1) // 2
    real_bins = 1 + (1 if N % 2 == 0 else 0)
    return real_bins + 4 * complex_bins


def cn_params(N: int, C_in: int, C_out: int) -> int:
    return N * C_in * C_out


def d8_params(C_in: int, C_out: int) -> int:
    mi, mo = C_in // 8, C_out // 8
    return 4 * mi * mo + (2 * mi) * (2 * mo)


def d8_mults(C_in: int, C_out: int) -> int:
    mi, mo = C_in // 8, C_out // 8
    return 4 * mi * mo + 2 * (2 * mi) * (2 * mo)
