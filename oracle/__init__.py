"""fp64 CPU oracle for kernelized linear attention -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  The product path (the HIP library and its Python
binding) never imports, links or calls it, and the two share no code.

The arithmetic lives in plain C (``la_oracle.c``, fp64, one sequential loop per
head, heads in parallel under OpenMP); this module only builds that library
with gcc, loads it with ctypes and marshals numpy arrays.  What each function
computes, with the passage it follows, is documented in ``la_oracle.h``.

Arrays are float64 numpy arrays of shape [..., N, d] (leading dimensions are
flattened into heads); bf16 / fp32 inputs are widened exactly by the caller.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblaoracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile la_oracle.c into liblaoracle.so with gcc (-O2, IEEE fp64, OpenMP)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, dp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.la_oracle_phi.restype = ctypes.c_double
    lib.la_oracle_phi.argtypes = [ctypes.c_double]
    lib.la_oracle_dphi.restype = ctypes.c_double
    lib.la_oracle_dphi.argtypes = [ctypes.c_double]
    for name in ("la_oracle_forward_noncausal", "la_oracle_forward_causal"):
        f = getattr(lib, name)
        f.restype = None
        f.argtypes = [i64, i64, i64, dp, dp, dp, dp, dp, dp, dp]
    for name in ("la_oracle_backward_causal", "la_oracle_backward_noncausal"):
        f = getattr(lib, name)
        f.restype = None
        f.argtypes = [i64, i64, i64, dp, dp, dp, dp, dp, dp, dp]
    lib.la_oracle_forward_causal_from.restype = None
    lib.la_oracle_forward_causal_from.argtypes = [i64, i64, i64, dp, dp, dp, dp, dp, dp, dp, dp, dp]
    lib.la_oracle_backward_causal_state.restype = None
    lib.la_oracle_backward_causal_state.argtypes = [i64, i64, i64] + [dp] * 13
    lib.la_oracle_favor_features.restype = None
    lib.la_oracle_favor_features.argtypes = [i64, i64, i64, dp, dp, dp]
    lib.la_oracle_forward_features.restype = None
    lib.la_oracle_forward_features.argtypes = [i64, i64, i64, i64, i32, dp, dp, dp, dp, dp, dp, dp]
    lib.la_oracle_backward_features.argtypes = [i64, i64, i64, i64, i32] + [dp] * 7
    lib.la_oracle_favor_features_backward.argtypes = [i64, i64, i64, dp, dp, dp, dp]
    lib.la_oracle_decode_step.restype = None
    lib.la_oracle_decode_step.argtypes = [i64, i64, dp, dp, dp, dp, dp, dp]
    lib.la_oracle_quadratic_forward.restype = None
    lib.la_oracle_quadratic_forward.argtypes = [i64, i64, i64, i32, dp, dp, dp, dp, dp]
    lib.la_oracle_quadratic_backward.restype = None
    lib.la_oracle_quadratic_backward.argtypes = [i64, i64, i64, i32, dp, dp, dp, dp, dp, dp, dp]
    lib.la_oracle_set_threads.restype = None
    lib.la_oracle_set_threads.argtypes = [i32]
    lib.la_oracle_get_threads.restype = i32
    lib.la_oracle_get_threads.argtypes = []
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _heads(x: np.ndarray):
    if x.ndim < 2:
        raise ValueError("expected [..., N, d]")
    n, d = x.shape[-2], x.shape[-1]
    bh = int(np.prod(x.shape[:-2])) if x.ndim > 2 else 1
    return bh, n, d


def set_threads(n: int) -> None:
    _load().la_oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().la_oracle_get_threads())


def phi(x: float) -> float:
    return float(_load().la_oracle_phi(float(x)))


def dphi(x: float) -> float:
    return float(_load().la_oracle_dphi(float(x)))


def _fwd(name, q, k, v, return_den, return_state):
    q, k, v = _f64(q), _f64(k), _f64(v)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must have the same shape")
    bh, n, d = _heads(q)
    o = np.empty_like(q)
    den = np.empty(q.shape[:-1], dtype=np.float64) if return_den else None
    S = np.empty(q.shape[:-2] + (d, d), dtype=np.float64) if return_state else None
    z = np.empty(q.shape[:-2] + (d,), dtype=np.float64) if return_state else None
    getattr(_load(), name)(bh, n, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den), _ptr(S), _ptr(z))
    out = [o]
    if return_den:
        out.append(den)
    if return_state:
        out += [S, z]
    return out[0] if len(out) == 1 else tuple(out)


def forward_causal(q, k, v, return_den=False, return_state=False, S0=None, z0=None):
    """Causal forward, recurrent form (returns o, [den], [S, z]).

    S0 [..., d, d] and z0 [..., d] (optional): the state the recurrence starts from."""
    if S0 is None and z0 is None:
        return _fwd("la_oracle_forward_causal", q, k, v, return_den, return_state)
    q, k, v = _f64(q), _f64(k), _f64(v)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must have the same shape")
    bh, n, d = _heads(q)
    S0 = None if S0 is None else _f64(S0)
    z0 = None if z0 is None else _f64(z0)
    if S0 is not None and S0.shape != q.shape[:-2] + (d, d):
        raise ValueError("S0 must be [..., d, d] matching q")
    if z0 is not None and z0.shape != q.shape[:-2] + (d,):
        raise ValueError("z0 must be [..., d] matching q")
    o = np.empty_like(q)
    den = np.empty(q.shape[:-1], dtype=np.float64) if return_den else None
    S = np.empty(q.shape[:-2] + (d, d), dtype=np.float64) if return_state else None
    z = np.empty(q.shape[:-2] + (d,), dtype=np.float64) if return_state else None
    _load().la_oracle_forward_causal_from(bh, n, d, _ptr(S0), _ptr(z0), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                          _ptr(den), _ptr(S), _ptr(z))
    out = [o]
    if return_den:
        out.append(den)
    if return_state:
        out += [S, z]
    return out[0] if len(out) == 1 else tuple(out)


def forward_noncausal(q, k, v, return_den=False, return_state=False):
    """Non-causal forward (returns o, [den], [S, z])."""
    return _fwd("la_oracle_forward_noncausal", q, k, v, return_den, return_state)


def _bwd(name, q, k, v, dout):
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    if not (q.shape == k.shape == v.shape == dout.shape):
        raise ValueError("q, k, v, dout must have the same shape")
    bh, n, d = _heads(q)
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    getattr(_load(), name)(bh, n, d, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv))
    return dq, dk, dv


def backward_causal(q, k, v, dout):
    """Gradients (dq, dk, dv) of sum(dout * forward_causal(q, k, v))."""
    return _bwd("la_oracle_backward_causal", q, k, v, dout)


def backward_causal_state(q, k, v, dout, S0=None, z0=None, dSN=None, dzN=None):
    """Gradients (dq, dk, dv, dS0, dz0) of sum(dout * o) + sum(dSN * S_N) + sum(dzN * z_N) for
    forward_causal(q, k, v, S0=S0, z0=z0) with final state (S_N, z_N)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    if not (q.shape == k.shape == v.shape == dout.shape):
        raise ValueError("q, k, v, dout must have the same shape")
    bh, n, d = _heads(q)
    st = q.shape[:-2]
    def opt(x, shape):
        if x is None:
            return None
        x = _f64(x)
        if x.shape != shape:
            raise ValueError(f"expected shape {shape}")
        return x
    S0, dSN = opt(S0, st + (d, d)), opt(dSN, st + (d, d))
    z0, dzN = opt(z0, st + (d,)), opt(dzN, st + (d,))
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    dS0, dz0 = np.empty(st + (d, d)), np.empty(st + (d,))
    _load().la_oracle_backward_causal_state(bh, n, d, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(S0), _ptr(z0),
                                            _ptr(dSN), _ptr(dzN), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dS0),
                                            _ptr(dz0))
    return dq, dk, dv, dS0, dz0


def backward_noncausal(q, k, v, dout):
    """Gradients (dq, dk, dv) of sum(dout * forward_noncausal(q, k, v))."""
    return _bwd("la_oracle_backward_noncausal", q, k, v, dout)


def decode_step(S, z, q, k, v):
    """One recurrent step; returns (o, S_new, z_new) and leaves the inputs untouched."""
    S, z = _f64(S).copy(), _f64(z).copy()
    q, k, v = _f64(q), _f64(k), _f64(v)
    d = q.shape[-1]
    bh = int(np.prod(q.shape[:-1])) if q.ndim > 1 else 1
    if S.shape != q.shape[:-1] + (d, d) or z.shape != q.shape:
        raise ValueError("state shapes do not match q")
    o = np.empty_like(q)
    _load().la_oracle_decode_step(bh, d, _ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(o))
    return o, S, z


def quadratic_forward(q, k, v, causal=True, return_den=False):
    """Brute-force O(N^2 d) form of the proof sketch (small inputs only)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    bh, n, d = _heads(q)
    o = np.empty_like(q)
    den = np.empty(q.shape[:-1], dtype=np.float64)
    _load().la_oracle_quadratic_forward(bh, n, d, int(bool(causal)), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den))
    return (o, den) if return_den else o


def quadratic_backward(q, k, v, dout, causal=True):
    """Brute-force gradients through the explicit n x n weights (small inputs only)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    bh, n, d = _heads(q)
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    _load().la_oracle_quadratic_backward(bh, n, d, int(bool(causal)), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                         _ptr(dq), _ptr(dk), _ptr(dv))
    return dq, dk, dv


def favor_features(x, omega):
    """FAVOR+ features m^{-1/2} exp(omega x - |x|^2/2) of the rows of x [..., d]; omega [m, d]."""
    x, omega = _f64(x), _f64(omega)
    d = x.shape[-1]
    if omega.ndim != 2 or omega.shape[1] != d:
        raise ValueError("omega must be [m, d]")
    m = omega.shape[0]
    rows = int(np.prod(x.shape[:-1])) if x.ndim > 1 else 1
    out = np.empty(x.shape[:-1] + (m,), dtype=np.float64)
    _load().la_oracle_favor_features(rows, d, m, _ptr(x), _ptr(omega), _ptr(out))
    return out


def forward_features(fq, fk, v, causal, return_den=False, return_state=False):
    """Linear attention on given features fq, fk [..., N, m] with values v [..., N, dv]."""
    fq, fk, v = _f64(fq), _f64(fk), _f64(v)
    if fq.shape != fk.shape or fq.shape[:-1] != v.shape[:-1]:
        raise ValueError("fq, fk must match, and share [..., N] with v")
    bh, n, m = _heads(fq)
    dv = v.shape[-1]
    o = np.empty(v.shape, dtype=np.float64)
    den = np.empty(fq.shape[:-1], dtype=np.float64) if return_den else None
    S = np.empty(fq.shape[:-2] + (m, dv), dtype=np.float64) if return_state else None
    z = np.empty(fq.shape[:-2] + (m,), dtype=np.float64) if return_state else None
    _load().la_oracle_forward_features(bh, n, m, dv, int(bool(causal)), _ptr(fq), _ptr(fk), _ptr(v), _ptr(o),
                                       _ptr(den), _ptr(S), _ptr(z))
    out = [o]
    if return_den:
        out.append(den)
    if return_state:
        out += [S, z]
    return out[0] if len(out) == 1 else tuple(out)


def backward_features(fq, fk, v, dout, causal):
    """Gradients (dfq, dfk, dv) of sum(dout * O) for forward_features(fq, fk, v, causal)."""
    fq, fk, v, dout = _f64(fq), _f64(fk), _f64(v), _f64(dout)
    if fq.shape != fk.shape or fq.shape[:-1] != v.shape[:-1] or dout.shape != v.shape:
        raise ValueError("fq, fk must match, and share [..., N] with v and dout")
    bh, n, m = _heads(fq)
    dv = v.shape[-1]
    dfq, dfk, dvo = np.empty(fq.shape), np.empty(fk.shape), np.empty(v.shape)
    _load().la_oracle_backward_features(bh, n, m, dv, int(bool(causal)), _ptr(fq), _ptr(fk), _ptr(v), _ptr(dout),
                                        _ptr(dfq), _ptr(dfk), _ptr(dvo))
    return dfq, dfk, dvo


def favor_features_backward(x, omega, dout):
    """Gradient with respect to x of sum(dout * favor_features(x, omega)); dout [..., m]."""
    x, omega, dout = _f64(x), _f64(omega), _f64(dout)
    d = x.shape[-1]
    m = omega.shape[0]
    if omega.shape != (m, d) or dout.shape != x.shape[:-1] + (m,):
        raise ValueError("omega must be [m, d] and dout [..., m]")
    rows = int(np.prod(x.shape[:-1])) if x.ndim > 1 else 1
    dx = np.empty(x.shape, dtype=np.float64)
    _load().la_oracle_favor_features_backward(rows, d, m, _ptr(x), _ptr(omega), _ptr(dout), _ptr(dx))
    return dx
