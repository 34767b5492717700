"""ctypes front end of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only users.  The product path (the HIP
library and its Python binding) never imports this package.

Functions take a problem dict as produced by
``nonlinear_rnn_evaluation_newton_amd.synthetic`` (float64 arrays holding the
stored values) and return float64 numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

OK, EINVAL, ENOMEM, NOT_CONVERGED, NONFINITE = 0, -1, -4, 1, 2
DENSE, DIAG, BLOCK2 = 0, 1, 2
NEWTON, QUASI, JACOBI = 0, 1, 2  # Jacobian used by a sweep: the cell's own, its diagonal, zero

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c (plain C, fp64, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", SRC, "-o", LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(LIB + ".tmp", LIB)
    return LIB


class _Model(C.Structure):
    _fields_ = [("cell", C.c_int), ("B", C.c_int), ("T", C.c_int), ("d", C.c_int), ("n", C.c_int),
                ("Wx", C.c_void_p), ("bx", C.c_void_p), ("Wh", C.c_void_p), ("bh", C.c_void_p),
                ("peep", C.c_void_p)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        lib = C.CDLL(LIB)
        P = C.c_void_p
        lib.orc_cell.argtypes = [P, P, P, P, P]
        lib.orc_cell_vjp.argtypes = [P, P, P, P, P, P]
        lib.orc_rollout.argtypes = [P, P, P, P]
        lib.orc_affine_solve.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, P, P, P]
        lib.orc_deer.argtypes = [P, P, P, C.c_double, C.c_int, P, P, P, P, C.c_int]
        lib.orc_deer_approx.argtypes = [P, C.c_int, P, P, C.c_double, C.c_int, P, P, P, P, C.c_int]
        lib.orc_adjoint.argtypes = [P] + [P] * 12
        lib.orc_lsim_discrete.argtypes = [C.c_int] * 5 + [P] * 8
        lib.orc_elk.argtypes = [P, C.c_double, P, P, C.c_double, C.c_int, P, P, P, P, C.c_int]
        lib.orc_elk_full.argtypes = [P, C.c_double, P, P, C.c_double, C.c_int, P, P, P, P, C.c_int]
        lib.orc_num_threads.restype = C.c_int
        _lib = lib
    return _lib


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


class _Bound:
    """Keeps the float64 copies alive while C holds their pointers."""

    def __init__(self, p: dict, B=None, T=None):
        self.keep = [_f64(p["W_x"]), _f64(p.get("b_x")), _f64(p["W_h"]), _f64(p.get("b_h")),
                     _f64(p.get("peep"))]
        self.m = _Model(p["cell"], p["B"] if B is None else B, p["T"] if T is None else T,
                        p["d"], p["n"], *[_ptr(a) for a in self.keep])

    @property
    def ref(self):
        return C.byref(self.m)


def _check(rc):
    if rc != OK:
        raise RuntimeError(f"oracle call failed with status {rc}")


def num_threads() -> int:
    return _load().orc_num_threads()


def jac_shape(p: dict) -> tuple:
    n, S = p["n"], p["S"]
    if p["cell"] == 2:
        return (S,)
    if p["cell"] == 3:
        return (n, 2, 2)
    return (S, S)


def cell(p: dict, s_prev, x_t):
    """One step: (f, J) at state s_prev [S] and input x_t [d]; J in the cell's structure."""
    lib = _load()
    bd = _Bound(p, B=1, T=1)
    s, xt = _f64(s_prev), _f64(x_t)
    f = np.zeros(p["S"])
    J = np.zeros(jac_shape(p))
    _check(lib.orc_cell(bd.ref, _ptr(s), _ptr(xt), _ptr(f), _ptr(J)))
    return f, J


def cell_vjp(p: dict, s_prev, x_t, lam):
    """One reverse step: (J^T lam, dU) by the chain rule."""
    lib = _load()
    bd = _Bound(p, B=1, T=1)
    s, xt, l = _f64(s_prev), _f64(x_t), _f64(lam)
    ds = np.zeros(p["S"])
    dU = np.zeros(p["G"] * p["n"])
    _check(lib.orc_cell_vjp(bd.ref, _ptr(s), _ptr(xt), _ptr(l), _ptr(ds), _ptr(dU)))
    return ds, dU


def rollout(p: dict, x=None, h0=None):
    """Sequential evaluation: h [B,T,S]."""
    lib = _load()
    x = _f64(p["x"] if x is None else x)
    h0 = _f64(p["h0"] if h0 is None else h0)
    B, T = x.shape[0], x.shape[1]
    bd = _Bound(p, B=B, T=T)
    h = np.zeros((B, T, p["S"]))
    _check(lib.orc_rollout(bd.ref, _ptr(x), _ptr(h0), _ptr(h)))
    return h


def deer(p: dict, tol=None, max_iters=None, x=None, h0=None, hist_cap=4096, approx=NEWTON):
    """CPU DEER: returns (h, iters, status, deltas[iters]).

    approx: NEWTON (the cell's Jacobian), QUASI (its diagonal) or JACOBI (zero).
    """
    lib = _load()
    x = _f64(p["x"] if x is None else x)
    h0 = _f64(p["h0"] if h0 is None else h0)
    B, T = x.shape[0], x.shape[1]
    tol = p["tol"] if tol is None else tol
    max_iters = p["max_iters"] if max_iters is None else max_iters
    bd = _Bound(p, B=B, T=T)
    h = np.zeros((B, T, p["S"]))
    it, st = C.c_int(0), C.c_int(0)
    deltas = np.zeros(hist_cap)
    _check(lib.orc_deer_approx(bd.ref, int(approx), _ptr(x), _ptr(h0), float(tol), int(max_iters), _ptr(h),
                               C.byref(it), C.byref(st), _ptr(deltas), hist_cap))
    return h, it.value, st.value, deltas[:min(it.value, hist_cap)].copy()


def elk(p: dict, lam: float, tol=None, max_iters=None, x=None, h0=None, hist_cap=4096):
    """Quasi-ELK (damping lam >= 0): returns (h, iters, status, deltas[iters])."""
    lib = _load()
    x = _f64(p["x"] if x is None else x)
    h0 = _f64(p["h0"] if h0 is None else h0)
    B, T = x.shape[0], x.shape[1]
    tol = p["tol"] if tol is None else tol
    max_iters = p["max_iters"] if max_iters is None else max_iters
    bd = _Bound(p, B=B, T=T)
    h = np.zeros((B, T, p["S"]))
    it, st = C.c_int(0), C.c_int(0)
    deltas = np.zeros(hist_cap)
    _check(lib.orc_elk(bd.ref, float(lam), _ptr(x), _ptr(h0), float(tol), int(max_iters), _ptr(h),
                       C.byref(it), C.byref(st), _ptr(deltas), hist_cap))
    return h, it.value, st.value, deltas[:min(it.value, hist_cap)].copy()


def elk_full(p: dict, lam: float, tol=None, max_iters=None, x=None, h0=None, hist_cap=4096):
    """ELK with the cell's own Jacobian (dense, 2x2 blocks or diagonal) and
    damping lam >= 0: returns (h, iters, status, deltas[iters])."""
    lib = _load()
    x = _f64(p["x"] if x is None else x)
    h0 = _f64(p["h0"] if h0 is None else h0)
    B, T = x.shape[0], x.shape[1]
    tol = p["tol"] if tol is None else tol
    max_iters = p["max_iters"] if max_iters is None else max_iters
    bd = _Bound(p, B=B, T=T)
    h = np.zeros((B, T, p["S"]))
    it, st = C.c_int(0), C.c_int(0)
    deltas = np.zeros(hist_cap)
    _check(lib.orc_elk_full(bd.ref, float(lam), _ptr(x), _ptr(h0), float(tol), int(max_iters), _ptr(h),
                            C.byref(it), C.byref(st), _ptr(deltas), hist_cap))
    return h, it.value, st.value, deltas[:min(it.value, hist_cap)].copy()


def adjoint(p: dict, h, g=None, x=None, h0=None):
    """Gradient of sum <g, h> through the recurrence at trajectory h.

    Returns a dict with lam [B,T,S], dx [B,T,d], dh0 [B,S], dW_x, db_x, dW_h,
    db_h and (LSTM) dpeep.
    """
    lib = _load()
    x = _f64(p["x"] if x is None else x)
    h0 = _f64(p["h0"] if h0 is None else h0)
    g = _f64(p["g"] if g is None else g)
    h = _f64(h)
    B, T = x.shape[0], x.shape[1]
    n, d, G, S = p["n"], p["d"], p["G"], p["S"]
    bd = _Bound(p, B=B, T=T)
    out = dict(lam=np.zeros((B, T, S)), dx=np.zeros((B, T, d)), dh0=np.zeros((B, S)),
               dW_x=np.zeros((G * n, d)), db_x=np.zeros(G * n),
               dW_h=np.zeros(np.shape(p["W_h"])), db_h=np.zeros(G * n),
               dpeep=np.zeros(2 * n) if p["cell"] == 3 else None)
    _check(lib.orc_adjoint(bd.ref, _ptr(x), _ptr(h0), _ptr(h), _ptr(g), _ptr(out["lam"]),
                           _ptr(out["dx"]), _ptr(out["dh0"]), _ptr(out["dW_x"]), _ptr(out["db_x"]),
                           _ptr(out["dW_h"]), _ptr(out["db_h"]), _ptr(out["dpeep"])))
    return out


def affine_solve(kind: int, A, b, reverse: bool = False):
    """Sequential y_t = A_t y_{t-1} + b_t (or reverse time), per sequence.

    DENSE: A [B,T,n,n], b [B,T,n]; DIAG: A, b [B,T,n]; BLOCK2: A [B,T,n,2,2], b [B,T,n,2].
    """
    lib = _load()
    A, b = _f64(A), _f64(b)
    B, T = b.shape[0], b.shape[1]
    n = b.shape[2]
    y = np.zeros_like(b)
    _check(lib.orc_affine_solve(kind, B, T, n, int(reverse), _ptr(A), _ptr(b), _ptr(y)))
    return y


def zoh(A, Bm, dt):
    """Zero-order-hold discretisation: Ad = exp(A dt), Bd = int_0^dt exp(A s) ds B,
    read off one matrix exponential of the augmented matrix [[A, B], [0, 0]] dt
    (scipy.linalg.expm)."""
    import scipy.linalg
    A, Bm = _f64(A), _f64(Bm)
    nx, m = Bm.shape
    M = np.zeros((nx + m, nx + m))
    M[:nx, :nx] = A * dt
    M[:nx, nx:] = Bm * dt
    E = scipy.linalg.expm(M)
    return E[:nx, :nx].copy(), E[:nx, nx:].copy()


def lsim(A, Bm, Cm, Dm, U, t, x0=None):
    """Linear state-space simulation dx/dt = A x + B u, y = C x + D u sampled at
    the uniform times t with the input held between samples (zero-order hold).

    U [B, T, m] (or [T, m]); x0 [B, nx] or None (= 0).  Returns (y [B, T, p],
    x [B, T, nx]) with x[:, k] the state at t[k]."""
    lib = _load()
    U = _f64(U)
    squeeze = U.ndim == 2
    if squeeze:
        U = U[None]
    Bn, T, m = U.shape
    A, Bm, Cm, Dm = _f64(A), _f64(Bm), _f64(Cm), _f64(Dm)
    nx, p = A.shape[0], Cm.shape[0]
    t = np.asarray(t, dtype=np.float64)
    dt = float(t[1] - t[0]) if T > 1 else 1.0
    if T > 2 and not np.allclose(np.diff(t), dt, rtol=1e-9, atol=0):
        raise ValueError("lsim needs uniformly spaced times")
    Ad, Bd = zoh(A, Bm, dt)
    x0 = None if x0 is None else _f64(np.broadcast_to(x0, (Bn, nx)))
    x = np.zeros((Bn, T, nx))
    y = np.zeros((Bn, T, p))
    _check(lib.orc_lsim_discrete(Bn, T, nx, m, p, _ptr(Ad), _ptr(Bd), _ptr(Cm), _ptr(Dm), _ptr(U), _ptr(x0),
                                 _ptr(x), _ptr(y)))
    return (y[0], x[0]) if squeeze else (y, x)
