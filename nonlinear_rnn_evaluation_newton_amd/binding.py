"""Thin Python front end of libpararnn (include/pararnn.h).

Argument marshalling only: torch tensors are passed as raw device pointers
with the current HIP stream; every step of the solve runs in the library's
kernels.  There is no fallback: if the library is missing or a call fails,
this module raises.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpararnn.so")

# status codes (include/pararnn.h)
PR_OK, PR_EINVAL, PR_EWORKSPACE, PR_EHIP, PR_EUNSUPPORTED, PR_ELOOKBACK = 0, -1, -2, -3, -5, -6
PR_NOT_CONVERGED, PR_NONFINITE = 1, 2
PR_F32, PR_BF16 = 0, 1
PR_JAC_DENSE, PR_JAC_DIAG, PR_JAC_BLOCK2, PR_JAC_ZERO = 0, 1, 2, 3

EXPORTS = ["pararnn_workspace_bytes", "pararnn_solve", "pararnn_adjoint", "pararnn_solve_adjoint",
           "pararnn_scan_workspace_bytes", "pararnn_affine_scan", "pararnn_strerror", "pararnn_last_error", "pararnn_trace", "pararnn_trace_read",
           "pararnn_trace_kernel", "pararnn_lsim_workspace_bytes", "pararnn_lsim", "pararnn_elk_workspace_bytes",
           "pararnn_solve_elk", "pararnn_affine_scan_noalloc"]
NOALLOC_SCRATCH_BYTES = 16 << 20  # PR_NOALLOC_SCRATCH_BYTES


class Problem(C.Structure):
    _fields_ = [("cell", C.c_int), ("jac", C.c_int), ("dtype", C.c_int), ("B", C.c_int), ("T", C.c_int),
                ("d", C.c_int), ("n", C.c_int)]


class Weights(C.Structure):
    _fields_ = [("W_x", C.c_void_p), ("b_x", C.c_void_p), ("W_h", C.c_void_p), ("b_h", C.c_void_p),
                ("peep", C.c_void_p)]


class Grads(C.Structure):
    _fields_ = [("W_x", C.c_void_p), ("b_x", C.c_void_p), ("W_h", C.c_void_p), ("b_h", C.c_void_p),
                ("peep", C.c_void_p)]


class PararnnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} ({status}): {last_error()}")


_lib = None


def lib():
    """Load libpararnn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = C.CDLL(LIB_PATH)
        P, I, F, S = C.c_void_p, C.c_int, C.c_float, C.c_size_t
        L.pararnn_workspace_bytes.argtypes = [P, I]
        L.pararnn_workspace_bytes.restype = S
        L.pararnn_solve.argtypes = [P, P, P, P, F, I, P, P, P, I, P, S, P]
        L.pararnn_solve.restype = I
        L.pararnn_adjoint.argtypes = [P, P, P, P, P, P, P, P, P, P, P, S, P]
        L.pararnn_adjoint.restype = I
        L.pararnn_solve_adjoint.argtypes = [P, P, P, P, F, I, P, P, P, I, P, P, P, P, P, P, S, P]
        L.pararnn_solve_adjoint.restype = I
        L.pararnn_scan_workspace_bytes.argtypes = [I, I, I, I]
        L.pararnn_scan_workspace_bytes.restype = S
        L.pararnn_affine_scan.argtypes = [I, I, I, I, I, P, P, P, P, S, P]
        L.pararnn_affine_scan.restype = I
        L.pararnn_affine_scan_noalloc.argtypes = [I, I, I, I, I, P, P, P, P]
        L.pararnn_affine_scan_noalloc.restype = I
        L.pararnn_strerror.argtypes = [I]
        L.pararnn_strerror.restype = C.c_char_p
        L.pararnn_last_error.argtypes = []
        L.pararnn_last_error.restype = C.c_char_p
        L.pararnn_trace.argtypes = [I]
        L.pararnn_trace.restype = I
        L.pararnn_trace_read.argtypes = [P, P, P, P]
        L.pararnn_trace_read.restype = I
        L.pararnn_trace_kernel.argtypes = [I, P, P]
        L.pararnn_trace_kernel.restype = I
        L.pararnn_lsim_workspace_bytes.argtypes = [I, I, I, I, I]
        L.pararnn_lsim_workspace_bytes.restype = S
        L.pararnn_lsim.argtypes = [I, I, I, I, I, P, P, P, P, F, P, P, P, P, P, S, P]
        L.pararnn_lsim.restype = I
        L.pararnn_elk_workspace_bytes.argtypes = [P]
        L.pararnn_elk_workspace_bytes.restype = S
        L.pararnn_solve_elk.argtypes = [P, P, P, P, F, F, I, P, P, P, I, P, S, P]
        L.pararnn_solve_elk.restype = I
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().pararnn_strerror(status).decode()


def last_error() -> str:
    return lib().pararnn_last_error().decode()


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_problem(cell, jac, dtype, B, T, d, n) -> Problem:
    return Problem(cell, jac, dtype, B, T, d, n)


def make_weights(W_x, b_x, W_h, b_h, peep=None) -> Weights:
    return Weights(_p(W_x), _p(b_x), _p(W_h), _p(b_h), _p(peep))


def workspace_bytes(prob: Problem, with_adjoint: bool = True) -> int:
    return lib().pararnn_workspace_bytes(C.byref(prob), int(with_adjoint))


def solve(prob: Problem, w: Weights, x, h0, tol: float, max_iters: int, h, workspace, hist_cap: int = 64,
          check: bool = True):
    """Runs pararnn_solve; returns (status, iters, delta history)."""
    it = C.c_int(0)
    hist = np.zeros(max(hist_cap, 1), dtype=np.float32)
    st = lib().pararnn_solve(C.byref(prob), C.byref(w), _p(x), _p(h0), float(tol), int(max_iters), _p(h),
                             C.byref(it), hist.ctypes.data_as(C.c_void_p), int(hist_cap), _p(workspace),
                             workspace.numel() * workspace.element_size(), _stream())
    if check and st < 0:
        raise PararnnError(st, "pararnn_solve")
    return st, it.value, hist[:min(it.value, hist_cap)].copy()


def elk_workspace_bytes(prob: Problem) -> int:
    return lib().pararnn_elk_workspace_bytes(C.byref(prob))


def solve_elk(prob: Problem, w: Weights, x, h0, lam: float, tol: float, max_iters: int, h, workspace,
              hist_cap: int = 64, check: bool = True):
    """Runs pararnn_solve_elk (quasi-ELK, damping lam); returns (status, iters, delta history)."""
    it = C.c_int(0)
    hist = np.zeros(max(hist_cap, 1), dtype=np.float32)
    st = lib().pararnn_solve_elk(C.byref(prob), C.byref(w), _p(x), _p(h0), float(lam), float(tol), int(max_iters),
                                 _p(h), C.byref(it), hist.ctypes.data_as(C.c_void_p), int(hist_cap), _p(workspace),
                                 workspace.numel() * workspace.element_size(), _stream())
    if check and st < 0:
        raise PararnnError(st, "pararnn_solve_elk")
    return st, it.value, hist[:min(it.value, hist_cap)].copy()


def adjoint(prob: Problem, w: Weights, x, h0, h, g, workspace, lam=None, dx=None, dh0=None, grads: dict | None = None,
            check: bool = True) -> int:
    gr = None
    if grads is not None:
        gr = Grads(*[_p(grads.get(k)) for k in ("W_x", "b_x", "W_h", "b_h", "peep")])
    st = lib().pararnn_adjoint(C.byref(prob), C.byref(w), _p(x), _p(h0), _p(h), _p(g), _p(lam), _p(dx), _p(dh0),
                               C.byref(gr) if gr is not None else None, _p(workspace),
                               workspace.numel() * workspace.element_size(), _stream())
    if check and st < 0:
        raise PararnnError(st, "pararnn_adjoint")
    return st


def solve_adjoint(prob: Problem, w: Weights, x, h0, tol: float, max_iters: int, h, g, workspace, lam=None, dx=None,
                  dh0=None, grads: dict | None = None, hist_cap: int = 64, check: bool = True):
    """Runs pararnn_solve_adjoint; returns (status, iters, delta history)."""
    it = C.c_int(0)
    hist = np.zeros(max(hist_cap, 1), dtype=np.float32)
    gr = None
    if grads is not None:
        gr = Grads(*[_p(grads.get(k)) for k in ("W_x", "b_x", "W_h", "b_h", "peep")])
    st = lib().pararnn_solve_adjoint(C.byref(prob), C.byref(w), _p(x), _p(h0), float(tol), int(max_iters), _p(h),
                                     C.byref(it), hist.ctypes.data_as(C.c_void_p), int(hist_cap), _p(g), _p(lam),
                                     _p(dx), _p(dh0), C.byref(gr) if gr is not None else None, _p(workspace),
                                     workspace.numel() * workspace.element_size(), _stream())
    if check and st < 0:
        raise PararnnError(st, "pararnn_solve_adjoint")
    return st, it.value, hist[:min(it.value, hist_cap)].copy()


def trace(enable: bool) -> None:
    st = lib().pararnn_trace(int(enable))
    if st < 0:
        raise PararnnError(st, "pararnn_trace")


def trace_read() -> dict:
    sm, sl, am, al = C.c_double(0), C.c_longlong(0), C.c_double(0), C.c_longlong(0)
    st = lib().pararnn_trace_read(C.byref(sm), C.byref(sl), C.byref(am), C.byref(al))
    if st < 0:
        raise PararnnError(st, "pararnn_trace_read")
    return dict(sweep_ms=sm.value, sweep_launches=sl.value, adjoint_ms=am.value, adjoint_launches=al.value)


TRACE_SWEEP, TRACE_ADJOINT, TRACE_PROJECTION, TRACE_ADJOINT_PRODUCTS, TRACE_DENSE_PRODUCTS = 0, 1, 2, 3, 4
TRACE_LSIM = 5


def trace_kernel(which: int):
    """(total ms, launches) of one traced category."""
    ms, n = C.c_double(0), C.c_longlong(0)
    st = lib().pararnn_trace_kernel(int(which), C.byref(ms), C.byref(n))
    if st < 0:
        raise PararnnError(st, "pararnn_trace_kernel")
    return ms.value, n.value


def scan_workspace_bytes(jac: int, B: int, T: int, n: int) -> int:
    return lib().pararnn_scan_workspace_bytes(jac, B, T, n)


def affine_scan(jac: int, A, b, y, workspace, reverse: bool = False, check: bool = True) -> int:
    B, T, n = b.shape[0], b.shape[1], b.shape[2]
    st = lib().pararnn_affine_scan(jac, B, T, n, int(reverse), _p(A), _p(b), _p(y), _p(workspace),
                                   workspace.numel() * workspace.element_size(), _stream())
    if check and st < 0:
        raise PararnnError(st, "pararnn_affine_scan")
    return st


def affine_scan_noalloc(jac: int, A, b, y, reverse: bool = False, check: bool = True) -> int:
    """pararnn_affine_scan_noalloc: the same scan with the library's static
    device scratch instead of a workspace."""
    B, T, n = b.shape[0], b.shape[1], b.shape[2]
    st = lib().pararnn_affine_scan_noalloc(jac, B, T, n, int(reverse), _p(A), _p(b), _p(y), _stream())
    if check and st < 0:
        raise PararnnError(st, "pararnn_affine_scan_noalloc")
    return st


def lsim_workspace_bytes(B: int, T: int, nx: int, m: int, p: int) -> int:
    return lib().pararnn_lsim_workspace_bytes(B, T, nx, m, p)


def lsim(A, Bm, Cm, Dm, dt: float, U, x0, x, y, workspace, check: bool = True) -> int:
    """pararnn_lsim on fp32 device tensors: U [B,T,m], x0 [B,nx] or None,
    outputs x [B,T,nx] (or None) and y [B,T,p]."""
    import torch
    for name, t in (("A", A), ("B", Bm), ("C", Cm), ("D", Dm), ("U", U), ("x0", x0), ("x", x), ("y", y)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError(f"lsim: {name} must be a contiguous float32 tensor, got {t.dtype}")
    B, T, m = U.shape[0], U.shape[1], U.shape[2]
    nx, p = A.shape[0], Cm.shape[0]
    st = lib().pararnn_lsim(B, T, nx, m, p, _p(A), _p(Bm), _p(Cm), _p(Dm), float(dt), _p(U), _p(x0), _p(x), _p(y),
                            _p(workspace), workspace.numel() * workspace.element_size(), _stream())
    if check and st < 0:
        raise PararnnError(st, "pararnn_lsim")
    return st


# ---------------------------------------------------------------------------
# moving a problem (as drawn by synthetic.py) to the device
# ---------------------------------------------------------------------------
class DeviceProblem:
    """Device copies of a synthetic problem in its storage dtype, plus a workspace."""

    def __init__(self, p: dict, device="cuda", with_adjoint: bool = True, elk: bool = False):
        import torch
        from . import synthetic as sy
        self.p = p
        self.device = device
        self.prob = make_problem(p["cell"], p["jac"], p["dtype"], p["B"], p["T"], p["d"], p["n"])
        self.tdtype = torch.bfloat16 if p["dtype"] == PR_BF16 else torch.float32

        def up(a):
            if a is None:
                return None
            st = sy.to_storage(np.asarray(a), p["dtype"])
            if p["dtype"] == PR_BF16:
                return torch.from_numpy(st.view(np.int16).copy()).to(device).view(torch.bfloat16)
            return torch.from_numpy(st.copy()).to(device)

        self.W_x, self.b_x, self.W_h, self.b_h = up(p["W_x"]), up(p["b_x"]), up(p["W_h"]), up(p["b_h"])
        self.peep = up(p["peep"])
        self.x = up(p["x"])
        self.h0 = up(p["h0"])
        self.g = up(p["g"]) if p.get("g") is not None else None
        self.w = make_weights(self.W_x, self.b_x, self.W_h, self.b_h, self.peep)
        nbytes = workspace_bytes(self.prob, with_adjoint)
        if nbytes == 0:
            raise RuntimeError(f"pararnn_workspace_bytes: {last_error()}")
        if elk:
            nbytes = elk_workspace_bytes(self.prob)
            if nbytes == 0:
                raise RuntimeError(f"pararnn_elk_workspace_bytes: {last_error()}")
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.h = torch.empty((p["B"], p["T"], p["S"]), dtype=self.tdtype, device=device)

    def solve(self, tol=None, max_iters=None, hist_cap=64, check=True):
        p = self.p
        tol = p["tol"] if tol is None else tol
        max_iters = p["max_iters"] if max_iters is None else max_iters
        return solve(self.prob, self.w, self.x, self.h0, tol, max_iters, self.h, self.ws, hist_cap, check)

    def solve_elk(self, lam, tol=None, max_iters=None, hist_cap=64, check=True):
        p = self.p
        tol = p["tol"] if tol is None else tol
        max_iters = p["max_iters"] if max_iters is None else max_iters
        return solve_elk(self.prob, self.w, self.x, self.h0, lam, tol, max_iters, self.h, self.ws, hist_cap, check)

    def adjoint(self, h=None, g=None, want_grads=True, check=True):
        import torch
        p = self.p
        h = self.h if h is None else h
        g = self.g if g is None else g
        lam = torch.empty_like(h)
        dx = torch.empty_like(self.x)
        dh0 = torch.empty((p["B"], p["S"]), dtype=self.tdtype, device=self.device)
        grads = None
        if want_grads:
            f32 = dict(dtype=torch.float32, device=self.device)
            grads = dict(W_x=torch.empty(tuple(self.W_x.shape), **f32), b_x=torch.empty(tuple(self.b_x.shape), **f32),
                         W_h=torch.empty(tuple(self.W_h.shape), **f32), b_h=torch.empty(tuple(self.b_h.shape), **f32))
            if self.peep is not None:
                grads["peep"] = torch.empty(tuple(self.peep.shape), **f32)
        st = adjoint(self.prob, self.w, self.x, self.h0, h, g, self.ws, lam, dx, dh0, grads, check)
        return st, dict(lam=lam, dx=dx, dh0=dh0, **({} if grads is None else {"d" + k: v for k, v in grads.items()}))
