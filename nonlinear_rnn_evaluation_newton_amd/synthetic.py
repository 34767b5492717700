"""Seeded synthetic workloads for the DEER / quasi-DEER Newton solver.

This module only draws random numbers and rounds them to a storage format.
It holds none of the method's arithmetic, imports nothing from the rest of the
package, and is shared by the tests, the benchmark and the fp64 oracle harness.

The five workloads follow the settings quoted for DEER-style evaluation:
a small tanh RNN with a dense 4x4 Jacobian; the scalar-state GRU at length 2^20
and batch 16 that the DEER paper times on a V100 ("Parallelizing non-linear
sequential models over the sequence length", Key results); a diagonal ParaGRU
and a CIFG/peephole ParaLSTM of the kind the Para-Seq README lists in its
"Main features" table; and a dense GRU with n = 64, where the DEER summary notes
the speedup collapses ("Surprising findings").

Draw order per workload (fp64, ``numpy.random.default_rng(seed)``):
input weights W_x; recurrent weights (gate order); peepholes; biases (only the
scalar GRU draws them); x; the upstream gradient g.  Values are then rounded
to the storage dtype (bf16 round-to-nearest-even for the bf16 workloads), and
every array handed out holds exactly the stored values as float64.
"""
from __future__ import annotations

import numpy as np

# Cell codes (same numbering as the C ABI).
CELL_TANH_RNN = 0
CELL_GRU = 1
CELL_GRU_DIAG = 2
CELL_LSTM_CIFG_DIAG = 3
CELL_LINEAR = 4

JAC_DENSE = 0
JAC_DIAG = 1
JAC_BLOCK2 = 2
JAC_ZERO = 3  # Jacobi sweeps (no Jacobian in the linear solve)

DT_F32 = 0
DT_BF16 = 1

CELL_NAMES = {
    CELL_TANH_RNN: "tanh_rnn",
    CELL_GRU: "gru",
    CELL_GRU_DIAG: "gru_diag",
    CELL_LSTM_CIFG_DIAG: "lstm_cifg_diag",
    CELL_LINEAR: "linear",
}


def n_gates(cell: int) -> int:
    return 3 if cell in (CELL_GRU, CELL_GRU_DIAG, CELL_LSTM_CIFG_DIAG) else 1


def state_width(cell: int, n: int) -> int:
    return 2 * n if cell == CELL_LSTM_CIFG_DIAG else n


def natural_jac(cell: int) -> int:
    if cell == CELL_GRU_DIAG:
        return JAC_DIAG
    if cell == CELL_LSTM_CIFG_DIAG:
        return JAC_BLOCK2
    return JAC_DENSE


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def round_storage(a: np.ndarray, dtype: int) -> np.ndarray:
    """Round fp64 values to what the storage dtype holds, returned as fp64."""
    if dtype == DT_BF16:
        return bf16_to_f64(bf16_bits(a))
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def to_storage(a: np.ndarray, dtype: int) -> np.ndarray:
    """fp64 values (already representable) -> the array the device stores."""
    if dtype == DT_BF16:
        return bf16_bits(a)
    return np.ascontiguousarray(a, dtype=np.float32)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
WORKLOADS = {
    1: dict(name="dense_tanh_rnn_n4", cell=CELL_TANH_RNN, B=2, T=256, d=2, n=4,
            dtype=DT_F32, tol=1e-6, max_iters=None),
    2: dict(name="gru_scalar_T1M", cell=CELL_GRU, B=16, T=1 << 20, d=1, n=1,
            dtype=DT_F32, tol=1e-6, max_iters=None),
    3: dict(name="paragru_diag_bf16", cell=CELL_GRU_DIAG, B=8, T=4096, d=1024, n=1024,
            dtype=DT_BF16, tol=0.0, max_iters=4),
    4: dict(name="paralstm_cifg_block2_bf16", cell=CELL_LSTM_CIFG_DIAG, B=4, T=8192, d=2048,
            n=2048, dtype=DT_BF16, tol=0.0, max_iters=4),
    5: dict(name="dense_gru_n64", cell=CELL_GRU, B=16, T=16384, d=32, n=64,
            dtype=DT_F32, tol=1e-5, max_iters=None),
}


def make_problem(cfg: int, seed: int | None = None, B: int | None = None, T: int | None = None,
                 d: int | None = None, n: int | None = None, with_g: bool = True) -> dict:
    """Draw workload ``cfg`` (1..5), optionally at reduced sizes.

    Returns a dict of plain Python / float64 numpy values.  ``max_iters``
    defaults to T when the workload runs to tolerance.
    """
    w = dict(WORKLOADS[cfg])
    B = w["B"] if B is None else B
    T = w["T"] if T is None else T
    d = w["d"] if d is None else d
    n = w["n"] if n is None else n
    cell, dtype = w["cell"], w["dtype"]
    G, S = n_gates(cell), state_width(cell, n)
    rng = np.random.default_rng(cfg if seed is None else seed)

    bx = np.zeros(G * n)
    bh = np.zeros(G * n)
    peep = None
    if cfg == 1:
        Wx = rng.normal(0.0, np.sqrt(1.0 / d), size=(n, d))
        Wh = rng.normal(0.0, np.sqrt(0.25 / n), size=(n, n))
    elif cfg == 2:
        Wx = rng.uniform(-1.0, 1.0, size=(3 * n, d))
        Wh = rng.uniform(-1.0, 1.0, size=(3 * n, n))
        bx = rng.uniform(-1.0, 1.0, size=3 * n)
        bh = rng.uniform(-1.0, 1.0, size=3 * n)
    elif cfg == 3:
        Wx = rng.normal(0.0, np.sqrt(1.0 / d), size=(3 * n, d))
        Wh = rng.uniform(-0.9, 0.9, size=3 * n)
    elif cfg == 4:
        Wx = rng.normal(0.0, np.sqrt(1.0 / d), size=(3 * n, d))
        Wh = rng.uniform(-0.5, 0.5, size=3 * n)
        peep = rng.uniform(-0.5, 0.5, size=2 * n)
    elif cfg == 5:
        Wx = rng.normal(0.0, np.sqrt(1.0 / d), size=(3 * n, d))
        Wh = rng.normal(0.0, np.sqrt(0.5 / n), size=(3 * n, n))
    else:
        raise ValueError(f"unknown workload {cfg}")
    x = rng.standard_normal(size=(B, T, d))
    g = None
    if with_g:
        if cell == CELL_LSTM_CIFG_DIAG:
            gh = rng.standard_normal(size=(B, T, n))
            g = np.zeros((B, T, S))
            g[..., 1::2] = gh           # the loss only sees h; dL/dc = 0
        else:
            g = rng.standard_normal(size=(B, T, S))

    r = lambda a: None if a is None else round_storage(a, dtype)
    max_iters = w["max_iters"] if w["max_iters"] is not None else T
    return dict(cfg=cfg, name=w["name"], cell=cell, jac=natural_jac(cell), dtype=dtype,
                B=B, T=T, d=d, n=n, G=G, S=S,
                W_x=r(Wx), b_x=r(bx), W_h=r(Wh), b_h=r(bh), peep=r(peep),
                x=r(x), g=r(g), h0=np.zeros((B, S)),
                tol=w["tol"], max_iters=max_iters)


def custom_problem(cell: int, B: int, T: int, d: int, n: int, seed: int = 0,
                   w_scale: float = 1.0, dtype: int = DT_F32, bias: bool = True,
                   h0: bool = False) -> dict:
    """A generic random problem for edge-case and property tests.

    Recurrent weights ~ N(0, w_scale^2/n) (dense) or U(-w_scale, w_scale)
    (diagonal); input weights ~ N(0, 1/d); biases ~ U(-0.5, 0.5) when
    ``bias``; x, g ~ N(0, 1); h0 ~ U(-0.5, 0.5) when ``h0`` else zero.
    """
    G, S = n_gates(cell), state_width(cell, n)
    rng = np.random.default_rng(seed)
    Wx = rng.normal(0.0, np.sqrt(1.0 / d), size=(G * n, d))
    if cell in (CELL_GRU_DIAG, CELL_LSTM_CIFG_DIAG):
        Wh = rng.uniform(-w_scale, w_scale, size=G * n)
    else:
        Wh = rng.normal(0.0, w_scale / np.sqrt(n), size=(G * n, n))
    peep = rng.uniform(-w_scale, w_scale, size=2 * n) if cell == CELL_LSTM_CIFG_DIAG else None
    if bias:
        bx = rng.uniform(-0.5, 0.5, size=G * n)
        bh = rng.uniform(-0.5, 0.5, size=G * n)
    else:
        bx, bh = np.zeros(G * n), np.zeros(G * n)
    x = rng.standard_normal(size=(B, T, d))
    g = rng.standard_normal(size=(B, T, S))
    hz = rng.uniform(-0.5, 0.5, size=(B, S)) if h0 else np.zeros((B, S))
    r = lambda a: None if a is None else round_storage(a, dtype)
    return dict(cfg=0, name=f"custom_{CELL_NAMES[cell]}", cell=cell, jac=natural_jac(cell),
                dtype=dtype, B=B, T=T, d=d, n=n, G=G, S=S,
                W_x=r(Wx), b_x=r(bx), W_h=r(Wh), b_h=r(bh), peep=r(peep),
                x=r(x), g=r(g), h0=r(hz), tol=1e-6, max_iters=T)


# The linear state-space workload (the README's lsim example, scaled up): a
# stable system of nx states driven by m inputs with p outputs, sampled every
# dt.  Draw order: A, B, C, D, x0, U.  A = -I + 0.5 G / sqrt(nx) with G
# standard normal keeps the eigenvalues' real parts negative for these sizes.
LSIM_WORKLOAD = dict(name="lsim_T1M", B=16, T=1 << 20, nx=4, m=1, p=1, dt=0.01)


def make_lsim(B: int | None = None, T: int | None = None, nx: int | None = None, m: int | None = None,
              p: int | None = None, dt: float | None = None, seed: int = 6, x0: bool = True) -> dict:
    w = LSIM_WORKLOAD
    B = w["B"] if B is None else B
    T = w["T"] if T is None else T
    nx = w["nx"] if nx is None else nx
    m = w["m"] if m is None else m
    p = w["p"] if p is None else p
    dt = w["dt"] if dt is None else dt
    rng = np.random.default_rng(seed)
    A = -np.eye(nx) + 0.5 * rng.standard_normal((nx, nx)) / np.sqrt(nx)
    Bm = rng.standard_normal((nx, m))
    Cm = rng.standard_normal((p, nx))
    Dm = rng.standard_normal((p, m))
    x0v = rng.standard_normal((B, nx)) if x0 else None
    U = rng.standard_normal((B, T, m))
    f32 = lambda a: None if a is None else round_storage(a, DT_F32)  # noqa: E731
    return dict(name=w["name"] if (B, T, nx, m, p) == (w["B"], w["T"], w["nx"], w["m"], w["p"]) else "lsim_custom",
                B=B, T=T, nx=nx, m=m, p=p, dt=float(np.float32(dt)), A=f32(A), Bm=f32(Bm), Cm=f32(Cm), Dm=f32(Dm),
                x0=f32(x0v), U=f32(U))
