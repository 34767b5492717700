"""GPU parity of the channel-parallel path (diagonal ParaGRU, 2x2-block
CIFG/peephole ParaLSTM; bf16 or fp32 storage) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from nonlinear_rnn_evaluation_newton_amd import binding as bd
from nonlinear_rnn_evaluation_newton_amd import synthetic as sy

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

ATOL = 1e-4     # fp32 storage: max-abs on h, lambda, dx, dh0 (scaled by max(1, |ref|))
RTOL_BF = 2e-2  # bf16 storage, fp32 arithmetic: ||gpu - ref||_inf / ||ref||_inf per tensor
RTOL_W = 1e-4   # fp32 weight gradients: norm-wise relative


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.lib()


def say(*a):
    print(*a, flush=True)


def to64(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))


def check_solve(p, tol, max_iters, bf16):
    say("case", p["name"], "B", p["B"], "T", p["T"], "d", p["d"], "n", p["n"], "tol", tol, "max_iters", max_iters,
        "bf16", bf16)
    dp = bd.DeviceProblem(p)
    st, it, dl = dp.solve(tol=tol, max_iters=max_iters)
    torch.cuda.synchronize()
    h = to64(dp.h)
    ho, ito, sto, dlo = oracle.deer(p, tol=tol, max_iters=max_iters)
    say("  gpu iters", it, "status", st, "deltas", dl, "| oracle", ito, sto, dlo)
    assert st == sto and it == ito
    if bf16:
        r = rel(h, ho)
        say("  rel err", r)
        assert r <= RTOL_BF
    else:
        err = np.abs(h - ho).max()
        say("  max abs err", err)
        assert err <= ATOL
    return dp, h


@pytest.mark.parametrize("cfg", [3, 4])
def test_reduced_bf16_configs(cfg):
    p = sy.make_problem(cfg, B=2, T=300, d=64, n=64)
    check_solve(p, p["tol"], p["max_iters"], True)


@pytest.mark.parametrize("cell", [sy.CELL_GRU_DIAG, sy.CELL_LSTM_CIFG_DIAG])
@pytest.mark.parametrize("n,d,T", [(64, 16, 200), (5, 3, 77), (130, 40, 1000), (256, 64, 4097), (7, 9, 1)])
def test_fp32_converged(cell, n, d, T):
    p = sy.custom_problem(cell, B=2, T=T, d=d, n=n, seed=n + T, w_scale=0.8, h0=True)
    check_solve(p, 1e-6, T, False)


@pytest.mark.parametrize("cell", [sy.CELL_GRU_DIAG, sy.CELL_LSTM_CIFG_DIAG])
def test_bf16_converged_small(cell):
    p = sy.custom_problem(cell, B=3, T=500, d=24, n=96, seed=4, w_scale=0.8, h0=True, dtype=sy.DT_BF16)
    check_solve(p, 0.0, 6, True)


def _slice_channels(p, ch):
    """The sub-problem of channels `ch` (channels are independent given x)."""
    n = p["n"]
    rows = np.concatenate([g * n + ch for g in range(3)])
    q = dict(p)
    q["n"] = len(ch)
    q["S"] = q["n"] * (2 if p["cell"] == sy.CELL_LSTM_CIFG_DIAG else 1)
    q["W_x"] = p["W_x"][rows]
    q["b_x"] = p["b_x"][rows]
    q["W_h"] = p["W_h"][rows]
    q["b_h"] = p["b_h"][rows]
    if p["peep"] is not None:
        q["peep"] = np.concatenate([p["peep"][ch], p["peep"][n + ch]])
    if p["cell"] == sy.CELL_LSTM_CIFG_DIAG:
        sidx = np.stack([2 * ch, 2 * ch + 1], 1).reshape(-1)
    else:
        sidx = ch
    q["h0"] = p["h0"][:, sidx]
    if p.get("g") is not None:
        q["g"] = p["g"][:, :, sidx]
    return q, sidx


@pytest.mark.parametrize("cfg", [3, 4])
def test_full_size_sampled_channels(cfg):
    """The full workload in the benchmark's launch configuration; the oracle
    checks 12 sampled channels (first, last, and random ones)."""
    p = sy.make_problem(cfg, with_g=False)
    say("full-size case", p["name"])
    dp = bd.DeviceProblem(p)
    st, it, dl = dp.solve()
    torch.cuda.synchronize()
    assert st == bd.PR_OK and it == p["max_iters"]
    rng = np.random.default_rng(100 + cfg)
    ch = np.unique(np.concatenate([[0, p["n"] - 1], rng.choice(p["n"], 10, replace=False)]))
    q, sidx = _slice_channels(p, ch)
    hq, itq, stq, dlq = oracle.deer(q, tol=p["tol"], max_iters=p["max_iters"])
    h = to64(dp.h[:, :, torch.as_tensor(sidx, device="cuda")])
    r = rel(h, hq)
    say("  sampled channels", ch, "rel err", r, "gpu deltas", dl)
    assert r <= RTOL_BF


@pytest.mark.parametrize("jac,SW", [(bd.PR_JAC_DIAG, 1), (bd.PR_JAC_BLOCK2, 2)])
@pytest.mark.parametrize("n", [1, 3, 64, 200])
@pytest.mark.parametrize("T", [1, 5, 63, 64, 65, 1000])
@pytest.mark.parametrize("reverse", [False, True])
def test_structured_scan_bit_exact(jac, SW, n, T, reverse):
    say("scan case", jac, n, T, reverse)
    rng = np.random.default_rng(7 * n + T + SW)
    B = 2
    if SW == 1:
        A = rng.integers(-1, 2, size=(B, T, n)).astype(float)
        b = rng.integers(-4, 5, size=(B, T, n)).astype(float)
        kind = oracle.DIAG
    else:
        A = np.zeros((B, T, n, 2, 2))
        col = rng.integers(0, 2, size=(B, T, n, 2))
        val = rng.integers(-1, 2, size=(B, T, n, 2)).astype(float)
        np.put_along_axis(A, col[..., None], val[..., None], axis=-1)
        b = rng.integers(-4, 5, size=(B, T, n, 2)).astype(float)
        kind = oracle.BLOCK2
    y_ref = oracle.affine_solve(kind, A, b, reverse=reverse)
    At = torch.tensor(A, dtype=torch.float32, device="cuda")
    bt = torch.tensor(b, dtype=torch.float32, device="cuda")
    yt = torch.empty_like(bt)
    ws = torch.empty(bd.scan_workspace_bytes(jac, B, T, n), dtype=torch.uint8, device="cuda")
    bd.affine_scan(jac, At, bt, yt, ws, reverse=reverse)
    torch.cuda.synchronize()
    assert np.array_equal(yt.cpu().numpy().astype(np.float64), y_ref)


def adjoint_compare(p, h, a, bf16):
    ref = oracle.adjoint(p, h)
    for key in ("lam", "dx", "dh0"):
        g = to64(a[key])
        if bf16:
            r = rel(g, ref[key])
            say("  ", key, "rel", r)
            assert r <= RTOL_BF, key
        else:
            err = np.abs(g - ref[key]).max()
            say("  ", key, "abs", err)
            assert err <= ATOL * max(1.0, np.abs(ref[key]).max()), key
    keys = ["dW_x", "db_x", "dW_h", "db_h"] + (["dpeep"] if p["cell"] == sy.CELL_LSTM_CIFG_DIAG else [])
    for key in keys:
        r = rel(to64(a[key]), ref[key])
        say("  ", key, "rel", r)
        assert r <= (RTOL_BF if bf16 else RTOL_W), key


@pytest.mark.parametrize("cell", [sy.CELL_GRU_DIAG, sy.CELL_LSTM_CIFG_DIAG])
@pytest.mark.parametrize("n,d,T", [(64, 16, 200), (5, 3, 77), (130, 40, 1001), (7, 9, 1)])
def test_adjoint_fp32(cell, n, d, T):
    p = sy.custom_problem(cell, B=2, T=T, d=d, n=n, seed=3 * n + T, w_scale=0.8, h0=True)
    say("adjoint case", p["name"], n, d, T)
    dp = bd.DeviceProblem(p)
    dp.solve(tol=1e-6, max_iters=T)
    st, a = dp.adjoint()
    torch.cuda.synchronize()
    assert st == bd.PR_OK
    adjoint_compare(p, to64(dp.h), a, False)


@pytest.mark.parametrize("cfg", [3, 4])
def test_adjoint_bf16_reduced(cfg):
    p = sy.make_problem(cfg, B=2, T=300, d=64, n=64)
    say("adjoint case", p["name"])
    dp = bd.DeviceProblem(p)
    dp.solve()
    st, a = dp.adjoint()
    torch.cuda.synchronize()
    assert st == bd.PR_OK
    adjoint_compare(p, to64(dp.h), a, True)


@pytest.mark.parametrize("cell", [sy.CELL_GRU_DIAG, sy.CELL_LSTM_CIFG_DIAG])
@pytest.mark.parametrize("B,T,d,n", [(3, 704, 264, 304), (1, 512, 512, 256), (3, 701, 264, 304)])
def test_bf16_large_products(cell, B, T, d, n):
    """Shapes that take the 256 x 256-tile bf16 products in all three places
    (input projection with bias, dx = dU W_x, dW_x = dU^T x read K-outer),
    with ragged row and column tails (first case), exact tile multiples
    (second) and a K tail of the K-outer product (third: 2103 rows)."""
    p = sy.custom_problem(cell, B=B, T=T, d=d, n=n, seed=T + n, w_scale=0.8, h0=True, dtype=sy.DT_BF16)
    say("large-product case", p["name"], "B", B, "T", T, "d", d, "n", n)
    dp, h = check_solve(p, 0.0, 3, True)
    st, a = dp.adjoint()
    torch.cuda.synchronize()
    assert st == bd.PR_OK
    adjoint_compare(p, h, a, True)


@pytest.mark.parametrize("cell", [sy.CELL_GRU_DIAG, sy.CELL_LSTM_CIFG_DIAG])
@pytest.mark.parametrize("T", [63, 64, 65, 128, 129])
def test_tile_boundaries(cell, T):
    """Sequence lengths around the 64-step tiles of the sweep and adjoint
    passes (one partial tile, exactly one or two full tiles, a one-step
    tail), with h0, biases and a channel count that leaves idle lanes."""
    p = sy.custom_problem(cell, B=2, T=T, d=12, n=66, seed=7 * T + cell, w_scale=0.8, h0=True)
    dp, h = check_solve(p, 1e-6, T, False)
    st, a = dp.adjoint()
    torch.cuda.synchronize()
    assert st == bd.PR_OK
    adjoint_compare(p, h, a, False)


def test_bf16_products_on_the_small_tile_gemm(monkeypatch):
    """A large-product shape with the 256 x 256-tile GEMM switched off
    (PARARNN_SMALL_GEMM): the 128 x 128-tile kernel on the same products."""
    monkeypatch.setenv("PARARNN_SMALL_GEMM", "1")
    p = sy.custom_problem(sy.CELL_LSTM_CIFG_DIAG, B=3, T=704, d=264, n=304, seed=11, w_scale=0.8, h0=True,
                          dtype=sy.DT_BF16)
    dp, h = check_solve(p, 0.0, 3, True)
    st, a = dp.adjoint()
    torch.cuda.synchronize()
    assert st == bd.PR_OK
    adjoint_compare(p, h, a, True)
