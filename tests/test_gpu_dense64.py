"""GPU parity of the dense n = 64 GRU path (full DEER with 64 x 64 Jacobians
composed on fp32 MFMA) against the fp64 oracle."""
import json
import os

import numpy as np
import pytest

import oracle
from nonlinear_rnn_evaluation_newton_amd import binding as bd
from nonlinear_rnn_evaluation_newton_amd import synthetic as sy

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

ATOL = 1e-4
RTOL_W = 1e-4
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.lib()


def say(*a):
    print(*a, flush=True)


def to64(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("B,T", [(2, 1000), (3, 64), (1, 1), (2, 65), (4, 300)])
def test_dense64_converged(B, T):
    p = sy.make_problem(5, B=B, T=T)
    say("case dense64 B", B, "T", T)
    dp = bd.DeviceProblem(p)
    st, it, dl = dp.solve()
    torch.cuda.synchronize()
    ho, ito, sto, dlo = oracle.deer(p)
    say("  gpu", it, st, dl, "| oracle", ito, sto, dlo)
    assert st == sto and it == ito
    err = np.abs(to64(dp.h) - ho).max()
    say("  max abs err", err)
    assert err <= ATOL


def test_dense64_biases_and_h0():
    p = sy.custom_problem(sy.CELL_GRU, B=3, T=500, d=7, n=64, seed=11, w_scale=0.7, h0=True)
    say("case dense64 custom")
    dp = bd.DeviceProblem(p)
    st, it, dl = dp.solve(tol=1e-5, max_iters=p["T"])
    ho, ito, sto, dlo = oracle.deer(p, tol=1e-5, max_iters=p["T"])
    say("  gpu", it, dl, "| oracle", ito, dlo)
    assert it == ito and st == sto
    assert np.abs(to64(dp.h) - ho).max() <= ATOL


def test_dense64_fixed_iterations_and_status():
    p = sy.make_problem(5, B=2, T=200)
    dp = bd.DeviceProblem(p)
    st, it, dl = dp.solve(tol=0.0, max_iters=2)
    assert (st, it) == (bd.PR_OK, 2)
    ho, *_ = oracle.deer(p, tol=0.0, max_iters=2)
    assert np.abs(to64(dp.h) - ho).max() <= ATOL
    st, it, _ = dp.solve(tol=1e-5, max_iters=1)
    assert (st, it) == (bd.PR_NOT_CONVERGED, 1)


def test_dense64_full_size():
    """The full workload in the benchmark's configuration: iteration count
    against the oracle's recorded history; h against the oracle's sequential
    rollout of three sampled sequences."""
    gold = json.load(open(os.path.join(GOLDEN, "dense64_gru_full_history.json")))
    p = sy.make_problem(5, with_g=False)
    say("case dense64 full size")
    dp = bd.DeviceProblem(p)
    st, it, dl = dp.solve()
    torch.cuda.synchronize()
    say("  gpu iters", it, "deltas", dl, "| oracle", gold["iters"], gold["deltas"])
    assert st == bd.PR_OK and it == gold["iters"]
    seqs = [0, 7, 15]
    q = dict(p, B=len(seqs), x=p["x"][seqs], h0=p["h0"][seqs])
    hs = oracle.rollout(q)
    err = np.abs(to64(dp.h[seqs]) - hs).max()
    say("  max abs err vs rollout (3 sequences)", err)
    assert err <= ATOL


def _adjoint_check(p, dp, a):
    ref = oracle.adjoint(p, to64(dp.h))
    for key in ("lam", "dx", "dh0"):
        err = np.abs(to64(a[key]) - ref[key]).max()
        say("  ", key, err)
        assert err <= ATOL * max(1.0, np.abs(ref[key]).max()), key
    for key in ("dW_x", "db_x", "dW_h", "db_h"):
        r = np.abs(to64(a[key]) - ref[key]).max() / max(np.abs(ref[key]).max(), 1e-30)
        say("  ", key, r)
        assert r <= RTOL_W, key


@pytest.mark.parametrize("B,T", [(2, 300), (1, 64), (3, 129)])
def test_dense64_adjoint(B, T):
    p = sy.make_problem(5, B=B, T=T)
    say("adjoint dense64 B", B, "T", T)
    dp = bd.DeviceProblem(p)
    dp.solve()
    st, a = dp.adjoint()
    torch.cuda.synchronize()
    assert st == bd.PR_OK
    _adjoint_check(p, dp, a)


def test_dense64_adjoint_biases_h0():
    p = sy.custom_problem(sy.CELL_GRU, B=2, T=200, d=5, n=64, seed=3, w_scale=0.7, h0=True)
    dp = bd.DeviceProblem(p)
    dp.solve(tol=1e-6, max_iters=p["T"])
    st, a = dp.adjoint()
    torch.cuda.synchronize()
    _adjoint_check(p, dp, a)
