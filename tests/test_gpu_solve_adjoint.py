"""pararnn_solve_adjoint (the solve and its adjoint in one call) through the
C ABI: the same results, bit for bit, as pararnn_solve followed by
pararnn_adjoint on every kernel family (the same kernels run in the same
order), and the statuses of both calls."""
import numpy as np
import pytest

from nonlinear_rnn_evaluation_newton_amd import binding as bd
from nonlinear_rnn_evaluation_newton_amd import synthetic as sy

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.lib()


def outputs(dp):
    p = dp.p
    f32 = dict(dtype=torch.float32, device="cuda")
    o = dict(lam=torch.full_like(dp.h, float("nan")), dx=torch.full_like(dp.x, float("nan")),
             dh0=torch.full((p["B"], p["S"]), float("nan"), dtype=dp.tdtype, device="cuda"),
             W_x=torch.full(tuple(dp.W_x.shape), float("nan"), **f32),
             b_x=torch.full(tuple(dp.b_x.shape), float("nan"), **f32),
             W_h=torch.full(tuple(dp.W_h.shape), float("nan"), **f32),
             b_h=torch.full(tuple(dp.b_h.shape), float("nan"), **f32))
    if dp.peep is not None:
        o["peep"] = torch.full(tuple(dp.peep.shape), float("nan"), **f32)
    return o


def grads_of(o):
    return {k: o[k] for k in ("W_x", "b_x", "W_h", "b_h", "peep") if k in o}


CASES = [
    ("scalar GRU (scalar pipeline)", lambda: sy.make_problem(2, B=3, T=4096)),
    ("tanh RNN n=4", lambda: sy.make_problem(1, B=2, T=300)),
    ("ParaGRU bf16", lambda: sy.custom_problem(sy.CELL_GRU_DIAG, B=2, T=300, d=24, n=96, seed=5, w_scale=0.8,
                                               h0=True, dtype=sy.DT_BF16)),
    ("ParaLSTM fp32", lambda: sy.custom_problem(sy.CELL_LSTM_CIFG_DIAG, B=2, T=200, d=12, n=40, seed=6,
                                                w_scale=0.8, h0=True)),
    ("dense GRU n=64", lambda: sy.make_problem(5, B=2, T=300)),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_matches_separate_calls(name, make):
    p = make()
    print("case", name, "B", p["B"], "T", p["T"], "n", p["n"], flush=True)
    dp = bd.DeviceProblem(p)
    max_iters = p["max_iters"]
    st1, it1, dl1 = dp.solve()
    o1 = outputs(dp)
    ra = bd.adjoint(dp.prob, dp.w, dp.x, dp.h0, dp.h, dp.g, dp.ws, o1["lam"], o1["dx"], o1["dh0"], grads_of(o1))
    torch.cuda.synchronize()
    h1 = dp.h.clone()
    dp.h.fill_(float("nan"))
    o2 = outputs(dp)
    st2, it2, dl2 = bd.solve_adjoint(dp.prob, dp.w, dp.x, dp.h0, p["tol"], max_iters, dp.h, dp.g, dp.ws, o2["lam"],
                                     o2["dx"], o2["dh0"], grads_of(o2))
    torch.cuda.synchronize()
    print("  separate", st1, it1, ra, "| combined", st2, it2, flush=True)
    assert st1 >= 0 and ra == bd.PR_OK and st2 == st1 and it2 == it1
    assert np.array_equal(dl1, dl2)
    assert torch.equal(dp.h, h1)
    for k in o1:
        assert torch.equal(o1[k], o2[k]), k


def run_separate(dp, tol, max_iters):
    st, it, dl = bd.solve(dp.prob, dp.w, dp.x, dp.h0, tol, max_iters, dp.h, dp.ws)
    o = outputs(dp)
    ra = bd.adjoint(dp.prob, dp.w, dp.x, dp.h0, dp.h, dp.g, dp.ws, o["lam"], o["dx"], o["dh0"], grads_of(o))
    torch.cuda.synchronize()
    assert ra == bd.PR_OK
    return st, it, dl, dp.h.clone(), o


def run_combined(dp, tol, max_iters):
    dp.h.fill_(float("nan"))
    o = outputs(dp)
    st, it, dl = bd.solve_adjoint(dp.prob, dp.w, dp.x, dp.h0, tol, max_iters, dp.h, dp.g, dp.ws, o["lam"], o["dx"],
                                  o["dh0"], grads_of(o))
    torch.cuda.synchronize()
    return st, it, dl, dp.h.clone(), o


def same(r1, r2):
    assert r1[0] == r2[0] and r1[1] == r2[1] and np.array_equal(r1[2], r2[2])
    assert torch.equal(r1[3], r2[3])
    for k in r1[4]:
        assert torch.equal(r1[4][k], r2[4][k]), k


def close(r1, r2, bf16):
    """The solve bit for bit; the adjoint within rounding (the per-channel
    cells' combined call composes the adjoint's tile aggregates in the last
    sweep's pass, in the other order along time)."""
    assert r1[0] == r2[0] and r1[1] == r2[1] and np.array_equal(r1[2], r2[2])
    assert torch.equal(r1[3], r2[3])
    for k in r1[4]:
        a, b = r1[4][k].float(), r2[4][k].float()
        scale = max(float(a.abs().max()), 1e-30)
        err = float((a - b).abs().max()) / scale
        print("  ", k, "rel diff", err, flush=True)
        assert err <= (1e-2 if bf16 and k in ("lam", "dx", "dh0") else 1e-5), k


@pytest.mark.parametrize("cell,n,dtype", [(sy.CELL_LSTM_CIFG_DIAG, 40, sy.DT_BF16), (sy.CELL_LSTM_CIFG_DIAG, 40, sy.DT_F32),
                                          (sy.CELL_GRU_DIAG, 70, sy.DT_BF16), (sy.CELL_GRU, 64, sy.DT_F32),
                                          (sy.CELL_TANH_RNN, 4, sy.DT_F32)])
def test_fixed_sweep_count_speculates(cell, n, dtype):
    """tol = 0 (a fixed number of sweeps): the adjoint is enqueued behind the
    only batch of sweeps, before the poll; results as the separate calls (the
    per-channel cells' adjoint within rounding, see close)."""
    p = sy.custom_problem(cell, B=2, T=257, d=5, n=n, seed=n, w_scale=0.5, h0=True, dtype=dtype)
    print("case fixed sweeps cell", cell, "n", n, "dtype", dtype, flush=True)
    dp = bd.DeviceProblem(p)
    ref = run_separate(dp, 0.0, 3)
    chan = cell in (sy.CELL_GRU_DIAG, sy.CELL_LSTM_CIFG_DIAG)
    for _ in range(2):
        if chan:
            close(ref, run_combined(dp, 0.0, 3), dtype == sy.DT_BF16)
        else:
            same(ref, run_combined(dp, 0.0, 3))


def test_scalar_speculation_hit_and_miss(monkeypatch):
    """n = d = 1 with tol > 0: a call on inputs converging within the first
    batch (3 sweeps here) makes the next call speculate; inputs needing a 4th
    sweep then miss, the solve state is restored from the poll's snapshot and
    the adjoint runs again at the end.  Every call matches the separate ones."""
    monkeypatch.setenv("PARARNN_POLL", "3,2")
    tol = 1e-3
    pb = sy.make_problem(2, B=3, T=4096)
    pa = dict(pb, x=pb["x"] * 0.03)  # converges in 3 sweeps at this tol; pb needs 4
    da, db = bd.DeviceProblem(pa), bd.DeviceProblem(pb)
    ref_a = run_separate(da, tol, pb["max_iters"])
    ref_b = run_separate(db, tol, pb["max_iters"])
    print("  sweeps: inputs a", ref_a[1], "inputs b", ref_b[1], flush=True)
    assert ref_a[1] == 3 and ref_b[1] == 4
    same(ref_a, run_combined(da, tol, pb["max_iters"]))  # no record yet: sequential
    same(ref_a, run_combined(da, tol, pb["max_iters"]))  # speculates and hits
    same(ref_b, run_combined(db, tol, pb["max_iters"]))  # speculates and misses
    same(ref_b, run_combined(db, tol, pb["max_iters"]))  # the record now says no: sequential


@pytest.mark.parametrize("make", [lambda: sy.make_problem(2, B=2, T=1024),
                                  lambda: sy.custom_problem(sy.CELL_GRU_DIAG, B=2, T=300, d=6, n=20, seed=2,
                                                            w_scale=0.8, h0=True)],
                         ids=["scalar GRU", "ParaGRU"])
def test_not_converged_matches_separate_calls(make):
    """max_iters below the sweeps needed: PR_NOT_CONVERGED from both, the
    adjoint taken at the last iterate either way."""
    p = make()
    dp = bd.DeviceProblem(p)
    ref = run_separate(dp, p["tol"], 2)
    assert ref[0] == bd.PR_NOT_CONVERGED and ref[1] == 2
    for _ in range(2):
        same(ref, run_combined(dp, p["tol"], 2))


def test_missing_adjoint_argument():
    """g is required: the call reports PR_EINVAL (the solve has run)."""
    p = sy.make_problem(2, B=2, T=1024)
    dp = bd.DeviceProblem(p)
    o = outputs(dp)
    st, it, _ = bd.solve_adjoint(dp.prob, dp.w, dp.x, dp.h0, p["tol"], p["max_iters"], dp.h, None, dp.ws, o["lam"],
                                 o["dx"], o["dh0"], grads_of(o), check=False)
    torch.cuda.synchronize()
    assert st == bd.PR_EINVAL and "g" in bd.last_error()
