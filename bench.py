"""Benchmark of the DEER / quasi-DEER hot path on one MI355X.

A step is one pass of the whole path over one batch: the Newton solve to
convergence (input projection, every sweep, the on-device stop rule and its
polls) followed by the adjoint (reverse scan, chain rule, weight-gradient
reductions).  Inputs are seeded synthetic data already resident in HBM.

Default workload: the scalar-state GRU at batch 16 and length 2^20 that the
DEER paper times on a V100 ("Parallelizing non-linear sequential models over
the sequence length", Key results: 15 ms DEER vs 8.7 s sequential).

Prints one JSON line (rank 0, N = 1).
"""
from __future__ import annotations

import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import argparse  # noqa: E402
import json  # noqa: E402
import time  # noqa: E402

from nonlinear_rnn_evaluation_newton_amd import synthetic as sy  # noqa: E402  (input generator only)


HBM_PEAK_GBS = 8000.0
ELK_KERNELS = ("quasi-ELK sweep: per-channel cells k_elkc_filter + k_elkc_filter_carry + k_elkc_smooth + "
               "k_elkc_smooth_carry + k_elkc_apply (the cell re-evaluated in each pass); dense GRU "
               "k_d64_gates<GM_QUASI>, small dense cells k_time_elk_jr, then k_elk_filter/gains/apply and "
               "their chunk carries")
ELK_FULL_KERNELS = ("ELK sweep (the cell's own Jacobian, full covariances): producer of J | r (k_elkf_jr_lstm or "
                    "k_elkf_jr_dense), then k_elkf_elem (chunk filtering elements), k_elkf_fcarry, k_elkf_gains "
                    "(in-chunk filter and smoother gains), k_elkf_scarry, k_elkf_apply")
ELK64_KERNELS = ("ELK sweep with the full 64x64 Jacobian: k_d64_gates (the Jacobian's factors and the residual), "
                 "k_elk64_rows (the damped step's normal equations, one 64x64 block row per step), per level of "
                 "the block cyclic reduction k_elk64_elim and k_elk64_keep, k_elk64_root, per level k_elk64_back, "
                 "k_elk64_apply")
FP32_MFMA_PEAK_TFS = 157.3


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    record (profiles/hbm_traffic.json: FETCH_SIZE and WRITE_SIZE passes scaled
    by a plain-copy calibration), or None when the workload has no record or
    a kernel source listed there has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(path)).get(workload)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    for src, sha in rec.get("sources", {}).items():
        try:
            if hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest() != sha:
                return None
        except OSError:
            return None
    return rec.get("traffic_bytes_per_launch")


def scalar_path(p: dict) -> bool:
    """The library's scalar-state kernels take n = d = 1 with T % 4 == 0."""
    return p["n"] == 1 and p["d"] == 1 and p["T"] % 4 == 0 and p["cell"] in (sy.CELL_GRU, sy.CELL_TANH_RNN,
                                                                              sy.CELL_LINEAR)


def units_of(p: dict) -> int:
    """Work units of one sweep: (b, t) for a dense state, (b, t, channel) else."""
    if p["cell"] in (sy.CELL_GRU_DIAG, sy.CELL_LSTM_CIFG_DIAG):
        return p["B"] * p["T"] * p["n"]
    return p["B"] * p["T"]


def sweep_bytes_per_unit(p: dict, k: int, adjoint_aggregates: bool = False) -> float:
    """Algorithmic HBM bytes per unit of one fused Newton sweep.

    Dense small state (time-parallel kernel): reads x (fused projection) and,
    from sweep 2 on, the current iterate h; writes the new h.  Per-channel
    cells: read U (3 gates), read h (sweep >= 2), write h; the last sweep of
    a fixed sweep count followed by the adjoint also reads g (it composes the
    adjoint's tile aggregates).  Sweep 1 starts from h = 0 and does not read it.
    """
    es = 2 if p["dtype"] == sy.DT_BF16 else 4
    sw = 2 if p["cell"] == sy.CELL_LSTM_CIFG_DIAG else 1
    if p["cell"] in (sy.CELL_GRU_DIAG, sy.CELL_LSTM_CIFG_DIAG):
        return 3 * es + sw * es + (sw * es if k >= 2 else 0) + (sw * es if adjoint_aggregates else 0)
    return p["d"] * 4 + p["n"] * 4 + (p["n"] * 4 if k >= 2 else 0)


def adjoint_bytes_per_unit(p: dict) -> float:
    """Adjoint scan kernel: dense small state reads x, h, g and writes lambda,
    dx; per-channel cells read U, h, g and write lambda and dU (3 gates)."""
    es = 2 if p["dtype"] == sy.DT_BF16 else 4
    sw = 2 if p["cell"] == sy.CELL_LSTM_CIFG_DIAG else 1
    if p["cell"] in (sy.CELL_GRU_DIAG, sy.CELL_LSTM_CIFG_DIAG):
        return 3 * es + 2 * sw * es + sw * es + 3 * es
    return 2 * p["d"] * 4 + 3 * p["n"] * 4


def host_cores() -> int:
    """Cores this process may run on (the affinity mask), else the CPU count."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def median_of_3(fn) -> float:
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return sorted(ts)[1]


def cpu_baseline(p: dict) -> dict:
    """The oracle's fp64 sequential rollout, timed on this host (median of 3).

    Per-channel cells are independent across channels given x, so for them a
    sample of channels is rolled out (the full input width, every sequence and
    step) and the time is scaled by n / sample; dense cells run in full.
    OpenMP runs over independent sequences only, so the threads that work are
    min(OpenMP threads, B).
    """
    import numpy as np
    import oracle
    omp = oracle.num_threads()
    threads = min(omp, p["B"])
    units = p["B"] * p["T"]
    if p["cell"] in (sy.CELL_GRU_DIAG, sy.CELL_LSTM_CIFG_DIAG):
        n = p["n"]

        def sub(ns):
            ch = np.arange(ns)
            rows = np.concatenate([g * n + ch for g in range(3)])
            q = dict(p, n=ns, S=ns * (2 if p["cell"] == sy.CELL_LSTM_CIFG_DIAG else 1), W_x=p["W_x"][rows],
                     b_x=p["b_x"][rows], W_h=p["W_h"][rows], b_h=p["b_h"][rows],
                     peep=None if p["peep"] is None else np.concatenate([p["peep"][ch], p["peep"][n + ch]]))
            q["h0"] = np.zeros((p["B"], q["S"]))
            return q

        t0 = time.perf_counter()
        oracle.rollout(sub(1))
        t1 = time.perf_counter() - t0
        ns = int(min(n, max(1, 4.0 / max(t1, 1e-3))))  # about 4 s of fp64 work per run
        q = sub(ns)
        ts = median_of_3(lambda: oracle.rollout(q))
        dt = ts * n / ns
        sample = (f"fp64 sequential rollout of {ns} of {n} channels (all {p['B']} sequences x {p['T']} steps, "
                  f"full input width), OpenMP over sequences; median of 3 runs {ts:.3f} s, scaled by {n}/{ns} "
                  f"to {dt:.3f} s for all channels")
    else:
        dt = median_of_3(lambda: oracle.rollout(p))
        sample = (f"full workload: fp64 sequential rollout of all {p['B']} sequences x {p['T']} steps, "
                  f"OpenMP over sequences; median of 3 runs {dt:.3f} s")
    return {"value": units / dt, "unit": "timesteps*batch/s", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": dt, "host_cores": host_cores(), "omp_threads": omp}


def bench_lsim(args) -> int:
    """One step = one pararnn_lsim call over the whole batch (discretisation,
    chunk aggregates, chunk carries, outputs)."""
    import numpy as np
    import torch

    from nonlinear_rnn_evaluation_newton_amd import binding as bd

    q = sy.make_lsim()
    B, T, nx, m, p = q["B"], q["T"], q["nx"], q["m"], q["p"]

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()

    A, Bm, Cm, Dm, U, x0 = (dev(q[k]) for k in ("A", "Bm", "Cm", "Dm", "U", "x0"))
    x = torch.empty((B, T, nx), device="cuda")
    y = torch.empty((B, T, p), device="cuda")
    ws = torch.empty(bd.lsim_workspace_bytes(B, T, nx, m, p), dtype=torch.uint8, device="cuda")

    def step():
        bd.lsim(A, Bm, Cm, Dm, q["dt"], U, x0, x, y, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if not args.no_trace:
        bd.trace(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    roofline = None
    if not args.no_trace:
        lm, ln = bd.trace_kernel(bd.TRACE_LSIM)
        bd.trace(False)
        # algorithmic bytes per step: read u (m floats), write x (nx) and y (p)
        per_call = 4.0 * (m + nx + p) * B * T
        achieved = per_call / (lm / ln * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                    "kernel": "k_lsim_disc + k_lsim_pass<aggregate> + k_lsim_carry + k_lsim_pass<apply> per call",
                    "avg_launch_us": round(lm / ln * 1e3, 2), "bytes_per_launch": per_call}
    line = {
        "metric": "timesteps*batch/sec of a linear state-space simulation (lsim, no Newton loop)",
        "value": B * T / (ms_step * 1e-3), "unit": "timesteps*batch/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": q["name"], "B": B, "T": T, "nx": nx, "m": m, "p": p, "dt": q["dt"],
                   "step": "one lsim call (zero-order hold)"},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        import oracle
        dt = median_of_3(lambda: oracle.lsim(q["A"], q["Bm"], q["Cm"], q["Dm"], q["U"], np.arange(T) * q["dt"],
                                             x0=q["x0"]))
        line["cpu_baseline"] = {"value": B * T / dt, "unit": "timesteps*batch/s",
                                "cores": min(oracle.num_threads(), B), "kind": "oracle",
                                "sample": f"full workload: fp64 sequential lsim of all {B} sequences x {T} steps, "
                                          f"OpenMP over sequences; median of 3 runs {dt:.3f} s",
                                "host_cores": host_cores(), "omp_threads": oracle.num_threads()}
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, help="workload 1..5 (default 2: GRU n=1, B=16, T=2^20)")
    ap.add_argument("--jac", choices=("own", "diag", "zero"), default="own",
                    help="Jacobian of the sweeps' linear solve: the cell's own (Newton), its diagonal "
                         "(quasi-DEER) or zero (Jacobi)")
    ap.add_argument("--elk", type=float, default=None, metavar="LAMBDA",
                    help="solve with ELK at damping LAMBDA: the cell's own Jacobian (full covariances), or "
                         "its diagonal (quasi-ELK) with --jac diag")
    ap.add_argument("--lsim", action="store_true",
                    help="time the linear state-space simulation workload (B=16, T=2^20, 4 states) instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true", help="do not bracket kernels with events")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 launches), to scale HBM counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU per process; --gpus N > 1 is not supported"}))
        return 2

    import numpy as np
    import torch

    from nonlinear_rnn_evaluation_newton_amd import binding as bd

    torch.cuda.set_device(0)
    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes, "launches": 3}))
        return 0
    if args.lsim:
        return bench_lsim(args)
    p = sy.make_problem(args.config)
    if args.jac != "own":
        p = dict(p, jac=sy.JAC_DIAG if args.jac == "diag" else sy.JAC_ZERO,
                 name=p["name"] + ("_quasi" if args.jac == "diag" else "_jacobi"))
    approx = args.jac != "own" and not (args.jac == "diag" and (p["cell"] == sy.CELL_GRU_DIAG or p["n"] == 1))
    elk = args.elk is not None
    if elk:
        p = dict(p, name=p["name"] + f"_elk{args.elk:g}")
        approx = True
    dp = bd.DeviceProblem(p, elk=elk)
    B, T = p["B"], p["T"]
    units = B * T

    f32 = dict(dtype=torch.float32, device="cuda")
    lam = torch.empty_like(dp.h)
    dx = torch.empty_like(dp.x)
    dh0 = torch.empty((B, p["S"]), dtype=dp.tdtype, device="cuda")
    grads = dict(W_x=torch.empty(tuple(dp.W_x.shape), **f32), b_x=torch.empty(tuple(dp.b_x.shape), **f32),
                 W_h=torch.empty(tuple(dp.W_h.shape), **f32), b_h=torch.empty(tuple(dp.b_h.shape), **f32))
    if dp.peep is not None:
        grads["peep"] = torch.empty(tuple(dp.peep.shape), **f32)

    iters_seen = []

    def solve():
        return dp.solve_elk(args.elk) if elk else dp.solve()

    def step():
        if elk:
            st, it, dl = solve()
            if st < 0 or st == bd.PR_NONFINITE:
                raise RuntimeError(f"solve failed: {st}")
            bd.adjoint(dp.prob, dp.w, dp.x, dp.h0, dp.h, dp.g, dp.ws, lam, dx, dh0, grads)
        else:  # the solve and its adjoint in one call
            st, it, dl = bd.solve_adjoint(dp.prob, dp.w, dp.x, dp.h0, p["tol"], p["max_iters"], dp.h, dp.g, dp.ws,
                                          lam, dx, dh0, grads)
            if st < 0 or st == bd.PR_NONFINITE:
                raise RuntimeError(f"solve failed: {st}")
        iters_seen.append(it)
        return it, dl

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps
    if not args.no_trace:
        bd.trace(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        it, dl = step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    tr = bd.trace_read() if not args.no_trace else None
    ms_step = (t1 - t0) * 1e3 / args.steps

    # solve alone (context; same inputs)
    torch.cuda.synchronize()
    s0 = time.perf_counter()
    for _ in range(args.steps):
        solve()
    torch.cuda.synchronize()
    ms_solve = (time.perf_counter() - s0) * 1e3 / args.steps

    # The scalar-state path enqueues the adjoint before the convergence poll
    # when the previous call on the same problem shape converged within its
    # first batch of sweeps, which every timed step above does.  Context:
    # the step when that never happens, from calls alternating with a problem
    # four steps shorter (whose own step costs the same), so every call misses.
    no_spec_ms = None
    if scalar_path(p) and not elk and not approx:
        q = sy.make_problem(args.config, T=T - 4)
        dq = bd.DeviceProblem(q)

        def step_q():
            st, _, _ = bd.solve_adjoint(dq.prob, dq.w, dq.x, dq.h0, q["tol"], q["max_iters"], dq.h, dq.g, dq.ws,
                                        lam, dx, dh0, grads)
            if st < 0 or st == bd.PR_NONFINITE:
                raise RuntimeError(f"solve failed: {st}")

        step_q()
        step()
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        for _ in range(args.steps):
            step_q()
            step()
        torch.cuda.synchronize()
        no_spec_ms = (time.perf_counter() - c0) * 1e3 / (2 * args.steps)
        del dq

    iters = iters_seen[-1]
    roofline = None
    extra = {}
    wu = units_of(p)
    chan = p["cell"] in (sy.CELL_GRU_DIAG, sy.CELL_LSTM_CIFG_DIAG)
    dense64 = p["cell"] == sy.CELL_GRU and p["n"] == 64
    if tr is not None and tr["sweep_launches"] > 0 and dense64 and elk and args.jac == "own":
        # ELK with the full 64 x 64 Jacobian: per step the sweep runs six
        # 64 x 64 products on fp32 MFMA (J^T J for the normal equations'
        # diagonal block; at the step's elimination W A, W A^T and A^T P; at
        # its row's updates A P and A Q) and one 64 x 64 inverse (VALU)
        flops = 6 * 2.0 * 64 ** 3
        avg_ms = tr["sweep_ms"] / tr["sweep_launches"]
        tfs = flops * B * T / (avg_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(tfs, 2), "peak": FP32_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                    "frac": round(tfs / FP32_MFMA_PEAK_TFS, 4), "traffic": None, "kernel": ELK64_KERNELS,
                    "avg_launch_us": round(avg_ms * 1e3, 2), "flops_per_launch": flops * B * T}
    elif tr is not None and tr["sweep_launches"] > 0 and dense64 and approx:
        # diagonal (or zero) Jacobian, n = 64: the sweep is the gates GEMM,
        # a per-channel scan and the update.  Algorithmic bytes per step: read
        # U (192 floats) and, from sweep 2 on, h (64); write h (64)
        per_solve_bytes = sum(4.0 * (192 + (64 if k >= 2 else 0) + 64) for k in range(1, iters + 1)) * units
        avg_ms = tr["sweep_ms"] / tr["sweep_launches"]
        achieved = per_solve_bytes / iters / (avg_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(p["name"]),
                    "kernel": ELK_KERNELS if elk else
                              "k_d64_gates<GM_QUASI> + k_d64q_carry + k_d64q_apply per sweep (gates GEMM with the "
                              "diagonal Jacobian and chunk aggregates; chunk carries; update)",
                    "avg_launch_us": round(avg_ms * 1e3, 2), "bytes_per_launch": per_solve_bytes / iters}
        dm, dn = bd.trace_kernel(bd.TRACE_DENSE_PRODUCTS)
        if dn > 0:
            extra["carry_kernel_us"] = round(dm / dn * 1e3, 2)
        if tr["adjoint_launches"] > 0:
            extra["adjoint_scan_us"] = round(tr["adjoint_ms"] / tr["adjoint_launches"] * 1e3, 2)
        gm, gn = bd.trace_kernel(bd.TRACE_ADJOINT_PRODUCTS)
        if gn > 0:
            extra["adjoint_products_us"] = round(gm / gn * 1e3, 2)
    elif tr is not None and tr["sweep_launches"] > 0 and dense64:
        # full DEER, n = 64: the chunk-product kernel composes one 64 x 64
        # Jacobian per step on fp32 MFMA (2 n^3 flops) and carries the offset
        # (2 n^2): 532,480 algorithmic flops per step
        dm, dn = bd.trace_kernel(bd.TRACE_DENSE_PRODUCTS)
        flops = 2.0 * 64 ** 3 + 2.0 * 64 ** 2
        tfs = flops * B * T / (dm / dn * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(tfs, 2), "peak": FP32_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                    "frac": round(tfs / FP32_MFMA_PEAK_TFS, 4), "traffic": measured_traffic(p["name"]),
                    "kernel": "k_d64_scanA (64x64 Jacobian chunk products, fp32 MFMA)",
                    "avg_launch_us": round(dm / dn * 1e3, 2), "flops_per_launch": flops * B * T}
        extra["sweep_avg_us"] = round(tr["sweep_ms"] / tr["sweep_launches"] * 1e3, 2)
        if tr["adjoint_launches"] > 0:
            extra["adjoint_scan_us"] = round(tr["adjoint_ms"] / tr["adjoint_launches"] * 1e3, 2)
        gm, gn = bd.trace_kernel(bd.TRACE_ADJOINT_PRODUCTS)
        if gn > 0:
            extra["adjoint_products_us"] = round(gm / gn * 1e3, 2)
    elif tr is not None and tr["sweep_launches"] > 0:
        # per-channel cells with a fixed sweep count: the step's last sweep
        # composes the adjoint's aggregates (pararnn_solve_adjoint)
        fused = chan and not elk and p["tol"] <= 0
        per_solve_bytes = sum(sweep_bytes_per_unit(p, k, fused and k == iters) for k in range(1, iters + 1)) * wu
        nsolves = tr["sweep_launches"] / iters
        avg_ms = tr["sweep_ms"] / tr["sweep_launches"]
        achieved = per_solve_bytes * nsolves / (tr["sweep_ms"] * 1e-3) / 1e9
        kname = ((ELK_FULL_KERNELS if args.jac == "own" and not (p["cell"] == sy.CELL_GRU_DIAG or p["n"] == 1)
                  else ELK_KERNELS) if elk else
                 "k_chan_carry + k_chan_pass per sweep (carry scan; cell, Jacobian, update and the next "
                 "sweep's tile aggregates, or in the last sweep of a fixed count the adjoint's)" if chan else
                 ("k_pipe<SweepPol>" if scalar_path(p) and not approx else "k_time_sweep") +
                 " (fused cell + Jacobian + scan + update)")
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(p["name"]),
                    "kernel": kname,
                    "avg_launch_us": round(avg_ms * 1e3, 2),
                    "bytes_per_launch": per_solve_bytes / iters}
        if tr["adjoint_launches"] > 0:
            adj_ms = tr["adjoint_ms"] / tr["adjoint_launches"]
            extra["adjoint_kernel"] = {"avg_launch_us": round(adj_ms * 1e3, 2),
                                       "achieved_GBs": round(adjoint_bytes_per_unit(p) * wu / (adj_ms * 1e-3) / 1e9, 1)}
        pm, pn = bd.trace_kernel(bd.TRACE_PROJECTION)
        if pn > 0:
            flops = 2.0 * B * T * p["d"] * p["G"] * p["n"]
            peak = 2500.0 if p["dtype"] == sy.DT_BF16 else FP32_MFMA_PEAK_TFS
            tfs = flops / (pm / pn * 1e-3) / 1e12
            extra["projection_gemm"] = {"avg_launch_us": round(pm / pn * 1e3, 2), "TFLOP/s": round(tfs, 1),
                                        "peak": peak, "frac": round(tfs / peak, 4)}
        gm, gn = bd.trace_kernel(bd.TRACE_ADJOINT_PRODUCTS)
        if gn > 0:
            extra["adjoint_products_us"] = round(gm / gn * 1e3, 2)

    bd.trace(False)
    value = units / (ms_step * 1e-3)
    line = {
        "metric": "timesteps*batch/sec per converged Newton solve; scan HBM GB/s; speedup vs seq",
        "value": value,
        "unit": "timesteps*batch/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if p["dtype"] == 1 else "f32",
        "data": "synthetic",
        "config": {"workload": p["name"], "cell": sy.CELL_NAMES[p["cell"]], "B": B, "T": T, "d": p["d"],
                   "n": p["n"], "tol": p["tol"], "max_iters": p["max_iters"], "step": "solve + adjoint",
                   "jacobian": (("the cell's, ELK damping %g" if args.jac == "own" else
                                 "diagonal, quasi-ELK damping %g") % args.elk) if elk else
                               {"own": "the cell's", "diag": "diagonal (quasi-DEER)", "zero": "zero (Jacobi)"}[args.jac]},
        "iters": iters,
        "final_delta": float(dl[-1]) if len(dl) else None,
        "solve_ms": ms_solve,
        "solve_value": units / (ms_solve * 1e-3),
        **({"step_ms_without_speculation": no_spec_ms} if no_spec_ms is not None else {}),
        "roofline": roofline,
        **extra,
    }
    if args.config == 2 and args.jac == "own":
        # context only: the pages time the forward evaluation alone, on a V100
        line["pages_context"] = {"v100_deer_forward_ms": 15.0, "this_forward_ms": round(ms_solve, 4),
                                 "forward_ratio": round(15.0 / ms_solve, 2)}
    if not args.no_cpu_baseline:
        cb = cpu_baseline(p)
        line["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample", "host_cores",
                                                     "omp_threads")}
        line["speedup_vs_seq"] = cb["seconds"] / (ms_solve * 1e-3)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
