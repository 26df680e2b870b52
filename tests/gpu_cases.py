"""Shared driver for GPU-vs-oracle parity cases (imported by the gpu tests,
the smoke check and the benchmark's parity leg)."""
from __future__ import annotations

import numpy as np
import torch

import lazy_score_matrix_amd as pw
import oracle
from parity import assert_topk, assert_values, grad_rule, topk_report, value_report


def dev():
    return torch.device("cuda:0")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


SWAP = {"add_rows": "add_columns", "add_columns": "add_rows", "weight_rows": "weight_columns",
        "weight_columns": "weight_rows"}


def bind_case(arrays, c):
    """Both expressions of a workload case; a transposed case reduces over
    the rows, i.e. binds (Y, X) with row and column ops swapped."""
    import workloads
    ops = [(n, workloads.resolve(a, arrays)) for n, a in c.ops]
    X, Y = arrays[c.x], arrays[c.y]
    if getattr(c, "transpose", False):
        X, Y = Y, X
        ops = [(SWAP.get(n, n), a) for n, a in ops]
    return bind_both(X, Y, c.metric, c.gamma, ops, same=c.x == c.y)


def bind_both(X, Y, metric, gamma=1.0, ops=(), same=False):
    """The GPU expression and the oracle expression of one score."""
    tX = to_dev(X)
    tY = tX if same else to_dev(Y)
    def dev_arg(a):
        if isinstance(a, np.ndarray):
            return to_dev(a)
        if isinstance(a, tuple):
            return tuple(dev_arg(x) for x in a)
        return a
    gops = [(n, dev_arg(a)) for n, a in ops]
    e = pw.lazy(tX, tY, metric, gamma=gamma, ops=gops)
    oe = oracle.Expr(X, X if same else Y, metric, gamma=gamma, ops=list(ops))
    return e, oe


EPS = {np.dtype(np.float32): 2.0 ** -24, np.dtype(np.float64): 2.0 ** -53}


def solve_report(oe, A, B, shift, rtol, rows=None):
    """Check a CG solution of (S + shift I) A = B against the oracle: the
    true residual r = B - (S + shift I) A (oracle product, higher precision)
    within rtol of |B| up to the recurrence's rounding drift, and, on a full
    system, |A - A*| <= |r| / shift per column (the smallest eigenvalue of
    S + shift I is at least shift for S positive semi-definite), A* the
    dense solve. On a row sample the residual is compared with |B| scaled
    to the sample's share of the rows (3x slack). Returns (ok, worst
    residual / bound)."""
    dtype = np.dtype(oe.np_dtype)
    A = np.asarray(A, np.float64).reshape(oe.N, -1)
    B64 = np.asarray(B, np.float64).reshape(oe.N, -1)
    KA, mag = oracle.matmul(oe, A.astype(dtype), rows)
    sel = slice(None) if rows is None else rows
    res = B64[sel] - (np.asarray(KA, np.float64) + shift * A[sel])
    rn = np.linalg.norm(res, axis=0)
    drift = 8 * oe.N * EPS[dtype] * (np.linalg.norm(np.asarray(mag, np.float64), axis=0)
                                     + shift * np.linalg.norm(A[sel], axis=0))
    if rows is None:
        bound = 1.05 * rtol * np.linalg.norm(B64, axis=0) + drift
    else:
        bound = 3 * rtol * np.sqrt(len(rows) / oe.N) * np.linalg.norm(B64, axis=0) + drift
    ok = bool(np.all(rn <= bound + 1e-300))
    if rows is None and ok:
        Astar, _ = oracle.solve(oe, shift, B64.astype(dtype))
        err = np.linalg.norm(A - Astar, axis=0)
        ok = bool(np.all(err <= (rn + drift) / shift * 1.01 + 1e-300))
    return ok, float(np.max(rn / np.maximum(bound, 1e-300)))


def grad_report(g, ref, dtype, terms, needed=None):
    """(ok, worst |gpu - oracle| / tol) for one gradient by parity.grad_rule:
    tol = rtol * (mag + |oracle|), rtol 1e-5 (float32) or 1e-12 (float64),
    mag the oracle's first-order error magnitude of that gradient (the
    header of oracle.cpp derives it term by term). `terms` (pairs summed)
    is informational. With `needed` (a list), also appends the worst
    |gpu - oracle| / (mag + |oracle|), the relative tolerance the case
    actually needs."""
    val, mag = ref
    ok, ratio, rel = grad_rule(g.detach().cpu().numpy(), val, mag, dtype)
    if needed is not None:
        needed.append(rel)
    return ok, ratio


def check_backward(e, oe, consumer, G, V=None, k=0, exclude_self=False, rows=None, cols=None, report=False,
                   what="", want=("X", "Y", "V", "ops")):
    """GPU backward of `consumer` against the oracle's chain rule: dX and
    row-op grads on `rows`, dY, dV and column-op grads on `cols` (all by
    default). Returns (ok, worst ratio) with report=True, else asserts."""
    dtype = np.dtype(oe.np_dtype)
    out = idx = None
    Vd = None if V is None else to_dev(V)
    if consumer == "softmax_matmul":
        out = e.softmax_matmul(Vd)
    elif consumer == "topk":
        _, idx = e.topk(k)
    got = e.backward(consumer, to_dev(G), V=Vd, out=out, indices=idx, exclude_self=exclude_self, want=want)
    ref = oracle.backward(oe, consumer, G, V, exclude_self=exclude_self,
                          indices=None if idx is None else idx.cpu().numpy(), rows=rows, cols=cols)
    sel_r = slice(None) if rows is None else torch.as_tensor(rows, device=dev())
    sel_c = slice(None) if cols is None else torch.as_tensor(cols, device=dev())
    checks = [("dX", got["X"][sel_r], ref["dX"], oe.M), ("dY", got["Y"][sel_c], ref["dY"], oe.N)]
    if V is not None:
        checks.append(("dV", got["V"][sel_c], ref["dV"], oe.N))
    for t, (name, _) in enumerate(oe.op_list):
        if ref["ops"][t] is not None and "ops" in want:
            rowop = name.endswith("_rows")
            checks.append(("op %d %s" % (t, name), got["ops"][t][sel_r if rowop else sel_c], ref["ops"][t],
                           oe.M if rowop else oe.N))
    worst, ok = 0.0, True
    for name, g, r, terms in checks:
        need = []
        good, ratio = grad_report(g, r, dtype, terms, need)
        print("GRAD %s %s %s terms=%d worst_err_over_tol=%.3g needed_rtol=%.3g"
              % (what, name, np.dtype(dtype).name, terms, ratio, need[0]), flush=True)
        worst = max(worst, ratio)
        if not report:
            assert good, "%s %s: worst |gpu - oracle| / tol = %.3g" % (what, name, ratio)
        ok &= good
    return ok, worst


def check_consumer(e, oe, consumer, V=None, exclude_self=False, k=0, largest=False, rows=None, exact=False,
                   what="", report=False, params=None):
    """Run `consumer` on the GPU and the oracle (optionally on a row subset of
    the oracle side) and assert parity. Returns (worst err/tol, plain rel)."""
    dtype = np.dtype(oe.np_dtype)
    if consumer.startswith("backward_"):
        p = dict(params or {})
        ok, ratio = check_backward(e, oe, consumer[len("backward_"):], p["G"], V=V, k=k, exclude_self=exclude_self,
                                   rows=rows, cols=None if rows is None else p.get("cols", rows), report=report,
                                   what=what)
        return (ok, ratio) if report else (ratio, 0.0)
    if consumer == "mmd":
        # One statistic for the whole pair of clouds: the oracle's, from
        # its dense scores (row samples do not apply).
        import lazy_score_matrix_amd as pw
        from parity import value_report
        unbiased = dict(params or {}).get("unbiased", True)
        g = pw.mmd_statistics(e.X, e.Y, e.metric, e.gamma, unbiased).cpu().numpy()
        o, mag = oracle.mmd2(oe.X, oe.Y, oe.metric, oe.gamma, unbiased)
        ok, ratio, rel = value_report(np.atleast_1d(g), np.atleast_1d(o), np.atleast_1d(mag), dtype,
                                      n_terms=oe.N * oe.M)
        if report:
            return ok, ratio
        assert ok, (what, "worst err/tol", ratio)
        return ratio, rel
    if consumer == "cg_solve":
        p = dict(params or {})
        A, info = e.solve(to_dev(V), p["shift"], rtol=p["rtol"], max_iter=p.get("max_iter", 1000))
        ok, ratio = solve_report(oe, A.cpu().numpy(), V, p["shift"], p["rtol"], rows)
        if report:
            return ok and info["converged"], ratio, info
        assert info["converged"], (what, info)
        assert ok, (what, "residual / bound", ratio, info)
        return ratio, info["max_rel_residual"]
    sel = slice(None) if rows is None else torch.as_tensor(rows, device=dev())
    vmax = float(np.max(np.abs(V))) if V is not None and V.size else 1.0
    if consumer == "matmul":
        g = e.matmul(to_dev(V))[sel]
        o, mag = oracle.matmul(oe, V, rows)
    elif consumer == "softmax_matmul":
        g = e.softmax_matmul(to_dev(V))[sel]
        o, mag = oracle.softmax_matmul(oe, V, rows)
    elif consumer == "displacement":
        g = e.displacement()[sel]
        o, mag = oracle.displacement(oe, rows)
        vmax = float(max(np.max(np.abs(oe.X)) if oe.X.size else 0, np.max(np.abs(oe.Y)) if oe.Y.size else 0, 1))
    elif consumer == "logsumexp":
        g = e.logsumexp(exclude_self=exclude_self)[sel]
        o, mag = oracle.logsumexp(oe, exclude_self=exclude_self, rows=rows)
    elif consumer == "mean":
        g = e.mean()[sel][:, None]
        o, mag = oracle.matmul(oe, np.ones((oe.M, 1), dtype=oe.np_dtype), rows)
        o, mag = o / oe.M, mag / oe.M
    elif consumer == "topk":
        gv, gi = e.topk(k, largest=largest)
        gv, gi = gv[sel].cpu().numpy(), gi[sel].cpu().numpy()
        ov, oi, om = oracle.topk(oe, k, largest=largest, extra=16, rows=rows)
        if report:
            return topk_report(gv, gi, ov, oi, om, k, largest, dtype, exact)
        assert_topk(gv, gi, ov, oi, om, k, largest, dtype, exact=exact, what=what)
        return 0.0, 0.0
    else:
        raise ValueError(consumer)
    g = g.cpu().numpy()
    if report:
        return value_report(g, o, mag, dtype, n_terms=max(oe.M, 1), vmax=vmax)
    return assert_values(g, o, mag, dtype, n_terms=max(oe.M, 1), vmax=vmax, what=what)
