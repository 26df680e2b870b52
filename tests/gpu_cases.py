"""Shared driver for GPU-vs-oracle parity cases (imported by the gpu tests,
the smoke check and the benchmark's parity leg)."""
from __future__ import annotations

import numpy as np
import torch

import lazy_score_matrix_amd as pw
import oracle
from parity import assert_topk, assert_values, topk_report, value_report


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


def check_consumer(e, oe, consumer, V=None, exclude_self=False, k=0, largest=False, rows=None, exact=False,
                   what="", report=False):
    """Run `consumer` on the GPU and the oracle (optionally on a row subset of
    the oracle side) and assert parity. Returns (worst err/tol, plain rel)."""
    dtype = np.dtype(oe.np_dtype)
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
