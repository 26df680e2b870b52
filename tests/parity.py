"""Comparison rules between the GPU library and the CPU oracle.

Values: |g - o| <= rtol * max(|o|, mag) + atol, element by element, where
mag is the oracle's first-order error magnitude of that output and
rtol = 1e-5 (float32) or 1e-12 (float64). The torchpairwise guide ("What to
Check", Precision) says fused kernels agree with other summation orders only
within floating tolerance; mag scales that tolerance to the conditioning of
each output. atol = n_terms * smallest normal * max|V| only absorbs
flush-to-zero differences. -inf must match -inf exactly.

Gradients: |g - o| <= rtol * (mag + |o|) with the same rtol, mag the
oracle's first-order error magnitude of that gradient.

Top-k: indices must be distinct and in range, values sorted with equal
values in ascending index order, each returned index must carry the value
the oracle gives it at that position (within tolerance), and wherever the
oracle's value at a position is separated by more than the tolerance from
its neighbours the index must equal the oracle's. With exact=True (integer
data) indices and values must match bit for bit.
"""
from __future__ import annotations

import numpy as np

RTOL = {np.dtype(np.float32): 1e-5, np.dtype(np.float64): 1e-12}
TINY = {np.dtype(np.float32): np.finfo(np.float32).tiny, np.dtype(np.float64): np.finfo(np.float64).tiny}


def to_np(t):
    return t.detach().cpu().numpy()


def value_report(g, o, mag, dtype, n_terms=1, vmax=1.0):
    """Returns (ok, worst ratio err/tol, max plain relative error)."""
    dtype = np.dtype(dtype)
    real = np.longdouble if dtype == np.float64 else np.float64
    g = np.asarray(g).astype(real)
    o = np.asarray(o).astype(real)
    mag = np.asarray(mag).astype(real)
    if g.shape != o.shape:
        raise AssertionError("shape %s vs oracle %s" % (g.shape, o.shape))
    if g.size == 0:
        return True, 0.0, 0.0
    ninf = np.isneginf(o)
    if np.any(np.isneginf(g) != ninf):
        return False, float("inf"), float("inf")
    fin = ~ninf
    if not np.all(np.isfinite(g[fin])):
        return False, float("inf"), float("inf")
    err = np.abs(g[fin] - o[fin])
    tol = RTOL[dtype] * np.maximum(np.abs(o[fin]), mag[fin]) + n_terms * TINY[dtype] * vmax
    ratio = float(np.max(err / tol)) if err.size else 0.0
    rel = float(np.max(err / np.maximum(np.abs(o[fin]), TINY[dtype]))) if err.size else 0.0
    return ratio <= 1.0, ratio, rel


def grad_rule(g, o, mag, dtype):
    """Gradients follow the same rule with the oracle's first-order
    gradient magnitude: |g - o| <= rtol (mag + |o|). Returns (ok, worst
    err/tol, worst |g - o| / (mag + |o|))."""
    dtype = np.dtype(dtype)
    o = np.asarray(o, np.float64)
    m = np.asarray(mag, np.float64)
    g = np.asarray(g, np.float64).reshape(o.shape)
    if o.size == 0:
        return True, 0.0, 0.0
    scale = m + np.abs(o) + 1e-300
    rel = float(np.max(np.abs(g - o) / scale))
    return rel <= RTOL[dtype], rel / RTOL[dtype], rel


def assert_values(g, o, mag, dtype, n_terms=1, vmax=1.0, what=""):
    ok, ratio, rel = value_report(g, o, mag, dtype, n_terms, vmax)
    assert ok, "%s: worst err/tol %.3g (plain rel err %.3g)" % (what, ratio, rel)
    return ratio, rel


def topk_report(gv, gi, ov, oi, omag, k, largest, dtype, exact=False):
    """Check GPU top-k (gv, gi: [R, k]) against the oracle's extended lists
    (ov, oi, omag: [R, k + extra]). Returns a list of failure strings."""
    dtype = np.dtype(dtype)
    real = np.longdouble if dtype == np.float64 else np.float64
    gv = np.asarray(gv).astype(real)
    gi = np.asarray(gi).astype(np.int64)
    ov = np.asarray(ov).astype(real)
    oi = np.asarray(oi).astype(np.int64)
    omag = np.asarray(omag).astype(real)
    rtol = RTOL[dtype]
    fails = []
    R = gv.shape[0]
    for r in range(R):
        # Rows with fewer kept pairs than k (masks): the oracle pads with
        # index -1 / NaN, and so must the GPU, past the same count.
        nv = int(np.sum(oi[r, :k] >= 0))
        if exact:
            if not np.array_equal(gi[r], oi[r, :k]) or not np.array_equal(gv[r], ov[r, :k], equal_nan=True):
                fails.append("row %d: exact mismatch gpu %s vs oracle %s" % (r, gi[r].tolist(), oi[r, :k].tolist()))
            continue
        if np.any(gi[r, nv:] != -1) or not np.all(np.isnan(gv[r, nv:])):
            fails.append("row %d: %d kept pairs, but positions past them are %s / %s"
                         % (r, nv, gi[r, nv:].tolist(), gv[r, nv:].tolist()))
            continue
        idx = gi[r, :nv]
        if len(set(idx.tolist())) != nv or (nv and idx.min() < 0):
            fails.append("row %d: indices not distinct / negative %s" % (r, idx.tolist()))
            continue
        v = gv[r]
        for p in range(nv - 1):
            before = v[p] > v[p + 1] if largest else v[p] < v[p + 1]
            if not (before or (v[p] == v[p + 1] and idx[p] < idx[p + 1])):
                fails.append("row %d: order broken at %d (%r,%d) (%r,%d)" % (r, p, v[p], idx[p], v[p + 1], idx[p + 1]))
                break
        pos = {j: q for q, j in enumerate(oi[r].tolist()) if j >= 0}
        tol = rtol * np.maximum(np.abs(ov[r]), omag[r])
        for p in range(nv):
            q = pos.get(int(idx[p]))
            if q is None:
                fails.append("row %d pos %d: index %d not among the oracle's first %d" % (r, p, idx[p], ov.shape[1]))
                break
            if abs(ov[r, q] - ov[r, p]) > tol[p] or abs(v[p] - ov[r, q]) > tol[q]:
                fails.append("row %d pos %d: value of index %d off (oracle %r at its pos %d, %r at pos %d, gpu %r)"
                             % (r, p, idx[p], ov[r, q], q, ov[r, p], p, v[p]))
                break
            sep_prev = p == 0 or abs(ov[r, p] - ov[r, p - 1]) > tol[p]
            sep_next = p + 1 >= ov.shape[1] or np.isnan(ov[r, p + 1]) or abs(ov[r, p + 1] - ov[r, p]) > tol[p]
            if sep_prev and sep_next and idx[p] != oi[r, p]:
                fails.append("row %d pos %d: separated value but index %d != oracle %d" % (r, p, idx[p], oi[r, p]))
                break
    return fails


def assert_topk(gv, gi, ov, oi, omag, k, largest, dtype, exact=False, what=""):
    fails = topk_report(gv, gi, ov, oi, omag, k, largest, dtype, exact)
    assert not fails, "%s: %d failing rows, first: %s" % (what, len(fails), fails[:3])
