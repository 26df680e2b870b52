"""CPU oracle for lazily evaluated pairwise scores (test infrastructure only).

Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package. The product library never does, and this
package never imports the product: the two share no code.

The arithmetic lives in ``oracle.cpp`` (a plain double loop over pairs,
float32 inputs evaluated in double and float64 inputs in x87 long double);
this module only builds it with g++ and marshals numpy arrays through ctypes.
The definitions it follows are those of the torchpairwise guide "Using
Torchpairwise in Models" (Task Map, Score Expressions and the Stein
Variational Gradient Descent section); each function below names its part.

Every function returns ``(result, mag)``: ``mag`` is the first-order error
magnitude of each result (see the header of ``oracle.cpp``), which the
parity tests use to scale the floating tolerance the guide's "What to Check"
section says fused kernels agree within. Results are numpy float64 arrays for
float32 inputs and numpy longdouble arrays for float64 inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
# PW_ORACLE_LIBRARY names a prebuilt oracle (e.g. a sanitized build); build()
# then leaves it as it is.
_PREBUILT = os.environ.get("PW_ORACLE_LIBRARY")
_LIB = _PREBUILT or os.path.join(_HERE, "liboracle.so")

# Score-arithmetic op codes understood by oracle.cpp (its own numbering).
OPS = {
    "mul": 0,             # s <- c * s
    "add": 1,             # s <- s + c
    "add_rows": 2,        # s <- s + a_i
    "add_columns": 3,     # s <- s + b_j
    "weight_rows": 4,     # s <- w_i * s
    "weight_columns": 5,  # s <- u_j * s
    "exp": 6,             # s <- exp(s)
}
METRICS = {"linear": 0, "sqeuclidean": 1, "rbf": 2, "cosine_distances": 3}
# Masks, given in the same op list (Score Expressions: boolean row/column
# masks; Task Map, Attention row: causal, band, same_group). A mask drops
# pairs from every consumer wherever it stands in the list:
#   ("mask_rows", bool[N]), ("mask_columns", bool[M])
#   ("causal", d)          keep j - i <= d (d = 0: j <= i)
#   ("band", (lo, hi))     keep -lo <= j - i <= hi
#   ("same_group", (g_rows[N], g_cols[M]))   keep g_rows[i] == g_cols[j]
MASKS = ("mask_rows", "mask_columns", "causal", "band", "same_group")

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile liboracle.so with g++ (OpenMP, no fast-math). Returns its path."""
    if _PREBUILT:
        return _LIB
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", "-Wall", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _CExpr(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("metric", ctypes.c_int),
        ("gamma", ctypes.c_double),
        ("X", ctypes.c_void_p),
        ("N", ctypes.c_int64),
        ("ldx", ctypes.c_int64),
        ("Y", ctypes.c_void_p),
        ("M", ctypes.c_int64),
        ("ldy", ctypes.c_int64),
        ("D", ctypes.c_int64),
        ("n_ops", ctypes.c_int),
        ("op_kind", ctypes.POINTER(ctypes.c_int)),
        ("op_scalar", ctypes.POINTER(ctypes.c_double)),
        ("op_vec", ctypes.POINTER(ctypes.c_void_p)),
        ("row_mask", ctypes.c_void_p),
        ("col_mask", ctypes.c_void_p),
        ("has_upper", ctypes.c_int),
        ("upper", ctypes.c_int64),
        ("has_lower", ctypes.c_int),
        ("lower", ctypes.c_int64),
        ("group_rows", ctypes.c_void_p),
        ("group_cols", ctypes.c_void_p),
    ]


def _open(path: str):
    """Open an oracle build at `path` and declare its C signatures."""
    lib = ctypes.CDLL(path)
    vp, i64, p64 = ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)
    pe = ctypes.POINTER(_CExpr)
    lib.oracle_scores.argtypes = [pe, p64, i64, vp, vp]
    lib.oracle_matmul.argtypes = [pe, vp, i64, i64, p64, i64, vp, vp]
    lib.oracle_displacement.argtypes = [pe, p64, i64, vp, vp]
    lib.oracle_logsumexp.argtypes = [pe, ctypes.c_int, p64, i64, vp, vp]
    lib.oracle_softmax_matmul.argtypes = [pe, vp, i64, i64, p64, i64, vp, vp]
    lib.oracle_topk.argtypes = [pe, ctypes.c_int, ctypes.c_int, p64, i64, vp, p64, vp]
    lib.oracle_backward.argtypes = [pe, ctypes.c_int, vp, i64, vp, i64, i64, ctypes.c_int, p64, ctypes.c_int,
                                    p64, i64, p64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_real_size.argtypes = [ctypes.c_int]
    lib.oracle_real_size.restype = ctypes.c_int
    assert lib.oracle_real_size(1) == np.dtype(np.longdouble).itemsize, "long double layout mismatch"
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            _lib = _open(build())
    return _lib


def set_threads(n: int) -> None:
    """Number of OpenMP threads every later oracle call uses."""
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _rows2d(a, dtype):
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s array, got %s" % (dtype, a.dtype))
    if a.ndim != 2:
        raise ValueError("expected a 2-D array")
    if a.shape[0] > 0 and a.strides[1] != a.itemsize and a.shape[1] > 1:
        a = np.ascontiguousarray(a)
    if a.strides[0] % a.itemsize:
        a = np.ascontiguousarray(a)
    ld = a.strides[0] // a.itemsize if a.shape[0] > 1 else a.shape[1]
    return a, max(int(ld), a.shape[1])


class Expr:
    """A bound pairwise score: metric on rows of X [N,D] and Y [M,D], then ops.

    ``ops`` is a list of ``(name, arg)`` with name in ``OPS``: ``arg`` is a
    float for "mul"/"add", a length-N array for "add_rows"/"weight_rows", a
    length-M array for "add_columns"/"weight_columns" and ``None`` for "exp"
    (Score Expressions section), or a mask of ``MASKS``.
    """

    def __init__(self, X, Y, metric, gamma=1.0, ops=()):
        X = np.asarray(X)
        if X.dtype not in (np.float32, np.float64):
            raise TypeError("oracle inputs are float32 or float64")
        self.np_dtype = X.dtype
        self.X, ldx = _rows2d(X, X.dtype)
        self.Y, ldy = _rows2d(Y, X.dtype)
        if self.X.shape[1] != self.Y.shape[1]:
            raise ValueError("X and Y feature dims differ")
        self.N, self.D = self.X.shape
        self.M = self.Y.shape[0]
        self.metric = metric
        self.gamma = float(gamma)
        self.real = np.float64 if X.dtype == np.float32 else np.longdouble
        self._keep = []
        kinds, scalars, vecs = [], [], []
        row_mask = col_mask = groups = None
        upper = lower = None
        self.op_list = []  # the score arithmetic ops, masks left out
        for name, arg in ops:
            if name in MASKS:
                if name == "mask_rows":
                    m = np.asarray(arg, dtype=bool).reshape(-1)
                    if m.shape[0] != self.N:
                        raise ValueError("mask_rows needs %d values" % self.N)
                    row_mask = m if row_mask is None else (row_mask & m)
                elif name == "mask_columns":
                    m = np.asarray(arg, dtype=bool).reshape(-1)
                    if m.shape[0] != self.M:
                        raise ValueError("mask_columns needs %d values" % self.M)
                    col_mask = m if col_mask is None else (col_mask & m)
                elif name == "causal":
                    d = 0 if arg is None else int(arg)
                    upper = d if upper is None else min(upper, d)
                elif name == "band":
                    lo, hi = int(arg[0]), int(arg[1])
                    upper = hi if upper is None else min(upper, hi)
                    lower = lo if lower is None else min(lower, lo)
                else:
                    if groups is not None:
                        raise ValueError("one same_group mask per expression")
                    gr = np.ascontiguousarray(np.asarray(arg[0], dtype=np.int64).reshape(-1))
                    gc = np.ascontiguousarray(np.asarray(arg[1], dtype=np.int64).reshape(-1))
                    if gr.shape[0] != self.N or gc.shape[0] != self.M:
                        raise ValueError("same_group needs %d row and %d column groups" % (self.N, self.M))
                    groups = (gr, gc)
                continue
            kinds.append(OPS[name])
            self.op_list.append((name, arg))
            if name in ("mul", "add"):
                scalars.append(float(arg))
                vecs.append(None)
            elif name == "exp":
                scalars.append(0.0)
                vecs.append(None)
            else:
                n = self.N if name.endswith("_rows") else self.M
                v = np.ascontiguousarray(np.asarray(arg, dtype=X.dtype).reshape(-1))
                if v.shape[0] != n:
                    raise ValueError("%s needs %d values" % (name, n))
                self._keep.append(v)
                scalars.append(0.0)
                vecs.append(v.ctypes.data)
        nops = len(kinds)
        self._kinds = (ctypes.c_int * max(nops, 1))(*kinds)
        self._scalars = (ctypes.c_double * max(nops, 1))(*scalars)
        self._vecs = (ctypes.c_void_p * max(nops, 1))(*vecs)
        masks = []
        for m in (row_mask, col_mask):
            m = None if m is None else np.ascontiguousarray(m.astype(np.uint8))
            masks.append(m)
            self._keep.append(m)
        if groups is not None:
            self._keep.extend(groups)
        self.masked = any(m is not None for m in masks) or upper is not None or lower is not None or \
            groups is not None
        self._c = _CExpr(
            0 if X.dtype == np.float32 else 1, METRICS[metric], self.gamma,
            self.X.ctypes.data, self.N, ldx, self.Y.ctypes.data, self.M, ldy, self.D,
            nops, self._kinds, self._scalars, self._vecs,
            None if masks[0] is None else masks[0].ctypes.data,
            None if masks[1] is None else masks[1].ctypes.data,
            int(upper is not None), 0 if upper is None else upper,
            int(lower is not None), 0 if lower is None else lower,
            None if groups is None else groups[0].ctypes.data,
            None if groups is None else groups[1].ctypes.data)

    def _rows(self, rows):
        if rows is None:
            return None, self.N
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
        if r.size and (r.min() < 0 or r.max() >= self.N):
            raise IndexError("row index out of range")
        return r, r.shape[0]

    def _out(self, *shape):
        return np.empty(shape, dtype=self.real), np.empty(shape, dtype=self.real)

    def _V(self, V):
        V, ldv = _rows2d(V, self.np_dtype)
        if V.shape[0] != self.M:
            raise ValueError("V needs M rows")
        return V, ldv


def _rp(r):
    return None if r is None else r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def scores(e: Expr, rows=None):
    """Dense scores s_ij for the listed rows (Score Expressions); masks are
    not applied here (they act in the consumers)."""
    lib = _load()
    r, n = e._rows(rows)
    out, mag = e._out(n, e.M)
    lib.oracle_scores(ctypes.byref(e._c), _rp(r), n, out.ctypes.data, mag.ctypes.data)
    return out, mag


def matmul(e: Expr, V, rows=None):
    """Kernel product sum_j s_ij V[j,:] (Task Map, Nadaraya-Watson row)."""
    lib = _load()
    V, ldv = e._V(V)
    r, n = e._rows(rows)
    out, mag = e._out(n, V.shape[1])
    lib.oracle_matmul(ctypes.byref(e._c), V.ctypes.data, V.shape[1], ldv, _rp(r), n, out.ctypes.data,
                      mag.ctypes.data)
    return out, mag


def displacement(e: Expr, rows=None):
    """sum_j s_ij (y_j - x_i) (Stein Variational Gradient Descent section)."""
    lib = _load()
    r, n = e._rows(rows)
    out, mag = e._out(n, e.D)
    lib.oracle_displacement(ctypes.byref(e._c), _rp(r), n, out.ctypes.data, mag.ctypes.data)
    return out, mag


def logsumexp(e: Expr, exclude_self=False, rows=None):
    """Row log-sum-exp over j, optionally without j == i (Task Map, InfoNCE row)."""
    lib = _load()
    r, n = e._rows(rows)
    out, mag = e._out(n)
    lib.oracle_logsumexp(ctypes.byref(e._c), int(bool(exclude_self)), _rp(r), n, out.ctypes.data,
                         mag.ctypes.data)
    return out, mag


def softmax_matmul(e: Expr, V, rows=None):
    """softmax over j of s_ij, then @ V (Intro example; Task Map, Attention row)."""
    lib = _load()
    V, ldv = e._V(V)
    r, n = e._rows(rows)
    out, mag = e._out(n, V.shape[1])
    lib.oracle_softmax_matmul(ctypes.byref(e._c), V.ctypes.data, V.shape[1], ldv, _rp(r), n,
                              out.ctypes.data, mag.ctypes.data)
    return out, mag


def topk(e: Expr, k, largest=False, extra=0, rows=None):
    """Row top-k by value, ties by lowest index (Task Map, k-NN and Chamfer rows).

    Returns ``(values, indices, mag)`` with ``k + extra`` positions per row;
    positions past the row's kept pairs hold NaN / -1.
    """
    lib = _load()
    r, n = e._rows(rows)
    kk = int(k) + int(extra)
    vals, mag = e._out(n, kk)
    idx = np.empty((n, kk), dtype=np.int64)
    lib.oracle_topk(ctypes.byref(e._c), kk, int(bool(largest)), _rp(r), n, vals.ctypes.data,
                    idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), mag.ctypes.data)
    return vals, idx, mag


CONSUMER_CODES = {"matmul": 0, "displacement": 1, "logsumexp": 2, "softmax_matmul": 3, "topk": 4}


def backward(e: Expr, consumer, G, V=None, exclude_self=False, indices=None, rows=None, cols=None):
    """First-order gradients of a consumer's output contracted with the
    upstream gradient G (guide: backward by replay; selections route
    gradients through the selected pairs only), per pair from the chain rule
    (see oracle.cpp). Row-side results (dX, row-op grads) for `rows`,
    column-side results (dY, dV, column-op grads) for `cols` (all by
    default). Returns a dict of arrays with their first-order error
    magnitudes (see oracle.cpp): dX, dY, dV, and "ops": per op its grad
    (rows or columns, None for a scalar op), each as (value, mag)."""
    lib = _load()
    code = CONSUMER_CODES[consumer]
    G = np.ascontiguousarray(np.asarray(G, dtype=e.np_dtype))
    if G.ndim == 1:
        G = G[:, None]
    if G.shape[0] != e.N:
        raise ValueError("G needs N rows")
    if V is not None:
        V, ldv = e._V(V)
        C = V.shape[1]
    else:
        V, ldv, C = None, 0, 0
    idx = None
    k = 0
    if indices is not None:
        idx = np.ascontiguousarray(np.asarray(indices, dtype=np.int64))
        k = idx.shape[1]
    r = np.arange(e.N, dtype=np.int64) if rows is None else np.ascontiguousarray(np.asarray(rows, np.int64))
    c = np.arange(e.M, dtype=np.int64) if cols is None else np.ascontiguousarray(np.asarray(cols, np.int64))
    nr, nc = r.shape[0], c.shape[0]
    n_ops = len(e._kinds) if e._c.n_ops else 0
    buf = {}
    for name, shape in (("dX", (nr, e.D)), ("dY", (nc, e.D)), ("dV", (nc, max(C, 1))),
                        ("dOr", (max(n_ops, 1), nr)), ("dOc", (max(n_ops, 1), nc))):
        buf[name] = np.zeros(shape, dtype=e.real)
        buf[name + "m"] = np.zeros(shape, dtype=e.real)
    p64 = ctypes.POINTER(ctypes.c_int64)
    lib.oracle_backward(ctypes.byref(e._c), code, G.ctypes.data, G.shape[1], None if V is None else V.ctypes.data, C,
                        ldv, int(bool(exclude_self)), None if idx is None else idx.ctypes.data_as(p64), k,
                        r.ctypes.data_as(p64), nr, c.ctypes.data_as(p64), nc,
                        *[buf[n].ctypes.data for n in ("dX", "dXm", "dY", "dYm", "dV", "dVm", "dOr", "dOrm", "dOc",
                                                       "dOcm")])
    ops = []
    names = [n for n, _ in e.op_list]
    for t, name in enumerate(names):
        if name in ("add_rows", "weight_rows"):
            ops.append((buf["dOr"][t], buf["dOrm"][t]))
        elif name in ("add_columns", "weight_columns"):
            ops.append((buf["dOc"][t], buf["dOcm"][t]))
        else:
            ops.append(None)
    return {"dX": (buf["dX"], buf["dXm"]), "dY": (buf["dY"], buf["dYm"]),
            "dV": (buf["dV"][:, :C], buf["dVm"][:, :C]), "ops": ops}


def solve(e: Expr, shift, B):
    """The exact solution of (S + shift * I) A = B for a square score S
    (Task Map, Kernel ridge / GP mean row: solve(K + a * eye_like(K), Y)):
    dense oracle scores, then a dense LU solve in float64 (numpy). Returns
    (A, cond) with cond the 2-norm condition number of S + shift * I, which
    bounds how far an iterative solution with a small residual may sit from A.
    """
    if e.N != e.M:
        raise ValueError("solve needs a square score")
    S, _ = scores(e)
    Kd = np.asarray(S, np.float64) + float(shift) * np.eye(e.N)
    Bd = np.asarray(B, np.float64).reshape(e.N, -1)
    return np.linalg.solve(Kd, Bd), float(np.linalg.cond(Kd))


def svgd_direction(x, score, gamma, rows=None):
    """SVGD direction (K@score - 2*gamma*K.displacement()) / n with K = rbf(x, x).

    The host composition of two consumers, as in the SVGD section's
    ``svgd_direction``; ``n`` is the number of particles.
    """
    e = Expr(x, x, "rbf", gamma=gamma)
    km, km_mag = matmul(e, score, rows)
    kd, kd_mag = displacement(e, rows)
    n = e.N
    g = e.real(gamma)
    phi = (km - 2 * g * kd) / n
    mag = (km_mag + 2 * g * kd_mag) / n
    return phi, mag


def mmd2(X, Y, metric="rbf", gamma=1.0, unbiased=True):
    """Squared maximum mean discrepancy between point clouds X [n, D] and
    Y [m, D] under the kernel k = the bound score (Task Map, MMD row:
    mmd_statistics, unbiased by default; one feature set is one cloud), from
    the dense oracle scores:
      unbiased: sum_{i != i'} k(x_i, x_i') / (n (n - 1))
                + sum_{j != j'} k(y_j, y_j') / (m (m - 1))
                - 2 sum_{i, j} k(x_i, y_j) / (n m)
      biased:   every pair, diagonals included, over n^2 and m^2.
    Batched clouds X [B, n, D] with Y [B or 1, m, D] give one value per
    element. Returns (value, mag): mag sums the three terms' magnitudes
    (|k| plus its first-order error magnitude, over the same pairs and
    weights), so that cancellation between the terms keeps a tolerance."""
    X = np.asarray(X)
    Y = np.asarray(Y)
    if X.ndim == 3:
        Yb = Y if Y.ndim == 3 else Y[None]
        outs = [mmd2(X[b], Yb[b if Yb.shape[0] > 1 else 0], metric, gamma, unbiased) for b in range(X.shape[0])]
        return np.array([o[0] for o in outs]), np.array([o[1] for o in outs])
    n, m = X.shape[0], Y.shape[0]
    if unbiased and (n < 2 or m < 2):
        raise ValueError("the unbiased statistic needs at least two points per cloud")

    def term(A, B, same):
        e = Expr(A, B, metric, gamma=gamma)
        k, mk = scores(e)
        real = k.dtype
        k = np.asarray(k, real)
        a = np.abs(k) + np.asarray(mk, real)
        if same and unbiased:
            keep = ~np.eye(k.shape[0], dtype=bool)
            return k[keep].sum(), a[keep].sum(), real
        return k.sum(), a.sum(), real

    sxx, axx, real = term(X, X, True)
    syy, ayy, _ = term(Y, Y, True)
    sxy, axy, _ = term(X, Y, False)
    one = real.type(1)
    cx = one / (n * (n - 1)) if unbiased else one / (n * n)
    cy = one / (m * (m - 1)) if unbiased else one / (m * m)
    cxy = one / (n * m)
    value = cx * sxx + cy * syy - 2 * cxy * sxy
    mag = cx * axx + cy * ayy + 2 * cxy * axy
    return value, mag


def mmd2_grad(X, Y, metric="rbf", gamma=1.0, unbiased=True, G=1.0):
    """Gradients of G * mmd2(X, Y) with respect to both clouds: each of the
    statistic's three sums is the kernel product of its pairs with a column
    of ones, so its gradient is that product's chain-rule backward (row and
    column sides) with the sum's coefficient as upstream gradient; distinct
    pairs of one cloud are its two strict triangles (band masks j > i and
    j < i). Batched clouds ([B, n, D] with Y [B or 1, m, D], G [B]) give
    per-element gradients; a cloud shared by the batch gets their sum.
    Returns ((dX, dX_mag), (dY, dY_mag)), each mag summing its pieces'."""
    X = np.asarray(X)
    Y = np.asarray(Y)
    if X.ndim == 3:
        Yb = Y if Y.ndim == 3 else Y[None]
        Gb = np.broadcast_to(np.asarray(G, np.float64), (X.shape[0],))
        parts = [mmd2_grad(X[b], Yb[b if Yb.shape[0] > 1 else 0], metric, gamma, unbiased, Gb[b])
                 for b in range(X.shape[0])]
        dX = np.stack([p[0][0] for p in parts]), np.stack([p[0][1] for p in parts])
        dY = np.stack([p[1][0] for p in parts]), np.stack([p[1][1] for p in parts])
        if Yb.shape[0] == 1 and X.shape[0] > 1:
            dY = dY[0].sum(0, keepdims=True), dY[1].sum(0, keepdims=True)
        return dX, dY
    n, m = X.shape[0], Y.shape[0]
    g = float(G)

    def pieces(A, B, ops, coef):
        # The backward of the product with unit upstream gradients, scaled.
        e = Expr(A, B, metric, gamma=gamma, ops=ops)
        r = backward(e, "matmul", np.ones((A.shape[0], 1), e.np_dtype), np.ones((B.shape[0], 1), e.np_dtype))
        c = e.real(coef)
        return (r["dX"][0] * c, r["dX"][1] * abs(c)), (r["dY"][0] * c, r["dY"][1] * abs(c))

    def within(A, k):
        if unbiased:
            c = g / (k * (k - 1))
            parts = pieces(A, A, [("band", (-1, 10 ** 9))], c) + pieces(A, A, [("band", (10 ** 9, -1))], c)
        else:
            parts = pieces(A, A, [], g / (k * k))
        return sum(p[0] for p in parts), sum(p[1] for p in parts)

    wx, wxm = within(X, n)
    wy, wym = within(Y, m)
    cx_, cy_ = pieces(X, Y, [], -2.0 * g / (n * m))
    return (wx + cx_[0], wxm + cx_[1]), (wy + cy_[0], wym + cy_[1])
