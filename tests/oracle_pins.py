"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each pin is a plain function that raises AssertionError on a mismatch. They
are collected as tests by test_oracle_pins.py and also run against oracle
builds with planted mistakes by test_oracle_mutants.py, which requires every
planted mistake to trip at least one pin.

Independent references used here: hand-derived closed forms
(tests/golden/closed_forms.json), torch float64 library routines on dense
tiny inputs (cdist, matmul, logsumexp, softmax, stable sort, argmin,
autograd), exact integer arithmetic, and identities of the definitions.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.json")
_MATH = {"exp": math.exp, "log": math.log, "abs": abs, "__builtins__": {}}
DTYPES = (np.float32, np.float64)


def _golden():
    with open(GOLDEN) as f:
        return {c["name"]: c for c in json.load(f)["cases"]}


def _ev(expr):
    return eval(expr, _MATH)  # expressions from the fixture: exp/log over literals only


def _close(a, b, rtol=1e-13, atol=1e-13, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, "%s: shape %s vs %s" % (what, a.shape, b.shape)
    ok = np.abs(a - b) <= atol + rtol * np.abs(b)
    assert ok.all(), "%s: max abs diff %g" % (what, np.max(np.abs(a - b)))


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- dense refs
def dense_scores_torch(X, Y, metric, gamma=1.0, ops=()):
    """Dense [N,M] scores in torch float64 from library routines."""
    Xt = torch.as_tensor(np.asarray(X, np.float64))
    Yt = torch.as_tensor(np.asarray(Y, np.float64))
    if metric == "linear":
        S = Xt @ Yt.T
    elif metric == "cosine_distances":
        S = 1 - torch.nn.functional.cosine_similarity(Xt[:, None, :], Yt[None, :, :], dim=-1, eps=1e-300)
    else:
        S = torch.cdist(Xt, Yt, compute_mode="donot_use_mm_for_euclid_dist") ** 2
        if metric == "rbf":
            S = torch.exp(-gamma * S)
    for name, arg in ops:
        if name == "mul":
            S = S * arg
        elif name == "add":
            S = S + arg
        elif name == "add_rows":
            S = S + torch.as_tensor(np.asarray(arg, np.float64))[:, None]
        elif name == "add_columns":
            S = S + torch.as_tensor(np.asarray(arg, np.float64))[None, :]
        elif name == "weight_rows":
            S = S * torch.as_tensor(np.asarray(arg, np.float64))[:, None]
        elif name == "weight_columns":
            S = S * torch.as_tensor(np.asarray(arg, np.float64))[None, :]
        elif name == "exp":
            S = torch.exp(S)
    return S


def _inputs(seed, n, m, d, dtype, scale=1.0):
    r = _rng(seed)
    X = (scale * r.standard_normal((n, d))).astype(dtype)
    Y = (scale * r.standard_normal((m, d))).astype(dtype)
    return X, Y


# ---------------------------------------------------------------- metric pins
def pin_metric_closed_forms():
    """Hand closed forms: x=(1,2), y=(3,5) (fixture metric_values)."""
    c = _golden()["metric_values"]
    for dt in DTYPES:
        X = np.array(c["X"], dt)
        Y = np.array(c["Y"], dt)
        for metric, exp_rows in c["expect"].items():
            out, _ = oracle.scores(oracle.Expr(X, Y, metric, gamma=c["gamma"]))
            want = [[_ev(v) for v in row] for row in exp_rows]
            _close(out, want, what="metric %s %s" % (metric, dt.__name__))


def pin_grid_distances():
    c = _golden()["grid_distances"]
    for dt in DTYPES:
        X = np.array(c["X"], dt)
        Y = np.array(c["Y"], dt)
        out, _ = oracle.scores(oracle.Expr(X, Y, "sqeuclidean"))
        want = [[_ev(v) for v in row] for row in c["expect"]["sqeuclidean"]]
        _close(out, want, rtol=0, atol=0, what="grid distances")


def pin_rbf_self_is_one():
    """rbf(x, x) = 1 exactly, for any x and gamma."""
    for dt in DTYPES:
        X, _ = _inputs(1, 13, 1, 7, dt, scale=3.0)
        out, _ = oracle.scores(oracle.Expr(X, X, "rbf", gamma=0.37))
        d = np.diag(np.asarray(out, np.float64))
        assert np.all(d == 1.0), "rbf(x,x) != 1"


def pin_metric_symmetry():
    """f(x, y) = f(y, x) for all four metrics."""
    for dt in DTYPES:
        X, Y = _inputs(2, 9, 11, 5, dt)
        for metric in ("linear", "sqeuclidean", "rbf", "cosine_distances"):
            a, _ = oracle.scores(oracle.Expr(X, Y, metric, gamma=0.3))
            b, _ = oracle.scores(oracle.Expr(Y, X, metric, gamma=0.3))
            _close(a, np.asarray(b).T, what="symmetry %s" % metric)


def pin_cosine_special_cases():
    """cosine distance: 0 for parallel, 1 for orthogonal or zero, 2 for
    antipodal vectors; unchanged by positive scaling of either side."""
    for dt in DTYPES:
        X = np.array([[1, 2, 2], [0, 0, 0], [3, 0, 0]], dt)
        Y = np.array([[2, 4, 4], [-1, -2, -2], [0, 5, 0]], dt)
        out, _ = oracle.scores(oracle.Expr(X, Y, "cosine_distances"))
        want = [[0, 2, 1 - 2 / 3.0], [1, 1, 1], [1 - 1 / 3.0, 1 + 1 / 3.0, 1]]
        _close(out, want, rtol=1e-14, atol=1e-14, what="cosine special cases")
        X2, Y2 = _inputs(4, 6, 8, 5, dt)
        a, _ = oracle.scores(oracle.Expr(X2, Y2, "cosine_distances"))
        b, _ = oracle.scores(oracle.Expr((4 * X2).astype(dt), (0.5 * Y2).astype(dt), "cosine_distances"))
        _close(a, b, rtol=1e-12, atol=1e-13, what="cosine scale invariance")


def pin_translation_invariance():
    """sqeuclidean and rbf are unchanged by a common shift (exact on integers)."""
    r = _rng(3)
    for dt in DTYPES:
        X = r.integers(-5, 6, (7, 4)).astype(dt)
        Y = r.integers(-5, 6, (8, 4)).astype(dt)
        t = np.array([3, -2, 7, 1], dt)
        for metric in ("sqeuclidean", "rbf"):
            a, _ = oracle.scores(oracle.Expr(X, Y, metric, gamma=0.25))
            b, _ = oracle.scores(oracle.Expr(X + t, Y + t, metric, gamma=0.25))
            _close(a, b, rtol=0, atol=0, what="translation %s" % metric)


def pin_metrics_vs_dense():
    """All metrics against torch float64 matmul / cdist / cosine_similarity on small random inputs."""
    for dt in DTYPES:
        for d in (1, 3, 16, 33, 64):
            X, Y = _inputs(10 + d, 7, 9, d, dt)
            for metric in ("linear", "sqeuclidean", "rbf", "cosine_distances"):
                out, mag = oracle.scores(oracle.Expr(X, Y, metric, gamma=0.05))
                ref = dense_scores_torch(X, Y, metric, 0.05).numpy()
                _close(out, ref, rtol=1e-12, atol=1e-12, what="dense %s D=%d" % (metric, d))
                assert np.all(np.asarray(mag, np.float64) >= np.abs(np.asarray(out, np.float64)) - 1e-12)


# ---------------------------------------------------------------- op chain pins
def pin_ops_each_vs_dense():
    """Every score op, alone and in sequence, against dense torch float64."""
    for dt in DTYPES:
        X, Y = _inputs(20, 6, 8, 4, dt)
        r = _rng(21)
        a = r.standard_normal(6).astype(dt)
        b = r.standard_normal(8).astype(dt)
        w = r.standard_normal(6).astype(dt)
        u = r.standard_normal(8).astype(dt)
        chains = [
            [("mul", 0.5)], [("add", 1.25)], [("add_rows", a)], [("add_columns", b)],
            [("weight_rows", w)], [("weight_columns", u)], [("mul", 0.1), ("exp", None)],
            [("mul", 2.0), ("add", 1.0)], [("add", 1.0), ("mul", 2.0)],
            [("add_rows", a), ("weight_columns", u)], [("weight_columns", u), ("add_rows", a)],
            [("mul", -0.5), ("add_rows", a), ("add_columns", b), ("exp", None), ("weight_rows", w)],
        ]
        for ops in chains:
            for metric in ("linear", "sqeuclidean"):
                out, _ = oracle.scores(oracle.Expr(X, Y, metric, ops=ops))
                ref = dense_scores_torch(X, Y, metric, 1.0, ops).numpy()
                _close(out, ref, rtol=1e-12, atol=1e-12,
                       what="ops %s %s" % ([o[0] for o in ops], metric))


def pin_op_order_matters():
    """Left-to-right application: (s*2)+1 differs from (s+1)*2 by exactly 1."""
    X, Y = _inputs(22, 3, 4, 2, np.float64)
    a, _ = oracle.scores(oracle.Expr(X, Y, "linear", ops=[("mul", 2.0), ("add", 1.0)]))
    b, _ = oracle.scores(oracle.Expr(X, Y, "linear", ops=[("add", 1.0), ("mul", 2.0)]))
    _close(np.asarray(b, np.float64) - np.asarray(a, np.float64), np.ones((3, 4)), what="op order")


# ---------------------------------------------------------------- matmul pins
def pin_matmul_golden():
    c = _golden()["grid_kernel_product"]
    for dt in DTYPES:
        e = oracle.Expr(np.array(c["X"], dt), np.array(c["Y"], dt), c["metric"], gamma=c["gamma"])
        out, _ = oracle.matmul(e, np.array(c["V"], dt))
        _close(out, [[_ev(v) for v in row] for row in c["expect"]], what="kernel product golden")


def pin_matmul_vs_dense():
    for dt in DTYPES:
        X, Y = _inputs(30, 9, 13, 5, dt)
        V = _rng(31).standard_normal((13, 6)).astype(dt)
        for metric in ("linear", "sqeuclidean", "rbf"):
            ops = [("mul", 0.3), ("add_columns", _rng(32).standard_normal(13).astype(dt))]
            out, mag = oracle.matmul(oracle.Expr(X, Y, metric, gamma=0.2, ops=ops), V)
            S = dense_scores_torch(X, Y, metric, 0.2, ops)
            ref = (S @ torch.as_tensor(V.astype(np.float64))).numpy()
            _close(out, ref, rtol=1e-12, atol=1e-12, what="matmul %s" % metric)


def pin_matmul_exact_integers():
    """Integer inputs, linear metric: the product is exact."""
    r = _rng(33)
    for dt in DTYPES:
        X = r.integers(-9, 10, (5, 3)).astype(dt)
        Y = r.integers(-9, 10, (7, 3)).astype(dt)
        V = r.integers(-9, 10, (7, 4)).astype(dt)
        out, _ = oracle.matmul(oracle.Expr(X, Y, "linear"), V)
        ref = X.astype(np.int64) @ Y.astype(np.int64).T @ V.astype(np.int64)
        assert np.array_equal(np.asarray(out, np.float64), ref.astype(np.float64)), "integer product"


def pin_row_mass_isolated_points():
    """Ones column = row mass; for points 100 apart (gamma 1) only the self pair
    survives, so the mass is exactly 1 and the product returns V_i."""
    for dt in DTYPES:
        X = (100.0 * np.arange(6, dtype=np.float64)[:, None] * np.array([[1.0, 0.5]])).astype(dt)
        V = np.concatenate([_rng(34).standard_normal((6, 2)), np.ones((6, 1))], 1).astype(dt)
        out, _ = oracle.matmul(oracle.Expr(X, X, "rbf", gamma=1.0), V)
        _close(out, V.astype(np.float64), rtol=0, atol=0, what="isolated row mass")


# ---------------------------------------------------------------- displacement pins
def pin_displacement_golden():
    c = _golden()["grid_displacement"]
    for dt in DTYPES:
        e = oracle.Expr(np.array(c["X"], dt), np.array(c["Y"], dt), c["metric"], gamma=c["gamma"])
        out, _ = oracle.displacement(e)
        _close(out, [[_ev(v) for v in row] for row in c["expect"]], what="displacement golden")


def pin_displacement_autograd():
    """For rbf, d/dx_i sum_j k(x_i, y_j) = 2 gamma sum_j k_ij (y_j - x_i)."""
    for dt in DTYPES:
        X, Y = _inputs(40, 6, 9, 3, dt)
        g = 0.7
        out, _ = oracle.displacement(oracle.Expr(X, Y, "rbf", gamma=g))
        Xt = torch.tensor(X.astype(np.float64), requires_grad=True)
        Yt = torch.tensor(Y.astype(np.float64))
        K = torch.exp(-g * ((Xt[:, None, :] - Yt[None, :, :]) ** 2).sum(-1))
        (grad,) = torch.autograd.grad(K.sum(), Xt)
        _close(out, grad.numpy() / (2 * g), rtol=1e-12, atol=1e-12, what="displacement autograd")


def pin_displacement_identity():
    """disp = S@Y - x_i * (S@1), via the oracle's own product on any expression."""
    for dt in DTYPES:
        X, Y = _inputs(41, 7, 10, 4, dt)
        e = oracle.Expr(X, Y, "sqeuclidean", ops=[("mul", -0.1), ("exp", None)])
        disp, _ = oracle.displacement(e)
        V = np.concatenate([Y, np.ones((10, 1), dt)], 1)
        prod, _ = oracle.matmul(e, V)
        prod = np.asarray(prod, np.float64)
        ref = prod[:, :4] - X.astype(np.float64) * prod[:, 4:5]
        _close(disp, ref, rtol=1e-11, atol=1e-11, what="displacement identity")


# ---------------------------------------------------------------- SVGD pin
def pin_svgd_autograd():
    """SVGD direction against the dense autograd form of the SVGD section:
    phi(x_i) = 1/n sum_j [k(x_j,x_i) grad log p(x_j) + grad_{x_j} k(x_j,x_i)]."""
    r = _rng(50)
    n, d, g = 12, 3, 1.0 / 16.0
    x = r.standard_normal((n, d))
    score = -x
    phi, _ = oracle.svgd_direction(x, score, g)
    xt = torch.tensor(x)
    xj = xt.clone().requires_grad_(True)
    K = torch.exp(-g * ((xj[:, None, :] - xt[None, :, :]) ** 2).sum(-1))  # K[j, i] = k(x_j, x_i)
    rep = torch.zeros(n, d, dtype=torch.float64)
    for i in range(n):
        (gi,) = torch.autograd.grad(K[:, i].sum(), xj, retain_graph=True)
        rep[i] = gi.sum(0)  # row j of gi is grad_{x_j} k(x_j, x_i)
    drive = K.detach().T @ torch.tensor(score)
    ref = (drive + rep) / n
    _close(phi, ref.numpy(), rtol=1e-12, atol=1e-12, what="svgd autograd")


# ---------------------------------------------------------------- logsumexp pins
def pin_lse_golden():
    c = _golden()["grid_logsumexp"]
    for dt in DTYPES:
        e = oracle.Expr(np.array(c["X"], dt), np.array(c["Y"], dt), c["metric"], ops=c["ops"])
        out, _ = oracle.logsumexp(e)
        _close(out, [_ev(v) for v in c["expect_logsumexp"]], what="lse golden")
        out, _ = oracle.logsumexp(e, exclude_self=True)
        _close(out, [_ev(v) for v in c["expect_logsumexp_exclude_self"]], what="lse golden exclude")


def pin_lse_equal_scores():
    """M equal scores s: lse = s + log M; excluding self, s + log(M - 1)."""
    for dt in DTYPES:
        M = 37
        X = np.full((5, 2), 0.5, dt)
        Y = np.tile(np.array([[1.0, 2.0]], dt), (M, 1))
        s = 0.5 * 1.0 + 0.5 * 2.0
        out, _ = oracle.logsumexp(oracle.Expr(X, Y, "linear"))
        _close(out, np.full(5, s + math.log(M)), what="lse equal")
        out, _ = oracle.logsumexp(oracle.Expr(X, Y, "linear"), exclude_self=True)
        _close(out, np.full(5, s + math.log(M - 1)), what="lse equal exclude")


def pin_lse_fully_excluded():
    """A row whose only pair is excluded has lse = -inf."""
    X = np.array([[1.0, 2.0]], np.float32)
    out, _ = oracle.logsumexp(oracle.Expr(X, X, "linear"), exclude_self=True)
    assert np.isneginf(np.asarray(out, np.float64)).all()


def pin_lse_vs_torch():
    for dt in DTYPES:
        X, Y = _inputs(60, 8, 8, 6, dt)
        b = _rng(61).standard_normal(8).astype(dt)
        ops = [("mul", 1.0 / 0.07), ("add_rows", b)]
        e = oracle.Expr(X, Y, "linear", ops=ops)
        S = dense_scores_torch(X, Y, "linear", 1.0, ops)
        out, _ = oracle.logsumexp(e)
        _close(out, torch.logsumexp(S, -1).numpy(), rtol=1e-12, what="lse torch")
        Sm = S.clone()
        Sm.fill_diagonal_(-float("inf"))
        out, _ = oracle.logsumexp(e, exclude_self=True)
        _close(out, torch.logsumexp(Sm, -1).numpy(), rtol=1e-12, what="lse torch exclude")


def pin_lse_row_shift():
    """lse(s + b_i) = b_i + lse(s)."""
    X, Y = _inputs(62, 6, 9, 3, np.float64)
    b = _rng(63).standard_normal(6)
    a, _ = oracle.logsumexp(oracle.Expr(X, Y, "sqeuclidean", ops=[("mul", -0.5)]))
    c, _ = oracle.logsumexp(oracle.Expr(X, Y, "sqeuclidean", ops=[("mul", -0.5), ("add_rows", b)]))
    _close(np.asarray(c, np.float64), np.asarray(a, np.float64) + b, rtol=1e-13, what="lse shift")


# ---------------------------------------------------------------- softmax pins
def pin_softmax_golden():
    c = _golden()["grid_softmax_matmul"]
    for dt in DTYPES:
        e = oracle.Expr(np.array(c["X"], dt), np.array(c["Y"], dt), c["metric"], ops=c["ops"])
        out, _ = oracle.softmax_matmul(e, np.array(c["V"], dt))
        _close(out, [[_ev(v) for v in row] for row in c["expect"]], what="softmax golden")


def pin_softmax_rows_sum_to_one():
    """V = ones gives 1; V = [V, 1] has last column 1."""
    for dt in DTYPES:
        X, Y = _inputs(70, 6, 11, 8, dt, scale=2.0)
        V = np.concatenate([_rng(71).standard_normal((11, 3)), np.ones((11, 1))], 1).astype(dt)
        out, _ = oracle.softmax_matmul(oracle.Expr(X, Y, "linear", ops=[("mul", 0.5)]), V)
        _close(np.asarray(out, np.float64)[:, -1], np.ones(6), what="softmax rows sum")


def pin_softmax_vs_torch():
    for dt in DTYPES:
        X, Y = _inputs(72, 7, 10, 5, dt)
        V = _rng(73).standard_normal((10, 4)).astype(dt)
        ops = [("mul", 1.0 / math.sqrt(5.0))]
        out, _ = oracle.softmax_matmul(oracle.Expr(X, Y, "linear", ops=ops), V)
        S = dense_scores_torch(X, Y, "linear", 1.0, ops)
        ref = torch.softmax(S, -1) @ torch.as_tensor(V.astype(np.float64))
        _close(out, ref.numpy(), rtol=1e-12, atol=1e-13, what="softmax torch")


def pin_softmax_add_rows_invariant():
    X, Y = _inputs(74, 5, 9, 3, np.float64)
    V = _rng(75).standard_normal((9, 2))
    b = 10 * _rng(76).standard_normal(5)
    a, _ = oracle.softmax_matmul(oracle.Expr(X, Y, "linear"), V)
    c, _ = oracle.softmax_matmul(oracle.Expr(X, Y, "linear", ops=[("add_rows", b)]), V)
    _close(a, c, rtol=1e-13, atol=1e-14, what="softmax add_rows invariance")


def pin_softmax_hard_limit():
    """A large scale turns softmax into the row argmax: the output is V[argmax]."""
    X, Y = _inputs(77, 6, 12, 4, np.float64)
    V = _rng(78).standard_normal((12, 3))
    out, _ = oracle.softmax_matmul(oracle.Expr(X, Y, "linear", ops=[("mul", 1e4)]), V)
    am = np.argmax(X @ Y.T, axis=1)
    _close(out, V[am], rtol=1e-9, atol=1e-9, what="softmax hard limit")


# ---------------------------------------------------------------- top-k pins
def pin_topk_golden():
    c = _golden()["grid_distances"]
    for dt in DTYPES:
        e = oracle.Expr(np.array(c["X"], dt), np.array(c["Y"], dt), "sqeuclidean")
        v, i, _ = oracle.topk(e, 3)
        assert np.array_equal(i, c["topk_smallest_3"]["indices"]), i
        _close(v, c["topk_smallest_3"]["values"], rtol=0, atol=0, what="topk golden values")
        v, i, _ = oracle.topk(e, 3, largest=True)
        assert np.array_equal(i, c["topk_largest_3"]["indices"]), i
        _close(v, c["topk_largest_3"]["values"], rtol=0, atol=0, what="topk largest golden")
        v, i, _ = oracle.topk(e, 1)
        assert np.array_equal(i[:, 0], c["min"]["indices"])
        _close(v[:, 0], c["min"]["values"], rtol=0, atol=0, what="min golden")


def _stable_ref(S, k, largest):
    key = -S if largest else S
    vals, idx = torch.sort(key, dim=-1, stable=True)
    return idx[:, :k].numpy()


def pin_topk_vs_stable_sort():
    """Integer grids (many exact ties) and duplicated rows: indices equal a
    stable sort's, lowest index first among equal values, both directions."""
    r = _rng(80)
    for dt in DTYPES:
        X = r.integers(-2, 3, (9, 2)).astype(dt)
        Y = r.integers(-2, 3, (23, 2)).astype(dt)
        Y[7] = Y[3]
        Y[15] = Y[3]
        S = dense_scores_torch(X, Y, "sqeuclidean")
        for k in (1, 5, 23):
            for largest in (False, True):
                v, i, _ = oracle.topk(oracle.Expr(X, Y, "sqeuclidean"), k, largest=largest)
                assert np.array_equal(i, _stable_ref(S, k, largest)), (k, largest)
                _close(v, torch.gather(S, 1, torch.as_tensor(i)).numpy(), rtol=1e-14, atol=0, what="topk vals")


def pin_topk_argmin():
    """k = 1 equals argmin (first occurrence), on random inputs."""
    for dt in DTYPES:
        X, Y = _inputs(81, 10, 30, 4, dt)
        _, i, _ = oracle.topk(oracle.Expr(X, Y, "sqeuclidean"), 1)
        S = dense_scores_torch(X, Y, "sqeuclidean")
        assert np.array_equal(i[:, 0], torch.argmin(S, -1).numpy())


def pin_topk_extra_positions():
    """Positions past M are padded with NaN / -1."""
    X, Y = _inputs(82, 2, 3, 2, np.float32)
    v, i, _ = oracle.topk(oracle.Expr(X, Y, "linear"), 3, extra=2)
    assert np.all(i[:, 3:] == -1) and np.all(np.isnan(np.asarray(v, np.float64)[:, 3:]))
    assert sorted(i[0, :3].tolist()) == [0, 1, 2]


# ---------------------------------------------------------------- row subsets
def pin_row_subset_matches_full():
    X, Y = _inputs(90, 17, 12, 3, np.float32)
    V = _rng(91).standard_normal((12, 2)).astype(np.float32)
    e = oracle.Expr(X, Y, "rbf", gamma=0.3)
    full, _ = oracle.matmul(e, V)
    rows = np.array([16, 0, 5])
    part, _ = oracle.matmul(e, V, rows=rows)
    _close(part, np.asarray(full)[rows], rtol=0, atol=0, what="row subset")
    lf, _ = oracle.logsumexp(e, exclude_self=True)
    lp, _ = oracle.logsumexp(e, exclude_self=True, rows=rows)
    _close(lp, np.asarray(lf)[rows], rtol=0, atol=0, what="row subset lse")


# ---------------------------------------------------------------- masks
# A mask drops pairs from the reduction (Score Expressions: boolean row and
# column masks; Task Map, Attention row: causal, band, same_group). The pins
# derive each masked result from unmasked oracle calls on the surviving
# columns, or from torch's own triangular routines, never from the mask
# predicate itself.

def _consumers(e, V, rows=None):
    """Every consumer's result on expression e (top-k: 3 smallest, 2 extra)."""
    return {
        "matmul": np.asarray(oracle.matmul(e, V, rows)[0], np.float64),
        "displacement": np.asarray(oracle.displacement(e, rows)[0], np.float64),
        "logsumexp": np.asarray(oracle.logsumexp(e, rows=rows)[0], np.float64),
        "softmax_matmul": np.asarray(oracle.softmax_matmul(e, V, rows)[0], np.float64),
        "topk": oracle.topk(e, 3, extra=2, rows=rows),
    }


def _check_row_against_subset(got, i, ref, cols):
    """Row i of a masked result equals the unmasked result over the kept
    columns `cols` (ref evaluated on Y[cols], V[cols]); top-k indices map
    back through cols."""
    for name in ("matmul", "displacement", "logsumexp", "softmax_matmul"):
        _close(got[name][i], ref[name][0], rtol=1e-12, atol=1e-12, what="%s row %d" % (name, i))
    gv, gi, _ = got["topk"]
    rv, ri, _ = ref["topk"]
    mapped = np.where(ri[0] >= 0, np.asarray(cols)[np.maximum(ri[0], 0)], -1)
    assert np.array_equal(gi[i], mapped), ("topk row", i, gi[i], mapped)
    _close(np.nan_to_num(np.asarray(gv[i], np.float64), nan=7.0), np.nan_to_num(np.asarray(rv[0], np.float64), nan=7.0),
           rtol=1e-14, atol=0, what="topk values row %d" % i)


def _subset_ref(X, Y, V, metric, gamma, ops, i, cols):
    e = oracle.Expr(X[i:i + 1], Y[cols], metric, gamma=gamma, ops=ops)
    return _consumers(e, V[cols])


def pin_mask_columns_is_column_subset():
    """A column mask equals evaluating on the kept columns only."""
    for dt in DTYPES:
        X, Y = _inputs(100, 6, 11, 3, dt)
        V = _rng(101).standard_normal((11, 2)).astype(dt)
        keep = np.array([1, 0, 1, 1, 0, 0, 1, 1, 0, 1, 1], bool)
        cols = np.nonzero(keep)[0]
        got = _consumers(oracle.Expr(X, Y, "rbf", 0.4, [("mask_columns", keep)]), V)
        for i in range(6):
            _check_row_against_subset(got, i, _subset_ref(X, Y, V, "rbf", 0.4, [], i, cols), cols)


def pin_mask_rows_empty_rows():
    """A row mask leaves kept rows unchanged and gives masked rows the
    empty-row results: zero sums, -inf log-sum-exp, zero softmax product and
    top-k positions NaN / -1."""
    X, Y = _inputs(102, 5, 7, 2, np.float64)
    V = _rng(103).standard_normal((7, 2))
    keep = np.array([1, 0, 1, 0, 1], bool)
    ops = [("mul", -1.0)]
    got = _consumers(oracle.Expr(X, Y, "sqeuclidean", ops=ops + [("mask_rows", keep)]), V)
    ref = _consumers(oracle.Expr(X, Y, "sqeuclidean", ops=ops), V)
    for i in range(5):
        if keep[i]:
            for name in ("matmul", "displacement", "logsumexp", "softmax_matmul"):
                _close(got[name][i], ref[name][i], rtol=0, atol=0, what=name)
            assert np.array_equal(got["topk"][1][i], ref["topk"][1][i])
        else:
            assert np.all(got["matmul"][i] == 0) and np.all(got["displacement"][i] == 0)
            assert np.all(got["softmax_matmul"][i] == 0) and np.isneginf(got["logsumexp"][i])
            assert np.all(got["topk"][1][i] == -1) and np.all(np.isnan(np.asarray(got["topk"][0][i], np.float64)))


def pin_causal_is_prefix():
    """causal(d): row i reduces over the prefix of columns j <= i + d
    (the rows whose prefix is empty get the empty-row results)."""
    X, Y = _inputs(104, 9, 9, 3, np.float32)
    V = _rng(105).standard_normal((9, 3)).astype(np.float32)
    for d in (0, 2, -3):
        got = _consumers(oracle.Expr(X, Y, "linear", ops=[("mul", 0.5), ("causal", d)]), V)
        for i in range(9):
            cols = np.arange(0, min(9, i + d + 1))
            if cols.size == 0:
                assert np.isneginf(got["logsumexp"][i]) and np.all(got["topk"][1][i] == -1)
                continue
            _check_row_against_subset(got, i, _subset_ref(X, Y, V, "linear", 1.0, [("mul", 0.5)], i, cols), cols)


def pin_band_is_window():
    """band(lo, hi): row i reduces over the window i - lo <= j <= i + hi."""
    X, Y = _inputs(106, 8, 12, 2, np.float64)
    V = _rng(107).standard_normal((12, 2))
    for lo, hi in ((1, 2), (0, 0), (3, -1)):
        got = _consumers(oracle.Expr(X, Y, "sqeuclidean", ops=[("band", (lo, hi)), ("mul", -1.0)]), V)
        for i in range(8):
            cols = np.arange(max(0, i - lo), min(12, i + hi + 1))
            if cols.size == 0:
                continue
            _check_row_against_subset(got, i, _subset_ref(X, Y, V, "sqeuclidean", 1.0, [("mul", -1.0)], i, cols),
                                      cols)


def pin_same_group_is_block():
    """same_group: row i reduces over the columns of its own group."""
    X, Y = _inputs(108, 10, 13, 3, np.float32)
    V = _rng(109).standard_normal((13, 2)).astype(np.float32)
    gr = np.array([0, 2, 1, 0, 5, 2, 2, 1, 0, 3])
    gc = np.array([1, 0, 0, 2, 1, 2, 0, 4, 2, 1, 0, 3, 3])
    got = _consumers(oracle.Expr(X, Y, "rbf", 0.2, [("same_group", (gr, gc))]), V)
    for i in range(10):
        cols = np.nonzero(gc == gr[i])[0]
        if cols.size == 0:
            assert np.all(got["matmul"][i] == 0) and np.isneginf(got["logsumexp"][i])
            continue
        _check_row_against_subset(got, i, _subset_ref(X, Y, V, "rbf", 0.2, [], i, cols), cols)


def pin_masks_vs_torch_triangles():
    """causal and band against torch.tril / torch.triu applied to dense
    scores: masked log-sum-exp and softmax(S)@V, several masks combined."""
    X, Y = _inputs(110, 12, 10, 4, np.float64)
    V = _rng(111).standard_normal((10, 3))
    S = dense_scores_torch(X, Y, "linear", ops=[("mul", 0.3)])
    ones = torch.ones(12, 10, dtype=torch.bool)
    rows = torch.as_tensor(np.array([1, 1, 0, 1, 1, 1, 1, 1, 1, 1, 1, 1], bool))
    for masks, K in (
            ([("causal", 0)], ones.tril(0)),
            ([("causal", 1), ("band", (2, 5))], ones.tril(1) & ones.triu(-2)),
            ([("band", (4, 1)), ("mask_rows", rows.numpy())], ones.tril(1) & ones.triu(-4) & rows[:, None])):
        e = oracle.Expr(X, Y, "linear", ops=[("mul", 0.3)] + masks)
        Sm = S.masked_fill(~K, float("-inf"))
        got, want = np.asarray(oracle.logsumexp(e)[0], np.float64), torch.logsumexp(Sm, -1).numpy()
        assert np.array_equal(np.isneginf(got), np.isneginf(want))
        fin = np.isfinite(want)
        _close(got[fin], want[fin], rtol=1e-13, atol=1e-13, what="lse")
        P = torch.softmax(Sm, -1).nan_to_num(0.0)
        _close(oracle.softmax_matmul(e, V)[0], (P @ torch.as_tensor(V)).numpy(), rtol=1e-12, atol=1e-13, what="smx")
        _close(oracle.matmul(e, V)[0], ((S * K) @ torch.as_tensor(V)).numpy(), rtol=1e-12, atol=1e-13, what="mm")


# ---------------------------------------------------------------- solve
def pin_solve_two_points_closed_form():
    """Two points at distance 1, rbf gamma: K + aI = [[1+a, e], [e, 1+a]]
    with e = exp(-gamma); its inverse applied to b = (1, 2) is written out
    from the 2x2 inverse formula."""
    g, a = 0.7, 0.25
    X = np.array([[0.0], [1.0]])
    A, cond = oracle.solve(oracle.Expr(X, X, "rbf", gamma=g), a, np.array([[1.0], [2.0]]))
    e, d = math.exp(-g), 1 + a
    det = d * d - e * e
    want = np.array([[(d * 1 - e * 2) / det], [(-e * 1 + d * 2) / det]])
    _close(A, want, rtol=1e-14, atol=1e-15, what="2x2 solve")
    assert abs(cond - (d + e) / (d - e)) < 1e-12 * cond


def pin_solve_shift_only():
    """With X far apart (rbf ~ identity), (K + aI) A = B gives A = B / (1 + a)."""
    X = (100.0 * np.arange(5, dtype=np.float64))[:, None]
    B = _rng(120).standard_normal((5, 3))
    A, _ = oracle.solve(oracle.Expr(X, X, "rbf", gamma=1.0), 3.0, B)
    _close(A, B / 4.0, rtol=1e-14, atol=1e-15, what="shift only")


# ---------------------------------------------------------------- MMD
def pin_mmd_two_points_closed_form():
    """Two one-point-apart clouds with a hand-derived statistic (fixture
    mmd_two_points), unbiased and biased."""
    c = _golden()["mmd_two_points"]
    X, Y = np.array(c["X"]), np.array(c["Y"])
    v, _ = oracle.mmd2(X, Y, "rbf", c["gamma"], unbiased=True)
    _close(v, _ev(c["expect_unbiased"]), rtol=1e-14, atol=1e-15, what="mmd unbiased")
    v, _ = oracle.mmd2(X, Y, "rbf", c["gamma"], unbiased=False)
    _close(v, _ev(c["expect_biased"]), rtol=1e-14, atol=1e-15, what="mmd biased")


def pin_mmd_linear_kernel_means():
    """With the linear kernel the sums reduce to vector sums:
    sum_{i != i'} x_i.x_i' = |sum x|^2 - sum |x_i|^2, sum_{i,j} x_i.y_j =
    (sum x).(sum y); the biased statistic is |mean x - mean y|^2."""
    r = _rng(130)
    X, Y = r.standard_normal((7, 3)), r.standard_normal((5, 3))
    sx, sy = X.sum(0), Y.sum(0)
    n, m = 7, 5
    want_u = ((sx @ sx - (X * X).sum()) / (n * (n - 1)) + (sy @ sy - (Y * Y).sum()) / (m * (m - 1))
              - 2 * (sx @ sy) / (n * m))
    v, _ = oracle.mmd2(X, Y, "linear", unbiased=True)
    _close(v, want_u, rtol=1e-12, atol=1e-14, what="linear mmd unbiased")
    dm = X.mean(0) - Y.mean(0)
    v, _ = oracle.mmd2(X, Y, "linear", unbiased=False)
    _close(v, dm @ dm, rtol=1e-12, atol=1e-14, what="linear mmd biased")


def pin_mmd_symmetric_and_batched():
    """MMD(X, Y) = MMD(Y, X); a batch of clouds gives each element's value,
    a cloud shared by the batch ([1, m, D]) included; the magnitude bounds
    the sum of the terms' absolute values."""
    r = _rng(131)
    X, Y = r.standard_normal((3, 6, 2)), r.standard_normal((3, 4, 2))
    for unb in (True, False):
        a, ma = oracle.mmd2(X[0], Y[0], "rbf", 0.4, unb)
        b, _ = oracle.mmd2(Y[0], X[0], "rbf", 0.4, unb)
        _close(a, b, rtol=1e-14, atol=1e-15, what="symmetry")
        assert ma >= abs(a)
        vb, _ = oracle.mmd2(X, Y, "rbf", 0.4, unb)
        for k in range(3):
            _close(vb[k], oracle.mmd2(X[k], Y[k], "rbf", 0.4, unb)[0], rtol=1e-15, atol=0, what="batch")
        vs, _ = oracle.mmd2(X, Y[:1], "rbf", 0.4, unb)
        _close(vs[2], oracle.mmd2(X[2], Y[0], "rbf", 0.4, unb)[0], rtol=1e-15, atol=0, what="shared cloud")


def _mmd2_torch(X, Y, metric, gamma, unbiased):
    """The statistic written out densely in torch float64 (squared
    distances as sums of squared differences, so that autograd is defined
    at coincident points)."""
    def k(A, B):
        if metric == "linear":
            return A @ B.T
        d2 = ((A[:, None, :] - B[None, :, :]) ** 2).sum(-1)
        return torch.exp(-gamma * d2) if metric == "rbf" else d2
    n, m = X.shape[0], Y.shape[0]
    kxx, kyy, kxy = k(X, X), k(Y, Y), k(X, Y)
    if unbiased:
        kxx = kxx * (1 - torch.eye(n, dtype=X.dtype))
        kyy = kyy * (1 - torch.eye(m, dtype=X.dtype))
        return kxx.sum() / (n * (n - 1)) + kyy.sum() / (m * (m - 1)) - 2 * kxy.sum() / (n * m)
    return kxx.sum() / (n * n) + kyy.sum() / (m * m) - 2 * kxy.sum() / (n * m)


def pin_mmd_value_and_gradient_vs_torch():
    """mmd2 and mmd2_grad against torch autograd of the dense statistic
    (float64), for the rbf, linear and squared-distance kernels, unbiased
    and biased, with a scaled upstream gradient."""
    r = _rng(132)
    X, Y = r.standard_normal((6, 3)), 0.5 + r.standard_normal((5, 3))
    for metric in ("rbf", "linear", "sqeuclidean"):
        for unb in (True, False):
            Xt = torch.tensor(X, requires_grad=True)
            Yt = torch.tensor(Y, requires_grad=True)
            v = _mmd2_torch(Xt, Yt, metric, 0.3, unb)
            gx, gy = torch.autograd.grad(1.7 * v, [Xt, Yt])
            ov, _ = oracle.mmd2(X, Y, metric, 0.3, unb)
            _close(ov, v.item(), rtol=1e-12, atol=1e-13, what="mmd %s value" % metric)
            (dx, dxm), (dy, dym) = oracle.mmd2_grad(X, Y, metric, 0.3, unb, 1.7)
            _close(dx, gx.numpy(), rtol=1e-11, atol=1e-12, what="mmd %s dX" % metric)
            _close(dy, gy.numpy(), rtol=1e-11, atol=1e-12, what="mmd %s dY" % metric)
            assert np.all(np.asarray(dxm) >= np.abs(np.asarray(dx)) * (1 - 1e-12))


def pin_mmd_gradient_batched_and_shared():
    """Batched gradients equal the per-element ones; a cloud shared by the
    batch gets the sum of the elements' gradients."""
    r = _rng(133)
    X, Y = r.standard_normal((3, 5, 2)), r.standard_normal((1, 4, 2))
    G = np.array([0.5, -1.0, 2.0])
    (dX, _), (dY, _) = oracle.mmd2_grad(X, Y, "rbf", 0.6, True, G)
    assert dX.shape == (3, 5, 2) and dY.shape == (1, 4, 2)
    want_y = 0
    for b in range(3):
        (dx, _), (dy, _) = oracle.mmd2_grad(X[b], Y[0], "rbf", 0.6, True, G[b])
        _close(dX[b], dx, rtol=1e-15, atol=0, what="batched dX")
        want_y = want_y + np.asarray(dy, np.float64)
    _close(dY[0], want_y, rtol=1e-13, atol=1e-15, what="shared dY")


# ---------------------------------------------------------------- backward
def _autograd_reference(X, Y, metric, gamma, ops, consumer, G, V=None, exclude_self=False, masks=(), indices=None):
    """Gradients of sum(out * G) by torch autograd on the dense float64
    computation: library routines only (cdist, cosine_similarity,
    logsumexp, softmax, matmul, gather)."""
    Xt = torch.tensor(np.asarray(X, np.float64), requires_grad=True)
    Yt = torch.tensor(np.asarray(Y, np.float64), requires_grad=True)
    leaves = [Xt, Yt]
    Vt = None
    if V is not None:
        Vt = torch.tensor(np.asarray(V, np.float64), requires_grad=True)
        leaves.append(Vt)
    if metric == "linear":
        S = Xt @ Yt.T
    elif metric == "cosine_distances":
        S = 1 - torch.nn.functional.cosine_similarity(Xt[:, None, :], Yt[None, :, :], dim=-1, eps=1e-300)
    else:
        diff = Xt[:, None, :] - Yt[None, :, :]
        S = (diff * diff).sum(-1)
        if metric == "rbf":
            S = torch.exp(-gamma * S)
    vec_leaves = []
    for name, arg in ops:
        if name in ("mul", "add"):
            S = S * arg if name == "mul" else S + arg
            vec_leaves.append(None)
        elif name == "exp":
            S = torch.exp(S)
            vec_leaves.append(None)
        else:
            a = torch.tensor(np.asarray(arg, np.float64), requires_grad=True)
            vec_leaves.append(a)
            if name == "add_rows":
                S = S + a[:, None]
            elif name == "add_columns":
                S = S + a[None, :]
            elif name == "weight_rows":
                S = S * a[:, None]
            else:
                S = S * a[None, :]
    N, M = S.shape
    keep = torch.ones(N, M, dtype=torch.bool)
    for name, arg in masks:
        if name == "causal":
            keep &= torch.ones(N, M, dtype=torch.bool).tril(arg)
        elif name == "mask_columns":
            keep &= torch.as_tensor(np.asarray(arg, bool))[None, :]
    if consumer == "logsumexp" and exclude_self:
        keep &= ~torch.eye(N, M, dtype=torch.bool)
    Gt = torch.as_tensor(np.asarray(G, np.float64))
    if consumer == "matmul":
        out = torch.where(keep, S, torch.zeros_like(S)) @ Vt
    elif consumer == "displacement":
        Sk = torch.where(keep, S, torch.zeros_like(S))
        out = Sk @ Yt - Sk.sum(1, keepdim=True) * Xt
    elif consumer == "logsumexp":
        out = torch.logsumexp(S.masked_fill(~keep, float("-inf")), -1)[:, None]
    elif consumer == "softmax_matmul":
        out = torch.softmax(S.masked_fill(~keep, float("-inf")), -1) @ Vt
    else:
        out = torch.gather(S, 1, torch.as_tensor(indices))
    loss = (out * Gt.reshape(out.shape)).sum()
    wanted = leaves + [a for a in vec_leaves if a is not None]
    grads = torch.autograd.grad(loss, wanted, allow_unused=True)
    res = {"dX": grads[0], "dY": grads[1]}
    if Vt is not None:
        res["dV"] = grads[2]
    it = iter(grads[len(leaves):])
    res["ops"] = [None if a is None else next(it) for a in vec_leaves]
    return res


def _compare_backward(got, ref, what, rtol=1e-10):
    def z(t):
        return np.zeros(1) if t is None else np.asarray(t.detach().numpy() if torch.is_tensor(t) else t, np.float64)
    for key in ("dX", "dY") + (("dV",) if "dV" in ref else ()):
        val, mag = got[key]
        want = z(ref[key])
        tol = rtol * (np.asarray(mag, np.float64) + np.abs(want)) + 1e-300
        assert np.all(np.abs(np.asarray(val, np.float64) - want) <= tol), (what, key, np.max(np.abs(val - want)))
    for t, (g, r) in enumerate(zip(got["ops"], ref["ops"])):
        if r is None:
            continue
        val, mag = g
        want = z(r)
        tol = rtol * (np.asarray(mag, np.float64) + np.abs(want)) + 1e-300
        assert np.all(np.abs(np.asarray(val, np.float64) - want) <= tol), (what, "op %d" % t)


def pin_backward_vs_autograd():
    """Every consumer and metric, an op chain with every vector kind and an
    exp, against torch autograd of the dense float64 computation."""
    r = _rng(130)
    N, M, D, C = 7, 9, 3, 2
    X = r.standard_normal((N, D))
    Y = r.standard_normal((M, D))
    V = r.standard_normal((M, C))
    chains = {
        "plain": [("mul", 0.7)],
        "rows_cols": [("mul", -0.5), ("add_rows", r.standard_normal(N)), ("add_columns", r.standard_normal(M)),
                      ("weight_rows", 0.5 + r.random(N)), ("weight_columns", 0.5 + r.random(M)), ("add", 0.1)],
        "exp": [("mul", -0.3), ("exp", None), ("weight_columns", r.random(M) + 0.2), ("add_rows", r.standard_normal(N))],
    }
    for metric in ("linear", "sqeuclidean", "rbf", "cosine_distances"):
        for cname, ops in chains.items():
            for consumer in ("matmul", "displacement", "logsumexp", "softmax_matmul"):
                G = r.standard_normal((N, {"matmul": C, "softmax_matmul": C, "displacement": D}.get(consumer, 1)))
                Vc = V if consumer in ("matmul", "softmax_matmul") else None
                e = oracle.Expr(X, Y, metric, gamma=0.4, ops=ops)
                got = oracle.backward(e, consumer, G, Vc)
                ref = _autograd_reference(X, Y, metric, 0.4, ops, consumer, G, Vc)
                _compare_backward(got, ref, "%s/%s/%s" % (metric, cname, consumer))


def pin_backward_masks_and_selection():
    """Masked pairs (causal, column mask), the excluded self pair, and
    top-k gradients routed through the selected pairs only."""
    r = _rng(131)
    N = M = 8
    X = r.standard_normal((N, 4))
    V = r.standard_normal((M, 3))
    keep = r.random(M) < 0.7
    for consumer in ("matmul", "logsumexp", "softmax_matmul"):
        G = r.standard_normal((N, 3 if consumer != "logsumexp" else 1))
        Vc = V if consumer != "logsumexp" else None
        masks = [("causal", 1), ("mask_columns", keep)]
        e = oracle.Expr(X, X, "linear", ops=[("mul", 0.5)] + masks)
        got = oracle.backward(e, consumer, G, Vc)
        ref = _autograd_reference(X, X, "linear", 1.0, [("mul", 0.5)], consumer, G, Vc, masks=masks)
        # X is both operands here: the torch leaves are separate copies, so
        # the gradient of X is the sum of the two sides.
        _compare_backward(got, ref, "masked %s" % consumer)
    G = r.standard_normal((N, 1))
    e = oracle.Expr(X, X, "sqeuclidean", ops=[("mul", -1.0)])
    got = oracle.backward(e, "logsumexp", G, exclude_self=True)
    ref = _autograd_reference(X, X, "sqeuclidean", 1.0, [("mul", -1.0)], "logsumexp", G, exclude_self=True)
    _compare_backward(got, ref, "exclude_self")
    v, idx, _ = oracle.topk(oracle.Expr(X, X, "sqeuclidean"), 3)
    G = r.standard_normal((N, 3))
    e = oracle.Expr(X, X, "sqeuclidean")
    got = oracle.backward(e, "topk", G, indices=idx)
    ref = _autograd_reference(X, X, "sqeuclidean", 1.0, [], "topk", G, indices=idx)
    _compare_backward(got, ref, "topk")


def pin_backward_finite_differences():
    """Central differences of the oracle's own forward (no autograd): dX
    of an rbf kernel product and of a log-sum-exp with a column bias."""
    r = _rng(132)
    X = r.standard_normal((4, 2))
    Y = r.standard_normal((5, 2))
    V = r.standard_normal((5, 2))
    G = r.standard_normal((4, 2))
    b = r.standard_normal(5)
    h = 1e-6
    for consumer, ops, Gc in (("matmul", [], G), ("logsumexp", [("mul", -0.5), ("add_columns", b)], G[:, :1])):
        got = oracle.backward(oracle.Expr(X, Y, "rbf", 0.6, ops), consumer, Gc, V if consumer == "matmul" else None)
        fd = np.zeros_like(X)
        for i in range(4):
            for d in range(2):
                vals = []
                for sgn in (1, -1):
                    Xp = X.copy()
                    Xp[i, d] += sgn * h
                    e = oracle.Expr(Xp, Y, "rbf", 0.6, ops)
                    out = oracle.matmul(e, V)[0] if consumer == "matmul" else oracle.logsumexp(e)[0][:, None]
                    vals.append(float(np.sum(np.asarray(out, np.float64) * Gc)))
                fd[i, d] = (vals[0] - vals[1]) / (2 * h)
        _close(np.asarray(got["dX"][0], np.float64), fd, rtol=1e-6, atol=1e-7, what="finite differences %s" % consumer)



# ---------------------------------------------------------------- magnitude pins
# The oracle's `mag` scales every tolerance of the comparison rule (What to
# Check, Precision). These pins compare it with values derived by hand from
# its definition (fixture entries expect_mag), for each metric, each kind of
# op and each consumer.

def _mags(got, want, what):
    _close(got, [[_ev(v) for v in row] for row in want] if isinstance(want[0], list) else [_ev(v) for v in want],
           rtol=1e-13, atol=1e-13, what=what)


def pin_mag_metric_closed_forms():
    c = _golden()["metric_values"]
    for dt in DTYPES:
        X, Y = np.array(c["X"], dt), np.array(c["Y"], dt)
        for metric, rows in c["expect_mag"].items():
            _, mag = oracle.scores(oracle.Expr(X, Y, metric, gamma=c["gamma"]))
            _mags(mag, rows, "mag metric %s %s" % (metric, dt.__name__))
    c = _golden()["grid_distances"]
    X, Y = np.array(c["X"], np.float32), np.array(c["Y"], np.float32)
    _, mag = oracle.scores(oracle.Expr(X, Y, "sqeuclidean"))
    _mags(mag, c["expect_mag"]["sqeuclidean"], "mag grid distances")


def pin_mag_op_chain_closed_forms():
    c = _golden()["op_chain_magnitudes"]
    for dt in DTYPES:
        X, Y = np.array(c["X"], dt), np.array(c["Y"], dt)
        for ch in c["chains"]:
            ops = [(n, np.array(a, dt) if isinstance(a, list) else a) for n, a in ch["ops"]]
            out, mag = oracle.scores(oracle.Expr(X, Y, c["metric"], ops=ops))
            name = "/".join(n for n, _ in ch["ops"])
            _close(out, [[_ev(ch["expect"])]], rtol=1e-13, atol=1e-13, what="chain %s" % name)
            _close(mag, [[_ev(ch["expect_mag"])]], rtol=1e-13, atol=1e-13, what="chain mag %s" % name)


def pin_mag_consumers_golden():
    g = _golden()
    for dt in DTYPES:
        c = g["grid_kernel_product"]
        e = oracle.Expr(np.array(c["X"], dt), np.array(c["Y"], dt), c["metric"], gamma=c["gamma"])
        _mags(oracle.matmul(e, np.array(c["V"], dt))[1], c["expect_mag"]["matmul"], "mag kernel product")
        c = g["grid_displacement"]
        e = oracle.Expr(np.array(c["X"], dt), np.array(c["Y"], dt), c["metric"], gamma=c["gamma"])
        _mags(oracle.displacement(e)[1], c["expect_mag"]["displacement"], "mag displacement")
        c = g["grid_logsumexp"]
        e = oracle.Expr(np.array(c["X"], dt), np.array(c["Y"], dt), c["metric"], ops=c["ops"])
        _mags(oracle.logsumexp(e)[1], c["expect_mag"]["logsumexp"], "mag logsumexp")
        _mags(oracle.logsumexp(e, exclude_self=True)[1], c["expect_mag"]["logsumexp_exclude_self"],
              "mag logsumexp exclude_self")
        c = g["grid_softmax_matmul"]
        e = oracle.Expr(np.array(c["X"], dt), np.array(c["Y"], dt), c["metric"], ops=c["ops"])
        _mags(oracle.softmax_matmul(e, np.array(c["V"], dt))[1], c["expect_mag"]["softmax_matmul"], "mag softmax")
        c = g["grid_distances"]
        e = oracle.Expr(np.array(c["X"], dt), np.array(c["Y"], dt), "sqeuclidean")
        _mags(oracle.topk(e, 3)[2], c["expect_mag"]["topk_smallest_3"], "mag topk")


# ---------------------------------------------------------------- comparison-rule pins
# The rule |g - o| <= rtol max(|o|, mag) (tests/parity.py) must accept what a
# correct float32 kernel may return -- the same sums rounded to float32 in
# other orders: blocked online softmax / log-sum-exp, the norm expansion of
# distances, a row factor applied after the sum -- and must reject the
# mistakes a tiled kernel can make: one key dropped at a split boundary, the
# self pair kept, a wrong scale, a swapped tie. Shapes are those of the
# attention, InfoNCE and Nadaraya-Watson workloads, reduced.
import parity  # noqa: E402

F32 = torch.float32


def _attention_case():
    r = _rng(500)
    Q = r.standard_normal((96, 64)).astype(np.float32)
    K = r.standard_normal((650, 64)).astype(np.float32)
    V = r.standard_normal((650, 64)).astype(np.float32)
    return Q, K, V, [("mul", 0.125)]


def _infonce_case():
    r = _rng(501)
    z = r.standard_normal((700, 64))
    z = (z / np.linalg.norm(z, axis=1, keepdims=True)).astype(np.float32)
    b = (math.sqrt(0.1) * r.standard_normal(700)).astype(np.float32)
    return z, b, [("mul", 1.0 / 0.07), ("add_rows", b)]


def _online_softmax_f32(S, V, bn=64):
    """softmax(S) @ V in float32, column blocks of bn in order, running
    (max, sum, acc) rescaled at every block."""
    n = S.shape[0]
    m = torch.full((n, 1), -float("inf"), dtype=F32)
    l = torch.zeros((n, 1), dtype=F32)
    acc = torch.zeros((n, V.shape[1]), dtype=F32)
    for j in range(0, S.shape[1], bn):
        s = S[:, j:j + bn]
        m2 = torch.maximum(m, s.max(1, keepdim=True).values)
        a = torch.exp(m - m2)
        p = torch.exp(s - m2)
        l = l * a + p.sum(1, keepdim=True)
        acc = acc * a + p @ V[j:j + bn]
        m = m2
    return acc / l, m + torch.log(l)


def pin_rule_accepts_float32_orders():
    # Attention: library softmax, and a blocked online softmax.
    Q, K, V, ops = _attention_case()
    o, mag = oracle.softmax_matmul(oracle.Expr(Q, K, "linear", ops=ops), V)
    S = (torch.from_numpy(Q) @ torch.from_numpy(K).T) * 0.125
    Vt = torch.from_numpy(V)
    for name, g in (("library", torch.softmax(S, -1) @ Vt), ("online", _online_softmax_f32(S, Vt)[0])):
        ok, ratio, _ = parity.value_report(g.numpy(), o, mag, np.float32, n_terms=650, vmax=float(np.abs(V).max()))
        assert ok, "attention %s: float32 result rejected (err/tol %.3g)" % (name, ratio)
    # InfoNCE: log-sum-exp without the self pair, library and online.
    z, b, ops = _infonce_case()
    o, mag = oracle.logsumexp(oracle.Expr(z, z, "linear", ops=ops), exclude_self=True)
    zt = torch.from_numpy(z)
    S = (zt @ zt.T) * np.float32(1.0 / 0.07) + torch.from_numpy(b)[:, None]
    S.fill_diagonal_(-float("inf"))
    ones = torch.ones((S.shape[0], 1), dtype=F32)
    for name, g in (("library", torch.logsumexp(S, -1)), ("online", _online_softmax_f32(S, ones)[1][:, 0])):
        ok, ratio, _ = parity.value_report(g.numpy(), o, mag, np.float32, n_terms=700)
        assert ok, "infonce %s: float32 result rejected (err/tol %.3g)" % (name, ratio)
    # Kernel product of rbf scores: direct distances, and the norm expansion
    # with the row factor 2^(-|x|^2) applied after the column sum.
    r = _rng(502)
    X = r.standard_normal((300, 3)).astype(np.float32)
    Y = r.standard_normal((333, 3)).astype(np.float32)
    Vk = np.concatenate([r.standard_normal((333, 3)), np.ones((333, 1))], 1).astype(np.float32)
    o, mag = oracle.matmul(oracle.Expr(X, Y, "rbf", gamma=0.5), Vk)
    Xt, Yt, Vt = torch.from_numpy(X), torch.from_numpy(Y), torch.from_numpy(Vk)
    direct = torch.exp(-0.5 * ((Xt[:, None, :] - Yt[None, :, :]) ** 2).sum(-1)) @ Vt
    sc = np.float32(math.sqrt(0.5 / math.log(2.0)))
    xs, ys = Xt * sc, Yt * sc
    t = 2 * (xs @ ys.T) - (ys * ys).sum(1)[None, :]
    expansion = (torch.exp2(t) @ Vt) * torch.exp2(-(xs * xs).sum(1))[:, None]
    for name, g in (("direct", direct), ("expansion", expansion)):
        ok, ratio, _ = parity.value_report(g.numpy(), o, mag, np.float32, n_terms=333, vmax=float(np.abs(Vk).max()))
        assert ok, "kernel product %s: float32 result rejected (err/tol %.3g)" % (name, ratio)


def _rejects(g, o, mag, n_terms, what, vmax=1.0):
    ok, ratio, _ = parity.value_report(g, o, mag, np.float32, n_terms=n_terms, vmax=vmax)
    assert not ok, "%s: the comparison rule accepts it (worst err/tol %.3g)" % (what, ratio)


def pin_rule_rejects_dropped_key():
    """The oracle's own result without one key -- the last column of a
    split, here column 64 and the last column -- fails the rule."""
    Q, K, V, ops = _attention_case()
    o, mag = oracle.softmax_matmul(oracle.Expr(Q, K, "linear", ops=ops), V)
    z, b, zops = _infonce_case()
    lo, lmag = oracle.logsumexp(oracle.Expr(z, z, "linear", ops=zops), exclude_self=True)
    r = _rng(503)
    X = r.standard_normal((200, 3)).astype(np.float32)
    Vk = np.concatenate([r.standard_normal((333, 3)), np.ones((333, 1))], 1).astype(np.float32)
    Y = r.standard_normal((333, 3)).astype(np.float32)
    mo, mmag = oracle.matmul(oracle.Expr(X, Y, "rbf", gamma=0.5), Vk)
    for drop in (64, -1):
        keep = np.ones(K.shape[0], bool)
        keep[drop] = False
        g, _ = oracle.softmax_matmul(oracle.Expr(Q, K[keep], "linear", ops=ops), V[keep])
        _rejects(g, o, mag, 650, "attention without key %d" % drop, float(np.abs(V).max()))
        keep = np.ones(z.shape[0], bool)
        keep[drop] = False
        # Column `drop` removed; the self pair of every row stays excluded.
        S = np.asarray(oracle.scores(oracle.Expr(z, z[keep], "linear", ops=zops))[0], np.float64)
        rows = np.arange(z.shape[0])
        cols = np.nonzero(keep)[0]
        S[rows[:, None] == cols[None, :]] = -np.inf
        mx = S.max(1)
        g = mx + np.log(np.exp(S - mx[:, None]).sum(1))
        _rejects(g, lo, lmag, 700, "infonce without key %d" % drop)
        keep = np.ones(Y.shape[0], bool)
        keep[drop] = False
        g, _ = oracle.matmul(oracle.Expr(X, Y[keep], "rbf", gamma=0.5), Vk[keep])
        _rejects(g, mo, mmag, 333, "kernel product without key %d" % drop, float(np.abs(Vk).max()))


def pin_rule_rejects_kept_self_pair_and_wrong_scale():
    z, b, ops = _infonce_case()
    o, mag = oracle.logsumexp(oracle.Expr(z, z, "linear", ops=ops), exclude_self=True)
    g, _ = oracle.logsumexp(oracle.Expr(z, z, "linear", ops=ops), exclude_self=False)
    _rejects(g, o, mag, 700, "infonce with the self pair kept")
    g, _ = oracle.logsumexp(oracle.Expr(z, z, "linear", ops=[("mul", 1.0 / 0.0701), ("add_rows", b)]),
                            exclude_self=True)
    _rejects(g, o, mag, 700, "infonce with temperature 0.0701")
    Q, K, V, aops = _attention_case()
    o, mag = oracle.softmax_matmul(oracle.Expr(Q, K, "linear", ops=aops), V)
    g, _ = oracle.softmax_matmul(oracle.Expr(Q, K, "linear", ops=[("mul", 0.1251)]), V)
    _rejects(g, o, mag, 650, "attention with scale 0.1251", float(np.abs(V).max()))


def pin_rule_topk_ties():
    """Top-k on a grid with exact ties: the float32 norm-expansion search
    (exact on small integers) passes, exactly and by the tolerance rule;
    swapping two tied positions, or two separated ones, fails both."""
    r = _rng(504)
    X = r.integers(-3, 4, (40, 2)).astype(np.float32)
    Y = r.integers(-3, 4, (150, 2)).astype(np.float32)
    k = 6
    ov, oi, om = oracle.topk(oracle.Expr(X, Y, "sqeuclidean"), k, extra=8)
    Xt, Yt = torch.from_numpy(X), torch.from_numpy(Y)
    d = (Xt * Xt).sum(1)[:, None] + (Yt * Yt).sum(1)[None, :] - 2 * (Xt @ Yt.T)
    gv, gi = torch.sort(d, dim=1, stable=True)
    gv, gi = gv[:, :k].numpy(), gi[:, :k].numpy()
    for exact in (True, False):
        fails = parity.topk_report(gv, gi, ov, oi, om, k, False, np.float32, exact=exact)
        assert not fails, "float32 expansion search rejected: %s" % fails[:2]
    ties = [(row, p) for row in range(X.shape[0]) for p in range(k - 1) if ov[row, p] == ov[row, p + 1]]
    seps = [(row, p) for row in range(X.shape[0]) for p in range(k - 1) if ov[row, p] != ov[row, p + 1]]
    assert ties and seps, "the grid has both tied and separated neighbours"
    for row, p in (ties[0], seps[0]):
        bi, bv = gi.copy(), gv.copy()
        bi[row, [p, p + 1]] = bi[row, [p + 1, p]]
        bv[row, [p, p + 1]] = bv[row, [p + 1, p]]
        for exact in (True, False):
            assert parity.topk_report(bv, bi, ov, oi, om, k, False, np.float32, exact=exact), \
                "swapped positions %d/%d of row %d accepted (exact=%s)" % (p, p + 1, row, exact)



# ---------------------------------------------------------------- gradient magnitude pins
def pin_backward_mag_golden():
    """Gradients and their first-order magnitudes on hand-derived cases
    (fixture backward_magnitudes): log-sum-exp, kernel product, softmax@V
    and an op chain with a weight and exp."""
    c = _golden()["backward_magnitudes"]

    def vals(x):
        return [[_ev(v) for v in row] for row in x] if isinstance(x[0], list) else [[_ev(v) for v in x]]

    for dt in DTYPES:
        X, Y = np.array(c["X"], dt), np.array(c["Y"], dt)
        e = oracle.Expr(X, Y, c["metric"])
        for cons in ("logsumexp", "matmul", "softmax_matmul"):
            cc = c[cons]
            V = np.array(cc["V"], dt) if "V" in cc else None
            r = oracle.backward(e, cons, np.array(cc["G"], dt), V=V)
            for key in ("dX", "dY", "dV"):
                if key in cc:
                    _close(r[key][0], vals(cc[key]), rtol=1e-13, atol=1e-15, what="%s %s" % (cons, key))
                    _close(r[key][1], vals(cc[key + "_mag"]), rtol=1e-13, atol=1e-15, what="%s %s mag" % (cons, key))
        ch = c["chain"]
        ops = [(n, np.array(a, dt) if isinstance(a, list) else a) for n, a in ch["ops"]]
        e = oracle.Expr(np.array(ch["X"], dt), np.array(ch["Y"], dt), c["metric"], ops=ops)
        r = oracle.backward(e, "matmul", np.array(ch["G"], dt), V=np.array(ch["V"], dt))
        _close(r["dX"][0], vals(ch["dX"]), rtol=1e-13, what="chain dX")
        _close(r["dX"][1], vals(ch["dX_mag"]), rtol=1e-13, what="chain dX mag")
        _close(r["ops"][0][0], [_ev(v) for v in ch["weight_rows"]], rtol=1e-13, what="chain weight grad")
        _close(r["ops"][0][1], [_ev(v) for v in ch["weight_rows_mag"]], rtol=1e-13, what="chain weight grad mag")


def _attention_grads_f32(Q, K, V, G, scale):
    """dQ, dK, dV of sum(softmax(Q K^T scale) V * G) by torch autograd in
    float32 (library matmuls, a differently ordered evaluation)."""
    Qt = torch.tensor(Q, requires_grad=True)
    Kt = torch.tensor(K, requires_grad=True)
    Vt = torch.tensor(V, requires_grad=True)
    O = torch.softmax((Qt @ Kt.T) * scale, -1) @ Vt
    return torch.autograd.grad((O * torch.from_numpy(G)).sum(), (Qt, Kt, Vt))


def pin_grad_rule_accepts_float32_autograd():
    """The gradient rule accepts float32 gradients taken by torch autograd
    of the dense form: attention softmax@V, the InfoNCE log-sum-exp without
    the self pair, and the rbf kernel product of narrow points."""
    Q, K, V, ops = _attention_case()
    G = _rng(510).standard_normal((Q.shape[0], V.shape[1])).astype(np.float32)
    ref = oracle.backward(oracle.Expr(Q, K, "linear", ops=ops), "softmax_matmul", G, V=V)
    for name, g in zip(("dX", "dY", "dV"), _attention_grads_f32(Q, K, V, G, 0.125)):
        ok, ratio, _ = parity.grad_rule(g.numpy(), *ref[name], np.float32)
        assert ok, "attention %s: float32 autograd rejected (err/tol %.3g)" % (name, ratio)
    z, b, zops = _infonce_case()
    g = _rng(511).standard_normal(z.shape[0]).astype(np.float32)
    ref = oracle.backward(oracle.Expr(z, z, "linear", ops=zops), "logsumexp", g, exclude_self=True)
    zt = torch.tensor(z, requires_grad=True)
    S = (zt @ zt.T) * np.float32(1.0 / 0.07) + torch.from_numpy(b)[:, None]
    S = S.masked_fill(torch.eye(z.shape[0], dtype=torch.bool), -float("inf"))
    (dz,) = torch.autograd.grad((torch.logsumexp(S, -1) * torch.from_numpy(g)).sum(), zt)
    # X and Y alias: the set's gradient is the sum of both sides'.
    ok, ratio, _ = parity.grad_rule(dz.numpy(), ref["dX"][0] + ref["dY"][0], ref["dX"][1] + ref["dY"][1], np.float32)
    assert ok, "infonce: float32 autograd rejected (err/tol %.3g)" % ratio
    r = _rng(512)
    X = r.standard_normal((300, 3)).astype(np.float32)
    Y = r.standard_normal((333, 3)).astype(np.float32)
    Vk = np.concatenate([r.standard_normal((333, 3)), np.ones((333, 1))], 1).astype(np.float32)
    Gk = r.standard_normal((300, 4)).astype(np.float32)
    ref = oracle.backward(oracle.Expr(X, Y, "rbf", gamma=0.5), "matmul", Gk, V=Vk)
    Xt, Yt, Vt = (torch.tensor(a, requires_grad=True) for a in (X, Y, Vk))
    Kt = torch.exp(-0.5 * ((Xt[:, None, :] - Yt[None, :, :]) ** 2).sum(-1))
    grads = torch.autograd.grad(((Kt @ Vt) * torch.from_numpy(Gk)).sum(), (Xt, Yt, Vt))
    for name, gg in zip(("dX", "dY", "dV"), grads):
        ok, ratio, _ = parity.grad_rule(gg.numpy(), *ref[name], np.float32)
        assert ok, "kernel product %s: float32 autograd rejected (err/tol %.3g)" % (name, ratio)


def pin_grad_rule_rejects_dropped_pair_and_kept_self():
    """The oracle's own gradients with one key dropped (a column mask), or
    with the self pair kept, fail the gradient rule."""
    Q, K, V, ops = _attention_case()
    G = _rng(513).standard_normal((Q.shape[0], V.shape[1])).astype(np.float32)
    ref = oracle.backward(oracle.Expr(Q, K, "linear", ops=ops), "softmax_matmul", G, V=V)
    for drop in (64, K.shape[0] - 1):
        keep = np.ones(K.shape[0], bool)
        keep[drop] = False
        got = oracle.backward(oracle.Expr(Q, K, "linear", ops=ops + [("mask_columns", keep)]), "softmax_matmul", G, V=V)
        for name in ("dX", "dY", "dV"):
            ok, ratio, _ = parity.grad_rule(got[name][0], *ref[name], np.float32)
            assert not ok, "attention %s without key %d accepted (err/tol %.3g)" % (name, drop, ratio)
    z, b, zops = _infonce_case()
    g = _rng(514).standard_normal(z.shape[0]).astype(np.float32)
    e = oracle.Expr(z, z, "linear", ops=zops)
    ref = oracle.backward(e, "logsumexp", g, exclude_self=True)
    got = oracle.backward(e, "logsumexp", g, exclude_self=False)
    for name in ("dX", "dY"):
        ok, ratio, _ = parity.grad_rule(got[name][0], *ref[name], np.float32)
        assert not ok, "infonce %s with the self pair kept accepted (err/tol %.3g)" % (name, ratio)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
