"""Planted mistakes in the oracle must each trip at least one pin (CPU only).

Each mutant is a one-line textual change to oracle.cpp -- a dropped term, a
wrong sign, a wrong index, a mixed-up operand, a reversed order -- compiled to
a temporary library. Every pin of oracle_pins.py is run against it; the test
passes only if some pin fails. Mutations keep every access in bounds.
"""
import concurrent.futures as cf
import inspect
import os
import subprocess

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.cpp")

MUTANTS = [
    ("linear_drops_first_feature",
     "for (int64_t d = 0; d < e.D; ++d) {\n        R p = x(i, d) * y(j, d);",
     "for (int64_t d = 1; d < e.D; ++d) {\n        R p = x(i, d) * y(j, d);"),
    ("difference_sign", "R diff = a - b;", "R diff = a + b;"),
    ("cosine_norm_not_rooted", "R den = std::sqrt(nx) * std::sqrt(ny);", "R den = nx * std::sqrt(ny);"),
    ("rbf_half_exponent", "s = rexp(-(R)e.gamma * sum_sq);", "s = rexp(-(R)e.gamma * sum_sq / 2);"),
    ("x_read_from_y", "R x(int64_t i, int64_t d) const { return (R)X[i * e.ldx + d]; }",
     "R x(int64_t i, int64_t d) const { return (R)Y[(i % e.M) * e.ldy + d]; }"),
    ("mul_divides", "case OP_MUL: s = (R)e.op_scalar[k] * s;", "case OP_MUL: s = s / (R)e.op_scalar[k];"),
    ("add_rows_by_column", "case OP_ADD_ROWS: s = s + vec(k, i);", "case OP_ADD_ROWS: s = s + vec(k, j % e.N);"),
    ("add_columns_by_row", "case OP_ADD_COLS: s = s + vec(k, j);", "case OP_ADD_COLS: s = s + vec(k, i % e.M);"),
    ("weight_rows_by_column", "R w = vec(k, i);", "R w = vec(k, j % e.N);"),
    ("weight_columns_by_row", "R u = vec(k, j);", "R u = vec(k, i % e.M);"),
    ("exp_sign", "R ex = rexp(s);", "R ex = rexp(-s);"),
    ("matmul_drops_score", "acc[c] += s * v;", "acc[c] += v;"),
    ("displacement_sign", "acc[d] += s * (yd - xd);", "acc[d] += s * (xd - yd);"),
    ("self_pair_misplaced", "if (exclude_self && j == i) continue;", "if (exclude_self && j == i + 1) continue;"),
    ("lse_drops_max", "out[r] = m + rlog(l);", "out[r] = rlog(l);"),
    ("softmax_unnormalised", "R p = rexp(s[t] - m) / l;", "R p = rexp(s[t] - m);"),
    ("tie_order_reversed", "return a.j < b.j;", "return a.j > b.j;"),
    ("largest_ignored", "return largest ? (a.v > b.v) : (a.v < b.v);", "return (a.v < b.v);"),
    ("row_mask_ignored", "if (e.row_mask && !e.row_mask[i]) return false;", ""),
    ("column_mask_by_row", "if (e.col_mask && !e.col_mask[j]) return false;",
     "if (e.col_mask && !e.col_mask[i % e.M]) return false;"),
    ("causal_strict", "if (e.has_upper && j - i > e.upper) return false;",
     "if (e.has_upper && j - i >= e.upper) return false;"),
    ("band_lower_sign", "if (e.has_lower && i - j > e.lower) return false;",
     "if (e.has_lower && j - i > e.lower) return false;"),
    ("group_of_row_index", "e.group_rows[i] != e.group_cols[j]", "e.group_rows[i] != e.group_cols[i % e.M]"),
    ("softmax_v_by_position", "const int64_t j = jx[t];", "const int64_t j = t;"),
    ("backward_exp_derivative", "          d = d * t[op + 1];", "          d = d * t[op];"),
    ("backward_weight_rows_grad", "if (side == 0) { gops[op] += d * t[op];", "if (side == 0) { gops[op] += d;"),
    ("backward_softmax_delta", "R a = gv(i, j) - delta[i];", "R a = gv(i, j);"),
    ("backward_distance_side_sign", "if (side == 1) c = -c;", ""),
    ("backward_displacement_direct", "gx[dd] += side == 0 ? -w : w;", "gx[dd] += w;"),
    ("backward_matmul_dv", "gvout[c] += t[n] * g(i, c);", "gvout[c] += g(i, c);"),
    ("backward_topk_position", "if (idx[i * k + p] == j) a += (R)G[i * ldg + p];",
     "if (idx[i * k + p] == j) a += (R)G[i * ldg];"),
    # Planted mistakes in the error magnitude `mag`, which scales every
    # tolerance of the comparison rule.
    ("mag_linear_times_1000", "mu += std::fabs(p);", "mu += 1000 * std::fabs(p);"),
    ("mag_distance_spread_from_difference", "R w = std::fabs(a) + std::fabs(b);", "R w = std::fabs(a - b);"),
    ("mag_rbf_without_spread", "mu = s * (1 + (R)e.gamma * spread);", "mu = s;"),
    ("mag_cosine_constant", "mu = 1 + 3 * adot / den;", "mu = 1;"),
    ("mag_mul_unscaled", "s = (R)e.op_scalar[k] * s; mu = std::fabs((R)e.op_scalar[k]) * mu;",
     "s = (R)e.op_scalar[k] * s; mu = mu;"),
    ("mag_add_ignores_new_score", "case OP_ADD: s = s + (R)e.op_scalar[k]; mu = mu + std::fabs(s);",
     "case OP_ADD: s = s + (R)e.op_scalar[k]; mu = mu;"),
    ("mag_exp_drops_one", "R ex = rexp(s); mu = ex * (1 + mu);", "R ex = rexp(s); mu = ex * mu;"),
    ("mag_weight_columns_unscaled", "s = u * s; mu = std::fabs(u) * mu;", "s = u * s; mu = mu;"),
    ("mag_matmul_times_1000", "m[c] += (std::fabs(s) + mu) * std::fabs(v);", "m[c] += 1000 * (std::fabs(s) + mu) * std::fabs(v);"),
    ("mag_displacement_drops_x", "m[d] += (std::fabs(s) + mu) * (std::fabs(yd) + std::fabs(xd));",
     "m[d] += (std::fabs(s) + mu) * std::fabs(yd);"),
    ("mag_lse_sum_not_max", "mumax = std::max(mumax, mu[t]);", "mumax = mumax + mu[t];"),
    ("mag_lse_drops_log", "mag[r] = mumax + rlog(l);", "mag[r] = mumax;"),
    ("mag_softmax_without_p", "av[c] += p * (1 + mu[t]) * std::fabs(v);", "av[c] += (1 + mu[t]) * std::fabs(v);"),
    ("mag_softmax_drops_cross_term", "mag[r * C + c] = av[c] + pmu * apv[c];", "mag[r * C + c] = av[c];"),
    ("mag_topk_of_first_pair", "mag[r * kk + p] = buf[p].mu;", "mag[r * kk + p] = buf[0].mu;"),
    # ... and in the gradients' first-order magnitudes.
    ("mag_backward_lse_without_mu", "*scale = std::fabs((R)G[i * ldg]) * p * (1 + mu + lm[i]);",
     "*scale = std::fabs((R)G[i * ldg]) * p;"),
    ("mag_backward_softmax_without_delta", "+ gv_abs(i, j) + dmag[i]);", "+ gv_abs(i, j));"),
    ("mag_backward_metric_grad_rounding", "gxm[dd] += dm * std::fabs(mg[dd]) + std::fabs(d) * mgm[dd];",
     "gxm[dd] += dm * std::fabs(mg[dd]);"),
    ("mag_backward_weight_rows_without_mu",
     "if (side == 0) { gops[op] += d * t[op]; gopsm[op] += dm * std::fabs(t[op]) + std::fabs(d) * mu[op]; }",
     "if (side == 0) { gops[op] += d * t[op]; gopsm[op] += dm * std::fabs(t[op]); }"),
    ("mag_backward_exp_factor", "dm = dm * t[op + 1] + std::fabs(d) * t[op + 1] * (1 + mu[op]);",
     "dm = dm * t[op + 1];"),
    ("mag_backward_matmul_dv_without_mu", "gvm[c] += (std::fabs(t[n]) + mu[n]) * std::fabs(g(i, c));",
     "gvm[c] += std::fabs(t[n]) * std::fabs(g(i, c));"),
]


def _build_one(tmpdir, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation %s does not match exactly once" % name
    path = os.path.join(tmpdir, name + ".cpp")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = os.path.join(tmpdir, "lib" + name + ".so")
    subprocess.run(["g++", "-O1", "-std=c++17", "-fopenmp", "-fPIC", "-shared", path, "-o", so], check=True)
    return name, so


@pytest.fixture(scope="module")
def mutant_libs(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("mutants"))
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        return dict(ex.map(lambda m: _build_one(d, *m), MUTANTS))


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, mutant_libs):
    lib = oracle._open(mutant_libs[name])
    prev = oracle._load()
    oracle._lib = lib
    caught = []
    try:
        for pin in ALL_PINS:
            try:
                pin()
            except AssertionError:
                caught.append(pin.__name__)
    finally:
        oracle._lib = prev
    assert caught, "no pin catches the planted mistake %s" % name


# Planted mistakes in the oracle's Python-level MMD (a composition of the
# dense oracle scores), applied to its source text and run in the oracle
# module's namespace.
PY_MUTANTS = [
    ("mmd_keeps_diagonal", "mmd2", "keep = ~np.eye(k.shape[0], dtype=bool)", "keep = np.ones_like(k, dtype=bool)"),
    ("mmd_unbiased_over_n_squared", "mmd2", "cx = one / (n * (n - 1)) if unbiased else one / (n * n)",
     "cx = one / (n * n)"),
    ("mmd_cross_term_once", "mmd2", "value = cx * sxx + cy * syy - 2 * cxy * sxy",
     "value = cx * sxx + cy * syy - cxy * sxy"),
    ("mmd_y_within_from_x", "mmd2", "syy, ayy, _ = term(Y, Y, True)", "syy, ayy, _ = term(X, X, True)"),
    ("mmd_grad_one_triangle", "mmd2_grad",
     "parts = pieces(A, A, [(\"band\", (-1, 10 ** 9))], c) + pieces(A, A, [(\"band\", (10 ** 9, -1))], c)",
     "parts = pieces(A, A, [(\"band\", (-1, 10 ** 9))], c)"),
    ("mmd_grad_row_side_only", "mmd2_grad", "return sum(p[0] for p in parts), sum(p[1] for p in parts)",
     "return sum(p[0] for p in parts[::2]), sum(p[1] for p in parts[::2])"),
    ("mmd_grad_cross_sign", "mmd2_grad", "cx_, cy_ = pieces(X, Y, [], -2.0 * g / (n * m))",
     "cx_, cy_ = pieces(X, Y, [], 2.0 * g / (n * m))"),
    ("mmd_grad_shared_cloud_not_summed", "mmd2_grad", "dY = dY[0].sum(0, keepdims=True), dY[1].sum(0, keepdims=True)",
     "dY = dY[0][:1], dY[1][:1]"),
]


@pytest.mark.parametrize("name", [m[0] for m in PY_MUTANTS])
def test_planted_python_mistake_is_caught(name):
    _, fn, old, new = next(m for m in PY_MUTANTS if m[0] == name)
    src = inspect.getsource(getattr(oracle, fn))
    assert src.count(old) == 1, "mutation %s does not match exactly once" % name
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), "<mutant %s>" % name, "exec"), ns)
    keep = getattr(oracle, fn)
    setattr(oracle, fn, ns[fn])
    caught = []
    try:
        for pin in ALL_PINS:
            try:
                pin()
            except AssertionError:
                caught.append(pin.__name__)
    finally:
        setattr(oracle, fn, keep)
    assert caught, "no pin catches the planted mistake %s" % name
