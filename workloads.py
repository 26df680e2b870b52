"""Seeded synthetic inputs for the pairwise-score workloads.

This module only draws random inputs and states each workload's parameters;
it holds none of the score arithmetic, so both the GPU library's tests and
the CPU oracle can take their inputs from it. Every draw uses a CPU
``torch.Generator`` seeded per workload, draws in float64 in the order
listed, then casts to the workload's dtype. ``scale`` arguments shrink a
workload (same distributions) for parity tests the oracle finishes quickly.

The pages print no dataset or benchmark for these tasks; the shapes follow
the uses the torchpairwise guide "Using Torchpairwise in Models" names in its
Task Map (attention, Nadaraya-Watson kernel product, InfoNCE log-sum-exp,
k-NN retrieval) and its Stein Variational Gradient Descent section.

Ops are listed in the neutral vocabulary of that guide's Score Expressions
section: ("mul", c), ("add", c), ("add_rows", name), ("add_columns", name),
("weight_rows", name), ("weight_columns", name), ("exp", None), and the
masks ("causal", d) and ("same_group", (rows, columns)); a vector argument
names an array of the workload's dict.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator("cpu")
    g.manual_seed(seed)
    return g


def _randn(g, *shape):
    return torch.randn(*shape, generator=g, dtype=torch.float64)


@dataclass
class Case:
    """One consumer call on a workload."""
    name: str
    consumer: str            # matmul | displacement | logsumexp | softmax_matmul | topk | mean | cg_solve | mmd
    #                          | backward_<consumer>
    x: str                   # array used as X
    y: str                   # array used as Y
    metric: str
    gamma: float = 1.0
    ops: list = field(default_factory=list)
    v: str | None = None     # array used as V (matmul / softmax_matmul)
    exclude_self: bool = False
    k: int = 0
    largest: bool = False
    transpose: bool = False  # reduce over rows instead (the transposed score)
    pairs: int | None = None  # pairs the masks keep (None: all N * M)
    params: dict = field(default_factory=dict)  # consumer settings (cg_solve: shift, rtol, max_iter; mmd: unbiased)


def rbf_small(n: int = 1024, m: int | None = None, d: int = 3, seed: int = 1001):
    """Nadaraya-Watson kernel product plus distance consumers, float32.

    X, Y ~ N(0,1) [n,3]; V = [randn(m,3), ones] so the last product column is
    the row mass. Consumers: rbf (gamma 0.5) product, log-sum-exp of -D/2 and
    top-8 smallest of D = sqeuclidean(X, Y).
    """
    m = n if m is None else m
    g = _gen(seed)
    X = _randn(g, n, d)
    Y = _randn(g, m, d)
    V0 = _randn(g, m, 3)
    V = torch.cat([V0, torch.ones(m, 1, dtype=torch.float64)], 1)
    arrays = {k: t.to(torch.float32).numpy() for k, t in dict(X=X, Y=Y, V=V).items()}
    cases = [
        Case("rbf_matmul", "matmul", "X", "Y", "rbf", gamma=0.5, v="V"),
        Case("sqeuclid_lse", "logsumexp", "X", "Y", "sqeuclidean", ops=[("mul", -0.5)]),
        Case("sqeuclid_topk", "topk", "X", "Y", "sqeuclidean", k=8),
    ]
    return arrays, cases


def rbf_large(n: int = 65536, seed: int = 1011):
    """The rbf kernel product of ``rbf_small`` at n = m = 65536 (float32)."""
    arrays, cases = rbf_small(n=n, seed=seed)
    return arrays, cases[:1]


def rbf_small_large(n: int = 65536, seed: int = 1015):
    """The three calls of ``rbf_small`` (rbf product with the row mass,
    log-sum-exp of -D/2, top-8 of D) at n = m = 65536, float32: the small
    configuration's consumers at a size where throughput is measured."""
    return rbf_small(n=n, seed=seed)


def attention(n: int = 16384, m: int | None = None, d: int = 64, c: int = 64, seed: int = 1002):
    """Softmax attention, float32: Q, K, V ~ N(0,1); scores linear(Q,K)/8."""
    m = n if m is None else m
    g = _gen(seed)
    Q = _randn(g, n, d)
    K = _randn(g, m, d)
    V = _randn(g, m, c)
    arrays = {k: t.to(torch.float32).numpy() for k, t in dict(Q=Q, K=K, V=V).items()}
    scale = 1.0 / math.sqrt(64.0)
    cases = [Case("attention", "softmax_matmul", "Q", "K", "linear", ops=[("mul", scale)], v="V")]
    return arrays, cases


def infonce(n: int = 65536, d: int = 64, seed: int = 1003):
    """InfoNCE row log-sum-exp excluding self, float32.

    z = rows of randn normalised to unit length (in float64, then cast);
    scores z.z^T / 0.07 plus a per-row bias b ~ N(0, variance 0.1).
    """
    g = _gen(seed)
    r = _randn(g, n, d)
    z = r / r.norm(dim=1, keepdim=True)
    b = math.sqrt(0.1) * _randn(g, n)
    arrays = {"z": z.to(torch.float32).numpy(), "b": b.to(torch.float32).numpy()}
    cases = [Case("infonce", "logsumexp", "z", "z", "linear", ops=[("mul", 1.0 / 0.07), ("add_rows", "b")],
                  exclude_self=True)]
    return arrays, cases


def knn(n_query: int = 65536, n_ref: int = 1 << 20, d: int = 32, centres: int = 256, seed: int = 1004):
    """k-NN retrieval, float32: top-10 smallest sqeuclidean distances.

    256 centres with coordinates N(0, 4) (sd 2), equal weights; references
    and queries are a uniformly drawn centre plus N(0, I) noise.
    """
    g = _gen(seed)
    cen = 2.0 * _randn(g, centres, d)
    lr = torch.randint(centres, (n_ref,), generator=g)
    R = cen[lr] + _randn(g, n_ref, d)
    lq = torch.randint(centres, (n_query,), generator=g)
    Q = cen[lq] + _randn(g, n_query, d)
    arrays = {"Q": Q.to(torch.float32).numpy(), "R": R.to(torch.float32).numpy()}
    cases = [Case("knn", "topk", "Q", "R", "sqeuclidean", k=10)]
    return arrays, cases


def svgd(n: int = 131072, d: int = 16, seed: int = 1005):
    """SVGD direction, float64: x ~ N(0, I), score = -x (standard normal
    target), rbf gamma = 1/16; one kernel product and one displacement."""
    g = _gen(seed)
    x = _randn(g, n, d)
    arrays = {"x": x.numpy(), "score": (-x).numpy()}
    gamma = 1.0 / 16.0
    cases = [
        Case("svgd_matmul", "matmul", "x", "x", "rbf", gamma=gamma, v="score"),
        Case("svgd_displacement", "displacement", "x", "x", "rbf", gamma=gamma),
    ]
    return arrays, cases


def chamfer(n: int = 65536, m: int = 65536, d: int = 3, seed: int = 1006):
    """Chamfer-style nearest neighbours in both directions, float32: D.min(-1)
    and D.min(-2) on D = sqeuclidean(X, Y) for two N(0, I) point clouds
    (Task Map, Chamfer row)."""
    g = _gen(seed)
    X = _randn(g, n, d)
    Y = _randn(g, m, d)
    arrays = {"X": X.to(torch.float32).numpy(), "Y": Y.to(torch.float32).numpy()}
    cases = [Case("chamfer_x_to_y", "topk", "X", "Y", "sqeuclidean", k=1),
             Case("chamfer_y_to_x", "topk", "X", "Y", "sqeuclidean", k=1, transpose=True)]
    return arrays, cases


def cosine_knn(n_query: int = 32768, n_ref: int = 524288, d: int = 64, seed: int = 1007):
    """Retrieval by cosine distance on encoded features, float32: top-10
    smallest cosine distances (Features page, "Prepare Once, Use Several
    Consumers": a cosine_distances head on extracted features)."""
    g = _gen(seed)
    R = _randn(g, n_ref, d)
    Q = _randn(g, n_query, d)
    arrays = {"Q": Q.to(torch.float32).numpy(), "R": R.to(torch.float32).numpy()}
    return arrays, [Case("cosine_knn", "topk", "Q", "R", "cosine_distances", k=10)]


def feature_mean(n: int = 65536, m: int = 65536, d: int = 16, seed: int = 1008):
    """Row mean of squared distances between two feature sets, float32 (Features
    page, Native Deployment: pairwise_expression(features, other,
    "sqeuclidean") then reduce("mean", -1))."""
    g = _gen(seed)
    F = _randn(g, n, d)
    G = _randn(g, m, d)
    arrays = {"F": F.to(torch.float32).numpy(), "G": G.to(torch.float32).numpy()}
    return arrays, [Case("feature_mean", "mean", "F", "G", "sqeuclidean")]


def attention_causal(n: int = 16384, d: int = 64, c: int = 64, seed: int = 1009):
    """Causal softmax attention, float32: Q, K, V ~ N(0,1), scores
    linear(Q,K)/8, pairs j <= i only (Task Map, Attention row:
    masks.causal()). Kept pairs n (n + 1) / 2."""
    arrays, cases = attention(n=n, d=d, c=c, seed=seed)
    c0 = cases[0]
    c0.name = "attention_causal"
    c0.ops = c0.ops + [("causal", 0)]
    c0.pairs = n * (n + 1) // 2
    return arrays, cases


def attention_packed(n: int = 16384, d: int = 64, c: int = 64, min_len: int = 256, max_len: int = 4096,
                     seed: int = 1010):
    """Packed causal attention, float32: sequences of lengths uniform in
    [min_len, max_len) laid end to end up to n rows (the last one cut), each
    attending causally within itself (masks.same_group on the sequence ids
    plus masks.causal())."""
    g = _gen(seed)
    lengths = []
    while sum(lengths) < n:
        lengths.append(int(torch.randint(min_len, max_len, (1,), generator=g)))
    lengths[-1] -= sum(lengths) - n
    seg = np.repeat(np.arange(len(lengths), dtype=np.int64), lengths)
    Q = _randn(g, n, d)
    K = _randn(g, n, d)
    V = _randn(g, n, c)
    arrays = {k: t.to(torch.float32).numpy() for k, t in dict(Q=Q, K=K, V=V).items()}
    arrays["seg"] = seg
    scale = 1.0 / math.sqrt(float(d))
    cases = [Case("attention_packed", "softmax_matmul", "Q", "K", "linear", v="V",
                  ops=[("mul", scale), ("same_group", ("seg", "seg")), ("causal", 0)],
                  pairs=sum(L * (L + 1) // 2 for L in lengths))]
    return arrays, cases


def attention_backward(n: int = 16384, d: int = 64, c: int = 64, seed: int = 1013):
    """Backward of the softmax attention workload, float32: the arrays of
    `attention` plus an upstream gradient dO ~ N(0, 1) [n, c]; gradients of
    Q, K and V (guide: backward by replay)."""
    arrays, cases = attention(n=n, d=d, c=c, seed=seed)
    g = _gen(seed + 1)
    arrays["dO"] = _randn(g, n, c).to(torch.float32).numpy()
    c0 = cases[0]
    c0.name = "attention_backward"
    c0.consumer = "backward_softmax_matmul"
    c0.params = {"G": "dO"}
    return arrays, cases


def attention_causal_backward(n: int = 16384, d: int = 64, c: int = 64, seed: int = 1014):
    """Backward of causal softmax attention, float32 (the arrays of
    `attention`, dO ~ N(0, 1)); kept pairs n (n + 1) / 2."""
    arrays, cases = attention_backward(n=n, d=d, c=c, seed=seed)
    c0 = cases[0]
    c0.name = "attention_causal_backward"
    c0.ops = c0.ops + [("causal", 0)]
    c0.pairs = n * (n + 1) // 2
    return arrays, cases


def kernel_ridge(n: int = 65536, d: int = 16, seed: int = 1012):
    """Kernel ridge regression / GP mean, float32 (Task Map, Kernel ridge row:
    solve(K + a * eye_like(K), Y, method="cg")): x ~ N(0, I) [n, 16], rbf
    gamma = 1/32, targets y = sin(x . w) + 0.1 noise with w ~ N(0, I/16),
    a = 10, relative residual 1e-3."""
    g = _gen(seed)
    X = _randn(g, n, d)
    w = _randn(g, d) / 4.0
    y = torch.sin(X @ w)[:, None] + 0.1 * _randn(g, n, 1)
    arrays = {"x": X.to(torch.float32).numpy(), "y": y.to(torch.float32).numpy()}
    cases = [Case("kernel_ridge", "cg_solve", "x", "x", "rbf", gamma=1.0 / 32, v="y",
                  params={"shift": 10.0, "rtol": 1e-3, "max_iter": 1000})]
    return arrays, cases


def mmd(n: int = 16384, m: int | None = None, d: int = 16, seed: int = 1016):
    """Two-sample test statistic, float32 (Task Map, MMD row:
    mmd_statistics(X[None], Y[None], kernel="rbf", gamma=g), unbiased by
    default): X ~ N(0, I) [n, 16] and Y ~ N(0.1, I) [m, 16], one cloud each;
    rbf gamma = 1/32. Its pairs are the n(n-1)/2 + m(m-1)/2 distinct
    within-cloud pairs and the n m cross pairs."""
    m = n if m is None else m
    g = _gen(seed)
    X = _randn(g, n, d)
    Y = 0.1 + _randn(g, m, d)
    arrays = {"X": X.to(torch.float32).numpy(), "Y": Y.to(torch.float32).numpy()}
    pairs = n * (n - 1) // 2 + m * (m - 1) // 2 + n * m
    cases = [Case("mmd", "mmd", "X", "Y", "rbf", gamma=1.0 / 32, pairs=pairs, params={"unbiased": True})]
    return arrays, cases


def resolve(arg, arrays):
    """An op argument with array names replaced by the arrays."""
    if isinstance(arg, str):
        return arrays[arg]
    if isinstance(arg, tuple):
        return tuple(resolve(a, arrays) for a in arg)
    return arg


# name -> (generator, full-size kwargs, reduced kwargs for quick parity runs)
WORKLOADS = {
    "rbf_small": (rbf_small, {}, {"n": 300, "m": 333}),
    "rbf_large": (rbf_large, {}, {"n": 2000}),
    "rbf_small_large": (rbf_small_large, {}, {"n": 1500}),
    "attention": (attention, {}, {"n": 700, "m": 650}),
    "infonce": (infonce, {}, {"n": 900}),
    "knn": (knn, {}, {"n_query": 500, "n_ref": 4099}),
    "svgd": (svgd, {}, {"n": 1100}),
    "chamfer": (chamfer, {}, {"n": 700, "m": 900}),
    "cosine_knn": (cosine_knn, {}, {"n_query": 300, "n_ref": 3000}),
    "feature_mean": (feature_mean, {}, {"n": 800, "m": 1000}),
    "attention_causal": (attention_causal, {}, {"n": 700}),
    "attention_packed": (attention_packed, {}, {"n": 900, "min_len": 40, "max_len": 300}),
    "kernel_ridge": (kernel_ridge, {}, {"n": 900}),
    "attention_backward": (attention_backward, {}, {"n": 700}),
    "attention_causal_backward": (attention_causal_backward, {}, {"n": 700}),
    "mmd": (mmd, {}, {"n": 600, "m": 500}),
}


def make(name: str, reduced: bool = False, **override):
    fn, full, small = WORKLOADS[name]
    kw = dict(small if reduced else full)
    kw.update(override)
    return fn(**kw)


def sample_rows(n: int, stride: int = 61, edge: int = 256) -> np.ndarray:
    """A row subset touching every tile position and both ragged ends:
    rows i with i % stride == 0, plus the first and last `edge` rows."""
    rows = set(range(0, n, stride)) | set(range(min(edge, n))) | set(range(max(0, n - edge), n))
    return np.array(sorted(rows), dtype=np.int64)
