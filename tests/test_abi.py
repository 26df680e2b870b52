"""The C ABI on the CPU: the library loads, exports every function the header
declares, and validates arguments on the host before any device work.

No call here reaches a HIP launch: pointers are fake (never dereferenced by
host validation), and each call fails validation, or has N == 0 / k == 0,
before the library would enqueue anything.
"""
import ctypes

import pytest

import lazy_score_matrix_amd as pw

FAKE = 0x10000  # aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    return pw.load_library()


def test_exports_every_header_function(lib):
    names = pw.header_functions()
    assert {"pw_bind", "pw_release", "pw_workspace_size", "pw_matmul", "pw_displacement", "pw_logsumexp",
            "pw_softmax_matmul", "pw_topk", "pw_error_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def bind(lib, dtype=0, metric=0, gamma=1.0, X=FAKE, N=10, ldx=None, Y=FAKE, M=12, ldy=None, D=4, ops=()):
    h = ctypes.c_void_p()
    arr = (pw._Op * max(len(ops), 1))()
    for t, (kind, scalar, vec) in enumerate(ops):
        arr[t].kind, arr[t].scalar, arr[t].vec = kind, scalar, vec
    rc = lib.pw_bind(ctypes.byref(h), dtype, metric, gamma, X, N, D if ldx is None else ldx, Y, M,
                     D if ldy is None else ldy, D, arr, len(ops))
    return rc, h


def test_error_strings(lib):
    for code in (0, -1, -2, -3, -4):
        assert lib.pw_error_string(code)
    assert lib.pw_error_string(0) == b"ok"


def test_bind_validation(lib):
    ok, h = bind(lib)
    assert ok == pw.PW_OK and h.value
    lib.pw_release(h)
    lib.pw_release(None)
    cases = [
        (dict(dtype=2), pw.PW_ERR_INVALID),
        (dict(metric=4), pw.PW_ERR_INVALID),
        (dict(metric=2, gamma=-1.0), pw.PW_ERR_INVALID),
        (dict(metric=2, gamma=float("nan")), pw.PW_ERR_INVALID),
        (dict(metric=2, gamma=float("inf")), pw.PW_ERR_INVALID),
        (dict(D=0), pw.PW_ERR_UNSUPPORTED),
        (dict(D=65), pw.PW_ERR_UNSUPPORTED),
        (dict(N=-1), pw.PW_ERR_INVALID),
        (dict(ldx=3), pw.PW_ERR_INVALID),
        (dict(ldy=2), pw.PW_ERR_INVALID),
        (dict(X=0), pw.PW_ERR_INVALID),
        (dict(Y=0), pw.PW_ERR_INVALID),
        (dict(X=FAKE + 2), pw.PW_ERR_INVALID),                       # misaligned
        (dict(N=2 ** 31), pw.PW_ERR_UNSUPPORTED),
        (dict(ops=[(0, float("nan"), None)]), pw.PW_ERR_INVALID),
        (dict(ops=[(2, 0.0, None)]), pw.PW_ERR_INVALID),             # add_rows without vector
        (dict(ops=[(5, 0.0, None)]), pw.PW_ERR_INVALID),             # weight_columns without vector
        (dict(ops=[(13, 0.0, None)]), pw.PW_ERR_INVALID),            # bad kind
        (dict(ops=[(0, 2.0, None)] * 17), pw.PW_ERR_UNSUPPORTED),    # > PW_MAX_OPS
        (dict(ops=[(0, 2.0, None), (6, 0, None)] * 5), pw.PW_ERR_UNSUPPORTED),  # > 8 fused stages
        (dict(ops=[(7, 0.0, None)]), pw.PW_ERR_INVALID),             # mask_rows without vector
        (dict(ops=[(8, 0.0, FAKE), (8, 0.0, FAKE)]), pw.PW_ERR_INVALID),  # two column masks
        (dict(ops=[(9, 0.5, None)]), pw.PW_ERR_INVALID),             # band bound not an integer
        (dict(ops=[(10, float("inf"), None)]), pw.PW_ERR_INVALID),   # band bound not finite
        (dict(ops=[(11, 0.0, FAKE)]), pw.PW_ERR_INVALID),            # row groups without column groups
        (dict(ops=[(11, 0.0, FAKE + 4), (12, 0.0, FAKE)]), pw.PW_ERR_INVALID),  # misaligned group ids
    ]
    for kw, want in cases:
        rc, h = bind(lib, **kw)
        assert rc == want, (kw, rc)
        assert not h.value
    # Boundary values accepted: D = 1 and 64, gamma = 0, X aliasing Y, empty sets.
    for kw in (dict(D=1), dict(D=64), dict(metric=2, gamma=0.0), dict(N=0, X=0), dict(M=0, Y=0),
               dict(ops=[(0, 0.5, None), (2, 0, FAKE), (3, 0, FAKE), (6, 0, None), (4, 0, FAKE), (5, 0, FAKE)]),
               dict(ops=[(7, 0, FAKE), (8, 0, FAKE + 1), (9, -3.0, None), (10, 2.0, None), (9, 5.0, None),
                         (11, 0, FAKE), (12, 0, FAKE), (0, 2.0, None)] * 1),
               dict(ops=[(0, 2.0, None)] * 16)):
        rc, h = bind(lib, **kw)
        assert rc == pw.PW_OK, kw
        lib.pw_release(h)


def ws_size(lib, h, consumer, C=0, k=0):
    n = ctypes.c_size_t()
    rc = lib.pw_workspace_size(h, consumer, C, k, ctypes.byref(n))
    return rc, n.value


def test_workspace_size_bounded(lib):
    """The workspace never grows with N*M: at fixed N it is constant in M
    (the guide's introduction bounds scratch by the tiles), and it scales with N (C + k)."""
    for cons, C, k in ((0, 4, 0), (1, 0, 0), (2, 0, 0), (3, 64, 0), (4, 0, 10)):
        sizes = []
        for M in (4096, 65536, 1 << 20, 1 << 24):
            rc, h = bind(lib, N=65536, M=M, D=32)
            assert rc == 0
            rc, n = ws_size(lib, h, cons, C, k)
            assert rc == 0
            sizes.append(n)
            lib.pw_release(h)
        assert max(sizes) <= sizes[0] * 1.01 + 4096, (cons, sizes)
        assert max(sizes) < 65536 * 64 * (C + k + 3) * 8 + (1 << 20)


def test_workspace_includes_epilogue_vectors(lib):
    rc, h = bind(lib, N=1000, M=3000, ops=[(2, 0, FAKE), (3, 0, FAKE)])
    assert rc == 0
    _, n = ws_size(lib, h, 2)
    assert n >= 2 * 1000 * 4 + 2 * 3000 * 4
    lib.pw_release(h)


def test_consumer_validation(lib):
    rc, h = bind(lib, N=10, M=12, D=4)
    assert rc == 0
    V = FAKE
    # matmul / softmax
    assert lib.pw_matmul(h, V, 0, 4, FAKE, 4, FAKE, 1 << 20, None) == pw.PW_ERR_INVALID      # C = 0
    assert lib.pw_matmul(h, V, 4, 3, FAKE, 4, FAKE, 1 << 20, None) == pw.PW_ERR_INVALID      # ldv < C
    assert lib.pw_matmul(h, V, 4, 4, FAKE, 3, FAKE, 1 << 20, None) == pw.PW_ERR_INVALID      # ldo < C
    assert lib.pw_matmul(h, 0, 4, 4, FAKE, 4, FAKE, 1 << 20, None) == pw.PW_ERR_INVALID      # V null
    assert lib.pw_matmul(h, V, 4, 4, 0, 4, FAKE, 1 << 20, None) == pw.PW_ERR_INVALID         # out null
    assert lib.pw_softmax_matmul(h, V, 4, 4, FAKE + 1, 4, FAKE, 1 << 20, None) == pw.PW_ERR_INVALID
    assert lib.pw_matmul(None, V, 4, 4, FAKE, 4, FAKE, 1 << 20, None) == pw.PW_ERR_INVALID
    # displacement / logsumexp
    assert lib.pw_displacement(h, FAKE, 3, FAKE, 1 << 20, None) == pw.PW_ERR_INVALID          # ldo < D
    assert lib.pw_logsumexp(h, 2, FAKE, FAKE, 1 << 20, None) == pw.PW_ERR_INVALID            # bad flag
    assert lib.pw_logsumexp(h, 0, 0, FAKE, 1 << 20, None) == pw.PW_ERR_INVALID
    # top-k
    assert lib.pw_topk(h, 13, 0, FAKE, FAKE, FAKE, 1 << 20, None) == pw.PW_ERR_INVALID       # k > M
    assert lib.pw_topk(h, -1, 0, FAKE, FAKE, FAKE, 1 << 20, None) == pw.PW_ERR_INVALID
    assert lib.pw_topk(h, 3, 2, FAKE, FAKE, FAKE, 1 << 20, None) == pw.PW_ERR_INVALID        # bad largest
    assert lib.pw_topk(h, 0, 0, 0, 0, 0, 0, None) == pw.PW_OK                               # k = 0: no-op
    lib.pw_release(h)
    # workspace too small / missing: reported before any launch
    rc, h = bind(lib, N=10, M=100000, D=4)
    rc, need = ws_size(lib, h, 0, 4)
    assert rc == 0 and need > 0
    assert lib.pw_matmul(h, V, 4, 4, FAKE, 4, FAKE, need - 1, None) == pw.PW_ERR_WORKSPACE
    assert lib.pw_matmul(h, V, 4, 4, FAKE, 4, 0, need, None) == pw.PW_ERR_WORKSPACE
    lib.pw_release(h)
    # k above the fused list size
    rc, h = bind(lib, N=10, M=100)
    assert lib.pw_topk(h, 65, 0, FAKE, FAKE, FAKE, 1 << 20, None) == pw.PW_ERR_UNSUPPORTED
    lib.pw_release(h)


def test_empty_rows_are_noops(lib):
    rc, h = bind(lib, N=0, X=0, M=12)
    assert rc == 0
    assert lib.pw_matmul(h, FAKE, 4, 4, 0, 4, 0, 0, None) == pw.PW_OK
    assert lib.pw_displacement(h, 0, 4, 0, 0, None) == pw.PW_OK
    assert lib.pw_logsumexp(h, 1, 0, 0, 0, None) == pw.PW_OK
    assert lib.pw_softmax_matmul(h, FAKE, 4, 4, 0, 4, 0, 0, None) == pw.PW_OK
    assert lib.pw_topk(h, 3, 0, 0, 0, 0, 0, None) == pw.PW_OK
    _, n = ws_size(lib, h, 3, 4)
    assert n == 0
    lib.pw_release(h)


def test_plan_describe(lib):
    rc, h = bind(lib, N=65536, M=65536, D=3)
    buf = ctypes.create_string_buffer(256)
    assert lib.pw_plan_describe(h, 0, 4, 0, buf, 256) == 0
    assert b"splits=" in buf.value
    lib.pw_release(h)


def test_product_has_no_oracle_dependency():
    """The product package neither imports nor links the oracle."""
    import os
    import re
    root = os.path.dirname(pw.__file__)
    for dirpath, _, files in os.walk(root):
        for f in files:
            if f.endswith((".py", ".h", ".hip", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "liboracle" not in text, f


def test_backward_validation(lib):
    """pw_backward rejects bad arguments on the host before any launch."""
    ok, h = bind(lib, N=12, M=12, D=16)
    gin, gout = pw._GradIn(), pw._GradOut()
    gin.G, gin.ldg = FAKE, 4
    gin.V, gin.C, gin.ldv = FAKE, 4, 4
    gin.out, gin.ldo = FAKE, 4
    assert lib.pw_backward(h, 5, ctypes.byref(gin), ctypes.byref(gout), FAKE, 1 << 30, None) == pw.PW_ERR_INVALID
    assert lib.pw_backward(h, 0, None, ctypes.byref(gout), FAKE, 1 << 30, None) == pw.PW_ERR_INVALID
    gin.C = 65
    gin.ldv = gin.ldg = gin.ldo = 65
    assert lib.pw_backward(h, 3, ctypes.byref(gin), ctypes.byref(gout), FAKE, 1 << 30, None) == pw.PW_ERR_UNSUPPORTED
    gin.C, gin.ldv, gin.ldg, gin.ldo = 4, 4, 3, 4                        # ldg < C
    assert lib.pw_backward(h, 0, ctypes.byref(gin), ctypes.byref(gout), FAKE, 1 << 30, None) == pw.PW_ERR_INVALID
    gin.ldg = 4
    gin.out = 0                                                          # softmax needs its forward output
    assert lib.pw_backward(h, 3, ctypes.byref(gin), ctypes.byref(gout), FAKE, 1 << 30, None) == pw.PW_ERR_INVALID
    gin.out = FAKE
    gin.indices, gin.k = FAKE, 13                                        # k > M
    assert lib.pw_backward(h, 4, ctypes.byref(gin), ctypes.byref(gout), FAKE, 1 << 30, None) == pw.PW_ERR_INVALID
    gout.dX, gout.lddx = FAKE, 15                                        # lddx < D
    assert lib.pw_backward(h, 0, ctypes.byref(gin), ctypes.byref(gout), FAKE, 1 << 30, None) == pw.PW_ERR_INVALID
    gout.lddx = 16
    n = ctypes.c_size_t()
    assert lib.pw_backward_workspace_size(h, 0, 4, 0, ctypes.byref(n)) == pw.PW_OK
    assert lib.pw_backward(h, 0, ctypes.byref(gin), ctypes.byref(gout), FAKE, n.value - 1, None) == pw.PW_ERR_WORKSPACE
    buf = ctypes.create_string_buffer(256)
    assert lib.pw_backward_plan_describe(h, 3, 4, 0, buf, 256) == pw.PW_OK and b"family=" in buf.value
    lib.pw_release(h)


def test_cg_solve_validation(lib):
    """pw_cg_solve rejects bad arguments on the host before any launch."""
    ok, h = bind(lib, N=12, M=12)
    assert ok == pw.PW_OK
    info = pw._SolveInfo()
    n = ctypes.c_size_t()
    assert lib.pw_cg_workspace_size(h, 3, ctypes.byref(n)) == pw.PW_OK and n.value > 0
    assert lib.pw_cg_workspace_size(h, 0, ctypes.byref(n)) == pw.PW_ERR_INVALID

    def call(shift=1.0, B=FAKE, C=3, ldb=3, A=FAKE, lda=3, max_iter=10, rtol=1e-6, check_every=4, ws=FAKE,
             ws_bytes=1 << 30, inf=True, handle=h):
        return lib.pw_cg_solve(handle, shift, B, C, ldb, A, lda, max_iter, rtol, check_every, ws, ws_bytes, None,
                               ctypes.byref(info) if inf else None)

    assert call(shift=0.0) == pw.PW_ERR_INVALID
    assert call(shift=-1.0) == pw.PW_ERR_INVALID
    assert call(shift=float("inf")) == pw.PW_ERR_INVALID
    assert call(C=0) == pw.PW_ERR_INVALID
    assert call(ldb=2) == pw.PW_ERR_INVALID
    assert call(lda=2) == pw.PW_ERR_INVALID
    assert call(max_iter=0) == pw.PW_ERR_INVALID
    assert call(check_every=0) == pw.PW_ERR_INVALID
    assert call(rtol=-1.0) == pw.PW_ERR_INVALID
    assert call(B=0) == pw.PW_ERR_INVALID
    assert call(A=FAKE + 2) == pw.PW_ERR_INVALID
    assert call(inf=False) == pw.PW_ERR_INVALID
    assert call(ws=0) == pw.PW_ERR_WORKSPACE
    assert call(ws_bytes=n.value - 1) == pw.PW_ERR_WORKSPACE
    lib.pw_release(h)
    ok, h2 = bind(lib, N=12, M=13)          # not square
    assert call(handle=h2) == pw.PW_ERR_INVALID
    lib.pw_release(h2)
    ok, h3 = bind(lib, N=0, M=0, X=0, Y=0)  # empty system: converged, nothing launched
    assert call(handle=h3, B=0, A=0) == pw.PW_OK and info.converged == 1 and info.iterations == 0
    lib.pw_release(h3)


def _plan(lib, consumer, C=0, k=0, **kw):
    rc, h = bind(lib, **kw)
    assert rc == pw.PW_OK
    buf = ctypes.create_string_buffer(512)
    assert lib.pw_plan_describe(h, consumer, C, k, buf, 512) == pw.PW_OK
    lib.pw_release(h)
    return dict(t.split("=", 1) for t in buf.value.decode().split() if "=" in t)


def test_blocked_vector_kernels_only_where_they_apply(lib):
    """The several-rows-per-thread vector kernels cover plain float scores of
    narrow points only: the kernel product and the row log-sum-exp of dot
    products and squared distances under at most one row-only stage (four
    rows, 256-column tiles, where that grid fills the chip), the rbf (or
    smaller) log-sum-exp and the row minimum (two rows). Score arithmetic they do not take, masks, cosine and float64
    plan one row per thread."""
    MATMUL, LSE, TOPK = 0, 2, 4
    N, M = 4100, 200000
    four = ("valu", "4", "1024", "256")
    # Too small a grid for 1024-row blocks: the finer kernels.
    for metric in (0, 1, 2):
        assert _plan(lib, MATMUL, 4, N=1024, M=1024, D=3, metric=metric)["rows"] == "1"
        assert _plan(lib, LSE, N=1024, M=1024, D=3, metric=metric)["rows"] == "2"
    for metric in (0, 1, 2):
        p = _plan(lib, MATMUL, 4, N=N, M=M, D=3, metric=metric)
        assert (p["family"], p["rows"], p["bm"], p["bn"]) == four, p
        p = _plan(lib, LSE, N=N, M=M, D=4, metric=metric)
        if metric == 2:
            assert p["rows"] == "2", p
        else:
            assert (p["family"], p["rows"], p["bm"], p["bn"]) == four, p
        assert _plan(lib, TOPK, 0, 1, N=N, M=M, D=2, metric=metric)["rows"] == "2"
    mul = [(pw.OPS["mul"], -0.5, None)]
    addr = [(pw.OPS["mul"], -0.5, None), (pw.OPS["add_rows"], 0.0, FAKE)]
    addc = [(pw.OPS["add_columns"], 0.0, FAKE)]
    maskc = [(pw.OPS["mask_columns"], 0.0, FAKE)]
    causal = [(pw.OPS["band_upper"], 0.0, None)]
    for metric in (0, 1):
        assert _plan(lib, LSE, N=N, M=M, D=3, ops=mul, metric=metric)["rows"] == "4"
        assert _plan(lib, LSE, N=N, M=M, D=3, ops=addr, metric=metric)["rows"] == "4"
    assert _plan(lib, LSE, N=N, M=M, D=3, ops=addr, metric=2)["rows"] == "2"
    one_row = [
        _plan(lib, MATMUL, 5, N=N, M=M, D=3),                 # value width above 4
        _plan(lib, MATMUL, 4, N=N, M=M, D=5),                 # five features
        _plan(lib, MATMUL, 4, N=N, M=M, D=3, metric=3),       # cosine
        _plan(lib, MATMUL, 4, N=N, M=M, D=3, dtype=1),        # float64
        _plan(lib, MATMUL, 4, N=N, M=M, D=3, ops=mul),        # score arithmetic
        _plan(lib, MATMUL, 4, N=N, M=M, D=3, ops=maskc),      # a column mask
        _plan(lib, LSE, N=N, M=M, D=3, ops=addc),             # a column stage
        _plan(lib, LSE, N=N, M=M, D=3, ops=causal),           # a pair mask
        _plan(lib, LSE, N=N, M=M, D=3, dtype=1),              # float64
        _plan(lib, TOPK, 0, 2, N=N, M=M, D=3),                # k = 2
        _plan(lib, TOPK, 0, 1, N=N, M=M, D=3, ops=maskc),     # a column mask
        _plan(lib, TOPK, 0, 1, N=N, M=M, D=3, metric=3),      # cosine
    ]
    for p in one_row:
        assert p["family"] == "valu" and p["rows"] == "1", p


def _bind_batched(lib, B=5, sx=0, sy=12 * 4, sv=0, N=10, M=12, D=4, ops=(), op_stride=(), metric=1):
    h = ctypes.c_void_p()
    arr = (pw._Op * max(len(ops), 1))()
    for t, (kind, scalar, vec) in enumerate(ops):
        arr[t].kind, arr[t].scalar, arr[t].vec = kind, scalar, vec
    bt = pw._Batch()
    bt.B, bt.sx, bt.sy, bt.sv = B, sx, sy, sv
    for t, s in enumerate(op_stride):
        bt.op_stride[t] = s
    rc = lib.pw_bind_batched(ctypes.byref(h), 0, metric, 1.0, FAKE, N, D, FAKE, M, D, D, arr, len(ops),
                             ctypes.byref(bt))
    return rc, h


def test_bind_batched_validation(lib):
    """A batch of B elements: strides >= 0, B in 1..65535, masks and scalar
    ops shared (stride 0); the plan reports the batch, the workspace holds
    one set of partials per element and never grows with N*M; backward and
    CG take unbatched handles only."""
    rc, h = _bind_batched(lib)
    assert rc == pw.PW_OK and h.value
    buf = ctypes.create_string_buffer(512)
    assert lib.pw_plan_describe(h, 0, 4, 0, buf, 512) == pw.PW_OK and b"batch=5" in buf.value
    n5 = ctypes.c_size_t()
    assert lib.pw_workspace_size(h, 4, 0, 3, ctypes.byref(n5)) == pw.PW_OK
    gin, gout = pw._GradIn(), pw._GradOut()
    assert lib.pw_backward(h, 0, ctypes.byref(gin), ctypes.byref(gout), FAKE, 1 << 20, None) == pw.PW_ERR_UNSUPPORTED
    nb = ctypes.c_size_t()
    assert lib.pw_backward_workspace_size(h, 0, 4, 0, ctypes.byref(nb)) == pw.PW_ERR_UNSUPPORTED
    assert lib.pw_cg_workspace_size(h, 1, ctypes.byref(nb)) == pw.PW_ERR_UNSUPPORTED
    lib.pw_release(h)
    # Per-element partials: a wide split plan at B = 1 and B = 7.
    sizes = []
    for B in (1, 7):
        rc, h = _bind_batched(lib, B=B, N=300, M=200000, D=32)
        n = ctypes.c_size_t()
        assert rc == pw.PW_OK and lib.pw_workspace_size(h, 4, 0, 10, ctypes.byref(n)) == pw.PW_OK
        sizes.append(n.value)
        lib.pw_release(h)
    assert sizes[1] > 6 * (sizes[0] - 4096) and sizes[1] < 300 * 200000, sizes
    assert _bind_batched(lib, B=0)[0] == pw.PW_ERR_INVALID
    assert _bind_batched(lib, B=65536)[0] == pw.PW_ERR_UNSUPPORTED
    assert _bind_batched(lib, sx=-1)[0] == pw.PW_ERR_INVALID
    assert _bind_batched(lib, sv=-4)[0] == pw.PW_ERR_INVALID
    addr = [(pw.OPS["add_rows"], 0.0, FAKE)]
    assert _bind_batched(lib, ops=addr, op_stride=(10,))[0] == pw.PW_OK
    assert _bind_batched(lib, ops=addr, op_stride=(-10,))[0] == pw.PW_ERR_INVALID
    maskc = [(pw.OPS["mask_columns"], 0.0, FAKE)]
    assert _bind_batched(lib, ops=maskc, op_stride=(12,))[0] == pw.PW_ERR_UNSUPPORTED
    assert _bind_batched(lib, ops=[(pw.OPS["mul"], 2.0, None)], op_stride=(3,))[0] == pw.PW_ERR_UNSUPPORTED
    assert lib.pw_bind_batched(ctypes.byref(ctypes.c_void_p()), 0, 1, 1.0, FAKE, 10, 4, FAKE, 12, 4, 4,
                               (pw._Op * 1)(), 0, None) == pw.PW_ERR_INVALID


def test_mean_validation_and_workspace(lib):
    """pw_mean: a null handle or an unaligned output is rejected, no rows is
    a no-op, and the workspace (a column of ones, the counts and the larger
    product workspace) grows with N + M, never with N*M; masks add the
    count product's needs, never more than one more product."""
    n = ctypes.c_size_t()
    assert lib.pw_mean_workspace_size(None, ctypes.byref(n)) == pw.PW_ERR_INVALID
    assert lib.pw_mean(None, FAKE, None, FAKE, 1 << 20, None) == pw.PW_ERR_INVALID
    rc, h = bind(lib, N=0, X=0, M=12)
    assert rc == 0 and lib.pw_mean(h, 0, None, 0, 0, None) == pw.PW_OK
    assert lib.pw_mean_workspace_size(h, ctypes.byref(n)) == pw.PW_OK and n.value == 0
    lib.pw_release(h)
    rc, h = bind(lib, N=100, M=120)
    assert lib.pw_mean(h, FAKE + 2, None, FAKE, 1 << 20, None) == pw.PW_ERR_INVALID
    assert lib.pw_mean(h, FAKE, FAKE + 2, FAKE, 1 << 20, None) == pw.PW_ERR_INVALID
    lib.pw_release(h)
    sizes = {}
    for M in (4096, 8192):
        for masked in (False, True):
            ops = [(pw.OPS["mask_columns"], 0.0, FAKE)] if masked else []
            rc, h = bind(lib, N=2048, M=M, D=8, ops=ops)
            assert rc == 0 and lib.pw_mean_workspace_size(h, ctypes.byref(n)) == pw.PW_OK
            prod = ctypes.c_size_t()
            assert lib.pw_workspace_size(h, 0, 1, 0, ctypes.byref(prod)) == pw.PW_OK
            assert n.value >= prod.value + 4 * (M + 2048)
            if not masked:
                assert n.value <= prod.value + 4 * (M + 2048) + 3 * 256
            sizes[M, masked] = n.value
            lib.pw_release(h)
    assert all(v < 2048 * M for (M, _), v in sizes.items())


def test_mmd_validation_and_workspace(lib):
    """pw_mmd2: the unbiased statistic needs two points per cloud, the
    biased one one; B in 1..65535; flags 0/1; every check precedes device
    work. The workspace holds three row-sum vectors per batch element and
    never grows with n*m."""
    n = ctypes.c_size_t()
    assert lib.pw_mmd2_workspace_size(0, 2, 1.0, 100, 80, 3, 2, None) == pw.PW_ERR_INVALID
    assert lib.pw_mmd2_workspace_size(0, 2, 1.0, 0, 80, 3, 2, ctypes.byref(n)) == pw.PW_ERR_INVALID
    assert lib.pw_mmd2_workspace_size(0, 2, 1.0, 100, 80, 3, 0, ctypes.byref(n)) == pw.PW_ERR_INVALID
    assert lib.pw_mmd2_workspace_size(0, 2, 1.0, 100, 80, 3, 65536, ctypes.byref(n)) == pw.PW_ERR_UNSUPPORTED
    assert lib.pw_mmd2_workspace_size(0, 2, 1.0, 100, 80, 65, 2, ctypes.byref(n)) == pw.PW_ERR_UNSUPPORTED
    args = lambda **kw: [kw.get(k, v) for k, v in (("dtype", 0), ("metric", 2), ("gamma", 1.0), ("X", FAKE), ("n", 100),
                         ("ldx", 3), ("sx", 300), ("Y", FAKE), ("m", 80), ("ldy", 3), ("sy", 240), ("D", 3), ("B", 2),
                         ("unbiased", 1), ("out", FAKE), ("ws", FAKE), ("wsb", 1 << 30), ("s", None))]
    assert lib.pw_mmd2(*args(n=1)) == pw.PW_ERR_INVALID          # unbiased needs two points
    assert lib.pw_mmd2(*args(unbiased=2)) == pw.PW_ERR_INVALID
    assert lib.pw_mmd2(*args(out=FAKE + 2)) == pw.PW_ERR_INVALID
    assert lib.pw_mmd2(*args(out=0)) == pw.PW_ERR_INVALID
    assert lib.pw_mmd2(*args(sx=-1)) == pw.PW_ERR_INVALID
    assert lib.pw_mmd2(*args(ldx=2)) == pw.PW_ERR_INVALID
    assert lib.pw_mmd2(*args(metric=7)) == pw.PW_ERR_INVALID
    assert lib.pw_mmd2(*args(ws=0)) == pw.PW_ERR_WORKSPACE
    sizes = []
    for m in (4096, 16384):
        assert lib.pw_mmd2_workspace_size(0, 2, 1.0, 2048, m, 3, 2, ctypes.byref(n)) == pw.PW_OK
        sizes.append(n.value)
        assert n.value >= 4 * (2 * (2048 + m + 2048))
        assert n.value < 2048 * m


def test_mmd_backward_validation(lib):
    """pw_mmd2_backward rejects what pw_mmd2 rejects, and a missing G or an
    output stride below D, before any device work; asking for neither
    gradient is a no-op."""
    n = ctypes.c_size_t()
    assert lib.pw_mmd2_backward_workspace_size(0, 2, 1.0, 100, 80, 3, ctypes.byref(n)) == pw.PW_OK and n.value > 0
    assert lib.pw_mmd2_backward_workspace_size(0, 2, 1.0, 100, 80, 3, None) == pw.PW_ERR_INVALID
    args = lambda **kw: [kw.get(k, v) for k, v in (("dtype", 0), ("metric", 2), ("gamma", 1.0), ("X", FAKE), ("n", 100),
                         ("ldx", 3), ("sx", 300), ("Y", FAKE), ("m", 80), ("ldy", 3), ("sy", 240), ("D", 3), ("B", 2),
                         ("unbiased", 1), ("G", FAKE), ("dX", FAKE), ("lddx", 3), ("dY", FAKE), ("lddy", 3),
                         ("ws", FAKE), ("wsb", 1 << 30), ("s", None))]
    assert lib.pw_mmd2_backward(*args(n=1)) == pw.PW_ERR_INVALID
    assert lib.pw_mmd2_backward(*args(G=0)) == pw.PW_ERR_INVALID
    assert lib.pw_mmd2_backward(*args(lddx=2)) == pw.PW_ERR_INVALID
    assert lib.pw_mmd2_backward(*args(lddy=2)) == pw.PW_ERR_INVALID
    assert lib.pw_mmd2_backward(*args(sy=-1)) == pw.PW_ERR_INVALID
    assert lib.pw_mmd2_backward(*args(D=65, ldx=65, ldy=65, lddx=65, lddy=65)) == pw.PW_ERR_UNSUPPORTED
    assert lib.pw_mmd2_backward(*args(ws=0)) == pw.PW_ERR_WORKSPACE
    assert lib.pw_mmd2_backward(*args(dX=0, dY=0)) == pw.PW_OK
