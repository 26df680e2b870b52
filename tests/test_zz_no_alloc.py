"""pw_topk_noalloc: the top-k entry point that allocates nothing, through the
C ABI, against pw_topk (same plan, same kernels, so the same bits).

Two calls in a row on one GPU share the library's static buffer; the second
is smaller, so it runs over what the first left there. A request larger
than the buffer is refused on the host before any device work.
"""
import ctypes

import numpy as np
import pytest
import torch

import lazy_score_matrix_amd as pw

FAKE = 0x10000  # aligned, never dereferenced


def _bind_fake(lib, N, M, D):
    h = ctypes.c_void_p()
    ops = (pw._Op * 1)()
    rc = lib.pw_bind(ctypes.byref(h), 0, 1, 1.0, FAKE, N, D, FAKE, M, D, D, ops, 0)
    assert rc == pw.PW_OK
    return h


def test_refuses_more_than_the_static_buffer():
    """Host-side: a top-64 of 2^20 queries on the matrix cores needs 1 GiB of
    partial lists, above the 64 MiB buffer: PW_ERR_SCRATCH, nothing run."""
    lib = pw.load_library()
    h = _bind_fake(lib, 1 << 20, 1 << 20, 32)
    try:
        need = ctypes.c_size_t()
        assert lib.pw_workspace_size(h, 4, 0, 64, ctypes.byref(need)) == pw.PW_OK
        assert need.value > (64 << 20)
        rc = lib.pw_topk_noalloc(h, 64, 0, FAKE, FAKE, None)
        assert rc == pw.PW_ERR_SCRATCH
        assert b"static buffer" in lib.pw_error_string(rc)
        # Invalid arguments are still reported as such.
        assert lib.pw_topk_noalloc(None, 4, 0, FAKE, FAKE, None) == pw.PW_ERR_INVALID
        assert lib.pw_topk_noalloc(h, 65, 0, FAKE, FAKE, None) == pw.PW_ERR_UNSUPPORTED
    finally:
        lib.pw_release(h)


def _data(seed, n, m, d, dtype):
    r = np.random.default_rng(seed)
    X = r.standard_normal((n, d)).astype(dtype)
    Y = r.standard_normal((m, d)).astype(dtype)
    Y[m // 2] = X[0]  # an exact copy
    return X, Y


# (seed, N, M, D, k, largest, dtype): the matrix-core search, then smaller
# calls of each engine.
CALLS = [
    (11, 1500, 5000, 32, 10, False, np.float32),
    (12, 300, 700, 32, 5, False, np.float32),
    (13, 257, 333, 3, 8, True, np.float32),
    (14, 100, 150, 16, 4, False, np.float64),
]


@pytest.mark.gpu
def test_noalloc_matches_topk_on_consecutive_calls():
    dev = torch.device("cuda:0")
    lib = pw.load_library()
    for seed, N, M, D, k, largest, dt in CALLS:
        print("case", seed, N, M, D, k, largest, dt.__name__, flush=True)
        X, Y = _data(seed, N, M, D, dt)
        e = pw.lazy(torch.from_numpy(X).to(dev), torch.from_numpy(Y).to(dev), "sqeuclidean")
        ref_v, ref_i = e.topk(k, largest)
        vals = torch.full((N, k), 7.0, dtype=e.dtype, device=dev)
        idx = torch.full((N, k), -7, dtype=torch.int64, device=dev)
        rc = lib.pw_topk_noalloc(e._h, k, int(largest), vals.data_ptr(), idx.data_ptr(),
                                 torch.cuda.current_stream(dev).cuda_stream)
        assert rc == pw.PW_OK, lib.pw_error_string(rc)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_i), "indices differ from pw_topk (case %d)" % seed
        assert torch.equal(vals, ref_v), "values differ from pw_topk (case %d)" % seed
        # The binding's method gives the same.
        v2, i2 = e.topk_noalloc(k, largest, torch.empty_like(vals), torch.empty_like(idx))
        torch.cuda.synchronize()
        assert torch.equal(i2, ref_i) and torch.equal(v2, ref_v)
