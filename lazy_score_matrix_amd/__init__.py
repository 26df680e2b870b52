"""Lazy pairwise scores reduced on the fly on an AMD Instinct MI355X.

Thin Python binding over the C ABI of ``libpw.so`` (include/pw.h): argument
marshalling only. Tensors are PyTorch device tensors; every step of the
computation runs in the library's HIP kernels on the current torch stream.
There is no CPU fallback: if the library is missing, every call raises.

    import lazy_score_matrix_amd as pw
    e = pw.lazy(Q, K, "linear", ops=[("mul", Q.shape[-1] ** -0.5)])
    out = e.softmax_matmul(V)                       # [N, C]

Op names follow the guide's "Score Expressions" section: ("mul", c),
("add", c), ("add_rows", a), ("add_columns", b), ("weight_rows", w),
("weight_columns", u), ("exp", None). Masks (``masks`` module) drop pairs
from every consumer: ("mask_rows", keep[N]), ("mask_columns", keep[M]),
("band_upper", d), ("band_lower", d), ("group_rows", g[N]),
("group_columns", g[M]), and the shorthands ("causal", d), ("band", (lo, hi))
and ("same_group", (g_rows, g_cols)).
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PW_LIBRARY names another build of libpw (e.g. one with sanitized host code).
LIB_PATH = os.environ.get("PW_LIBRARY") or os.path.join(_HERE, "libpw.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "pw.h")

PW_OK, PW_ERR_INVALID, PW_ERR_UNSUPPORTED, PW_ERR_WORKSPACE, PW_ERR_HIP, PW_ERR_SCRATCH = 0, -1, -2, -3, -4, -5
DTYPES = {torch.float32: 0, torch.float64: 1}
METRICS = {"linear": 0, "sqeuclidean": 1, "rbf": 2, "cosine_distances": 3, "cosine": 3}
OPS = {"mul": 0, "add": 1, "add_rows": 2, "add_columns": 3, "weight_rows": 4, "weight_columns": 5, "exp": 6,
       "mask_rows": 7, "mask_columns": 8, "band_upper": 9, "band_lower": 10, "group_rows": 11, "group_columns": 12}
MASK_OPS = ("mask_rows", "mask_columns", "band_upper", "band_lower", "group_rows", "group_columns")
# Row and column roles of every op, swapped by the transposed view.
_SWAP = {"add_rows": "add_columns", "add_columns": "add_rows", "weight_rows": "weight_columns",
         "weight_columns": "weight_rows", "mask_rows": "mask_columns", "mask_columns": "mask_rows",
         "band_upper": "band_lower", "band_lower": "band_upper", "group_rows": "group_columns",
         "group_columns": "group_rows"}
CONSUMERS = {"matmul": 0, "displacement": 1, "logsumexp": 2, "softmax_matmul": 3, "topk": 4}
MAX_OPS, MAX_D, MAX_K = 16, 64, 64


class PwError(RuntimeError):
    """A libpw status other than PW_OK (HIP runtime or workspace errors)."""


class _Op(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("scalar", ctypes.c_double), ("vec", ctypes.c_void_p)]


class _Batch(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("sx", ctypes.c_int64), ("sy", ctypes.c_int64), ("sv", ctypes.c_int64),
                ("op_stride", ctypes.c_int64 * 16)]


class _SolveInfo(ctypes.Structure):
    _fields_ = [("converged", ctypes.c_int), ("status", ctypes.c_int), ("iterations", ctypes.c_int),
                ("max_rel_residual", ctypes.c_double)]


SOLVE_STATUS = {0: "converged", 1: "max_iter", 2: "breakdown"}


class _GradIn(ctypes.Structure):
    _fields_ = [("G", ctypes.c_void_p), ("ldg", ctypes.c_int64), ("V", ctypes.c_void_p), ("C", ctypes.c_int64),
                ("ldv", ctypes.c_int64), ("out", ctypes.c_void_p), ("ldo", ctypes.c_int64),
                ("indices", ctypes.c_void_p), ("k", ctypes.c_int), ("exclude_self", ctypes.c_int),
                ("lse", ctypes.c_void_p)]


class _GradOut(ctypes.Structure):
    _fields_ = [("dX", ctypes.c_void_p), ("lddx", ctypes.c_int64), ("dY", ctypes.c_void_p), ("lddy", ctypes.c_int64),
                ("dV", ctypes.c_void_p), ("lddv", ctypes.c_int64), ("dops", ctypes.c_void_p * 16)]

_lock = threading.Lock()
_lib = None


def load_library(path: str = LIB_PATH):
    """Open libpw.so and declare its signatures. Raises if it is not built."""
    global _lib
    with _lock:
        if _lib is not None and path == LIB_PATH:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                "libpw.so is not built (%s); run `python -m lazy_score_matrix_amd.build` first" % path)
        lib = ctypes.CDLL(path)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        c_int = ctypes.c_int
        lib.pw_bind.argtypes = [ctypes.POINTER(vp), c_int, c_int, ctypes.c_double, vp, i64, i64, vp, i64, i64, i64,
                                ctypes.POINTER(_Op), c_int]
        lib.pw_release.argtypes = [vp]
        lib.pw_bind_batched.argtypes = [ctypes.POINTER(vp), c_int, c_int, ctypes.c_double, vp, i64, i64, vp, i64, i64,
                                        i64, ctypes.POINTER(_Op), c_int, ctypes.POINTER(_Batch)]
        lib.pw_release.restype = None
        lib.pw_workspace_size.argtypes = [vp, c_int, i64, c_int, ctypes.POINTER(sz)]
        lib.pw_matmul.argtypes = [vp, vp, i64, i64, vp, i64, vp, sz, vp]
        lib.pw_softmax_matmul.argtypes = [vp, vp, i64, i64, vp, i64, vp, sz, vp]
        lib.pw_softmax_matmul_lse.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp, sz, vp]
        lib.pw_displacement.argtypes = [vp, vp, i64, vp, sz, vp]
        lib.pw_logsumexp.argtypes = [vp, c_int, vp, vp, sz, vp]
        lib.pw_topk.argtypes = [vp, c_int, c_int, vp, vp, vp, sz, vp]
        lib.pw_topk_noalloc.argtypes = [vp, c_int, c_int, vp, vp, vp]
        lib.pw_mean_workspace_size.argtypes = [vp, ctypes.POINTER(sz)]
        lib.pw_mean.argtypes = [vp, vp, vp, vp, sz, vp]
        lib.pw_mmd2_workspace_size.argtypes = [c_int, c_int, ctypes.c_double, i64, i64, i64, i64, ctypes.POINTER(sz)]
        lib.pw_mmd2.argtypes = [c_int, c_int, ctypes.c_double, vp, i64, i64, i64, vp, i64, i64, i64, i64, i64, c_int,
                                vp, vp, sz, vp]
        lib.pw_mmd2_backward_workspace_size.argtypes = [c_int, c_int, ctypes.c_double, i64, i64, i64,
                                                        ctypes.POINTER(sz)]
        lib.pw_mmd2_backward.argtypes = [c_int, c_int, ctypes.c_double, vp, i64, i64, i64, vp, i64, i64, i64, i64,
                                         i64, c_int, vp, vp, i64, vp, i64, vp, sz, vp]
        lib.pw_plan_describe.argtypes = [vp, c_int, i64, c_int, ctypes.c_char_p, sz]
        lib.pw_backward_workspace_size.argtypes = [vp, c_int, i64, c_int, ctypes.POINTER(sz)]
        lib.pw_backward_plan_describe.argtypes = [vp, c_int, i64, c_int, ctypes.c_char_p, sz]
        lib.pw_backward.argtypes = [vp, c_int, ctypes.POINTER(_GradIn), ctypes.POINTER(_GradOut), vp, sz, vp]
        lib.pw_cg_workspace_size.argtypes = [vp, i64, ctypes.POINTER(sz)]
        lib.pw_cg_solve.argtypes = [vp, ctypes.c_double, vp, i64, i64, vp, i64, c_int, ctypes.c_double, c_int, vp, sz,
                                    vp, ctypes.POINTER(_SolveInfo)]
        lib.pw_set_tile_events.argtypes = [vp, vp]
        lib.pw_error_string.argtypes = [c_int]
        lib.pw_error_string.restype = ctypes.c_char_p
        if path == LIB_PATH:
            _lib = lib
        return lib


def header_functions(header: str = HEADER):
    """Names of the functions include/pw.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|void|const char \*)\s*(pw_\w+)\s*\(", text, flags=re.M)))


def check(rc: int, what: str = "") -> None:
    if rc == PW_OK:
        return
    msg = "%s: %s (%d)" % (what, load_library().pw_error_string(rc).decode(), rc)
    if rc == PW_ERR_INVALID:
        raise ValueError(msg)
    if rc == PW_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise PwError(msg)


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def expand_ops(ops):
    """Op list with the mask shorthands causal / band / same_group expanded."""
    out = []
    for op in ops:
        name, arg = op
        if name == "causal":
            out.append(("band_upper", 0 if arg is None else int(arg)))
        elif name == "band":
            out += [("band_lower", int(arg[0])), ("band_upper", int(arg[1]))]
        elif name == "same_group":
            out += [("group_rows", arg[0]), ("group_columns", arg[1])]
        else:
            out.append((name, arg))
    return out


def _rows(t, name):
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    if t.numel() == 0 or t.shape[0] == 1:
        return max(t.shape[1], 1)
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError("%s must have unit column stride" % name)
    return t.stride(0)


class LazyScores:
    """A bound lazy score matrix S[i, j] = ops(f(x_i, y_j)) (never stored)."""

    def __init__(self, X: torch.Tensor, Y: torch.Tensor, metric: str = "linear", gamma: float = 1.0, ops=()):
        lib = load_library()
        if X.dtype not in DTYPES or Y.dtype != X.dtype:
            raise TypeError("X and Y must both be float32 or both float64")
        if not X.is_cuda or Y.device != X.device:
            raise ValueError("X and Y must be on the same GPU")
        if metric not in METRICS:
            raise ValueError("unknown metric %r" % metric)
        self.X, self.Y, self.metric, self.gamma = X, Y, metric, float(gamma)
        self.N, self.D = X.shape
        self.M = Y.shape[0]
        self.dtype, self.device = X.dtype, X.device
        if Y.shape[1] != self.D:
            raise ValueError("X and Y feature dims differ")
        ldx, ldy = _rows(X, "X"), _rows(Y, "Y")
        self._keep = []
        ops = expand_ops(ops)
        arr = (_Op * max(len(ops), 1))()
        for t, (name, arg) in enumerate(ops):
            if name not in OPS:
                raise ValueError("unknown op %r" % name)
            arr[t].kind = OPS[name]
            if name in ("mul", "add", "band_upper", "band_lower"):
                arr[t].scalar = float(arg)
            elif name in ("mask_rows", "mask_columns", "group_rows", "group_columns"):
                v = arg
                n = self.N if name.endswith("_rows") else self.M
                want = (torch.bool, torch.uint8) if name.startswith("mask") else (torch.int64,)
                if (not torch.is_tensor(v) or v.dtype not in want or v.device != self.device or v.numel() != n
                        or not v.is_contiguous()):
                    raise ValueError("%s needs a contiguous %s vector of %d elements on %s"
                                     % (name, " or ".join(str(w) for w in want), n, self.device))
                self._keep.append(v)
                arr[t].vec = v.data_ptr()
            elif name != "exp":
                v = arg
                n = self.N if name.endswith("_rows") else self.M
                if (not torch.is_tensor(v) or v.dtype != self.dtype or v.device != self.device
                        or v.numel() != n or not v.is_contiguous()):
                    raise ValueError("%s needs a contiguous %s vector of %d elements on %s"
                                     % (name, self.dtype, n, self.device))
                self._keep.append(v)
                arr[t].vec = v.data_ptr()
        self.ops = ops
        h = ctypes.c_void_p()
        check(lib.pw_bind(ctypes.byref(h), DTYPES[X.dtype], METRICS[metric], self.gamma, X.data_ptr(), self.N, ldx,
                          Y.data_ptr(), self.M, ldy, self.D, arr, len(ops)), "pw_bind")
        self._h = h
        self._lib = lib

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pw_release(h)
            self._h = None

    # -- workspace -----------------------------------------------------
    def workspace_size(self, consumer: str, C: int = 0, k: int = 0) -> int:
        n = ctypes.c_size_t()
        check(self._lib.pw_workspace_size(self._h, CONSUMERS[consumer], int(C), int(k), ctypes.byref(n)),
              "pw_workspace_size")
        return n.value

    def workspace(self, consumer: str, C: int = 0, k: int = 0) -> torch.Tensor:
        return torch.empty(max(self.workspace_size(consumer, C, k), 1), dtype=torch.uint8, device=self.device)

    def plan(self, consumer: str, C: int = 0, k: int = 0) -> str:
        buf = ctypes.create_string_buffer(512)
        check(self._lib.pw_plan_describe(self._h, CONSUMERS[consumer], int(C), int(k), buf, 512), "pw_plan_describe")
        return buf.value.decode()

    def _ws(self, ws, consumer, C=0, k=0):
        if ws is None:
            ws = self.workspace(consumer, C, k)
        return ws, ws.numel() * ws.element_size()

    def _value(self, V, what):
        if V.dtype != self.dtype or V.device != self.device or V.shape[0] != self.M:
            raise ValueError("V must be [M, C] %s on %s" % (self.dtype, self.device))
        return _rows(V, "V")

    # -- consumers ------------------------------------------------------
    def matmul(self, V: torch.Tensor, out=None, workspace=None, mask=None) -> torch.Tensor:
        """out[i, c] = sum_j S[i, j] V[j, c] over the kept pairs."""
        if mask is not None:
            return self.masked(mask).matmul(V, out, workspace)
        if out is None and _needs_grad(self, V):
            return _replay(self, "matmul", V)
        ldv = self._value(V, "matmul")
        C = V.shape[1]
        out = torch.empty(self.N, C, dtype=self.dtype, device=self.device) if out is None else out
        ws, nb = self._ws(workspace, "matmul", C)
        check(self._lib.pw_matmul(self._h, V.data_ptr(), C, ldv, out.data_ptr(), _rows(out, "out"), ws.data_ptr(),
                                  nb, _stream(self.device)), "pw_matmul")
        return out

    __matmul__ = matmul

    def softmax_matmul(self, V: torch.Tensor, out=None, workspace=None, mask=None, lse=None) -> torch.Tensor:
        """out[i, c] = sum_j softmax_j(S[i, :])[j] V[j, c], over the pairs
        `mask` (op entries, e.g. masks.causal()) and the bound masks keep.
        With `lse` (an [N] tensor) each row's log-sum-exp is written too."""
        if mask is not None:
            return self.masked(mask).softmax_matmul(V, out, workspace, lse=lse)
        if out is None and lse is None and _needs_grad(self, V):
            return _replay(self, "softmax_matmul", V)
        ldv = self._value(V, "softmax_matmul")
        C = V.shape[1]
        out = torch.empty(self.N, C, dtype=self.dtype, device=self.device) if out is None else out
        ws, nb = self._ws(workspace, "softmax_matmul", C)
        if lse is None:
            check(self._lib.pw_softmax_matmul(self._h, V.data_ptr(), C, ldv, out.data_ptr(), _rows(out, "out"),
                                              ws.data_ptr(), nb, _stream(self.device)), "pw_softmax_matmul")
        else:
            if lse.dtype != self.dtype or lse.device != self.device or lse.numel() != self.N or not lse.is_contiguous():
                raise ValueError("lse must be a contiguous [N] %s tensor on %s" % (self.dtype, self.device))
            check(self._lib.pw_softmax_matmul_lse(self._h, V.data_ptr(), C, ldv, out.data_ptr(), _rows(out, "out"),
                                                  lse.data_ptr(), ws.data_ptr(), nb, _stream(self.device)),
                  "pw_softmax_matmul_lse")
        return out

    def displacement(self, out=None, workspace=None, mask=None) -> torch.Tensor:
        """out[i, d] = sum_j S[i, j] (Y[j, d] - X[i, d]) over the kept pairs."""
        if mask is not None:
            return self.masked(mask).displacement(out, workspace)
        if out is None and _needs_grad(self):
            return _replay(self, "displacement")
        out = torch.empty(self.N, self.D, dtype=self.dtype, device=self.device) if out is None else out
        ws, nb = self._ws(workspace, "displacement")
        check(self._lib.pw_displacement(self._h, out.data_ptr(), _rows(out, "out"), ws.data_ptr(), nb,
                                        _stream(self.device)), "pw_displacement")
        return out

    def logsumexp(self, exclude_self: bool = False, out=None, workspace=None, mask=None) -> torch.Tensor:
        """out[i] = log sum_j exp(S[i, j]) over the kept pairs, optionally
        without j == i (-inf for a row with none)."""
        if mask is not None:
            return self.masked(mask).logsumexp(exclude_self, out, workspace)
        if out is None and _needs_grad(self):
            return _replay(self, "logsumexp", exclude_self=bool(exclude_self))
        out = torch.empty(self.N, dtype=self.dtype, device=self.device) if out is None else out
        ws, nb = self._ws(workspace, "logsumexp")
        check(self._lib.pw_logsumexp(self._h, int(bool(exclude_self)), out.data_ptr(), ws.data_ptr(), nb,
                                     _stream(self.device)), "pw_logsumexp")
        return out

    def topk(self, k: int, largest: bool = False, values=None, indices=None, workspace=None, mask=None):
        """The k first kept pairs of each row by (value, index): values and
        int64 indices [N, k]; positions past a row's kept pairs hold NaN / -1."""
        if mask is not None:
            return self.masked(mask).topk(k, largest, values, indices, workspace)
        if values is None and _needs_grad(self):
            return _replay(self, "topk", k=int(k), largest=bool(largest))
        values = torch.empty(self.N, k, dtype=self.dtype, device=self.device) if values is None else values
        indices = torch.empty(self.N, k, dtype=torch.int64, device=self.device) if indices is None else indices
        ws, nb = self._ws(workspace, "topk", 0, k)
        check(self._lib.pw_topk(self._h, int(k), int(bool(largest)), values.data_ptr(), indices.data_ptr(),
                                ws.data_ptr(), nb, _stream(self.device)), "pw_topk")
        return values, indices

    def topk_noalloc(self, k: int, largest: bool, values: torch.Tensor, indices: torch.Tensor):
        """topk into the caller's values [N, k] and int64 indices [N, k]
        through pw_topk_noalloc: no workspace, no allocation (the library's
        static device buffer serves instead; calls on one GPU must not
        overlap)."""
        if values.shape != (self.N, k) or indices.shape != (self.N, k) or not values.is_contiguous() or \
                not indices.is_contiguous() or values.dtype != self.dtype or indices.dtype != torch.int64:
            raise ValueError("values and indices must be contiguous [N, k] tensors of the bound dtype and int64")
        check(self._lib.pw_topk_noalloc(self._h, int(k), int(bool(largest)), values.data_ptr(), indices.data_ptr(),
                                        _stream(self.device)), "pw_topk_noalloc")
        return values, indices

    # -- backward -------------------------------------------------------
    def backward(self, consumer: str, G: torch.Tensor, V=None, out=None, indices=None, exclude_self=False,
                 want=("X", "Y", "V", "ops"), grads=None, workspace=None, lse=None):
        """Gradients of sum(consumer output * G) by replay (guide: backward
        re-evaluates the pairs; selections route gradients through the
        selected pairs only). Returns {"X": dX, "Y": dY, "V": dV, "ops": [per
        op: gradient of its vector or None]}; only the entries in `want` are
        computed. `out` is the forward output (softmax_matmul: required;
        logsumexp: optional), `indices` the top-k indices."""
        G2 = G[:, None] if G.dim() == 1 else G
        if G2.dtype != self.dtype or G2.device != self.device or G2.shape[0] != self.N:
            raise ValueError("G must be [N, *] %s on %s" % (self.dtype, self.device))
        gin = _GradIn()
        gin.G, gin.ldg = G2.data_ptr(), _rows(G2, "G")
        keep = [G2]
        if V is not None:
            gin.V, gin.C, gin.ldv = V.data_ptr(), V.shape[1], self._value(V, "backward")
        if out is not None:
            o2 = out[:, None] if out.dim() == 1 else out
            gin.out, gin.ldo = o2.data_ptr(), _rows(o2, "out")
            keep.append(o2)
        if indices is not None:
            idx = indices.contiguous()
            keep.append(idx)
            gin.indices, gin.k = idx.data_ptr(), idx.shape[1]
        gin.exclude_self = int(bool(exclude_self))
        if lse is not None:
            gin.lse = lse.data_ptr()
            keep.append(lse)
        res = {"X": None, "Y": None, "V": None, "ops": [None] * len(self.ops)}
        gout = _GradOut()
        given = grads or {}

        def new(*shape, key=None):
            if key in given:
                return given[key]
            return torch.empty(*shape, dtype=self.dtype, device=self.device)
        if "X" in want:
            res["X"] = new(self.N, self.D, key="X")
            gout.dX, gout.lddx = res["X"].data_ptr(), max(self.D, 1)
        if "Y" in want:
            res["Y"] = new(self.M, self.D, key="Y")
            gout.dY, gout.lddy = res["Y"].data_ptr(), max(self.D, 1)
        if "V" in want and V is not None:
            res["V"] = new(self.M, V.shape[1], key="V")
            gout.dV, gout.lddv = res["V"].data_ptr(), V.shape[1]
        if "ops" in want:
            for t, (name, arg) in enumerate(self.ops):
                if name in ("add_rows", "weight_rows", "add_columns", "weight_columns"):
                    res["ops"][t] = new(self.N if name.endswith("_rows") else self.M)
                    gout.dops[t] = res["ops"][t].data_ptr()
        C = V.shape[1] if V is not None else 0
        n = ctypes.c_size_t()
        check(self._lib.pw_backward_workspace_size(self._h, CONSUMERS[consumer], C, gin.k, ctypes.byref(n)),
              "pw_backward_workspace_size")
        ws = workspace if workspace is not None else torch.empty(max(n.value, 1), dtype=torch.uint8,
                                                                 device=self.device)
        if ws.numel() < n.value:
            raise ValueError("workspace needs %d bytes" % n.value)
        check(self._lib.pw_backward(self._h, CONSUMERS[consumer], ctypes.byref(gin), ctypes.byref(gout),
                                    ws.data_ptr(), ws.numel(), _stream(self.device)), "pw_backward")
        return res

    def backward_plan(self, consumer: str, C: int = 0, want_ops: bool = False) -> str:
        buf = ctypes.create_string_buffer(256)
        check(self._lib.pw_backward_plan_describe(self._h, CONSUMERS[consumer], int(C), int(bool(want_ops)), buf, 256),
              "pw_backward_plan_describe")
        return buf.value.decode()

    def backward_workspace(self, consumer: str, C: int = 0, k: int = 0) -> torch.Tensor:
        n = ctypes.c_size_t()
        check(self._lib.pw_backward_workspace_size(self._h, CONSUMERS[consumer], int(C), int(k), ctypes.byref(n)),
              "pw_backward_workspace_size")
        return torch.empty(max(n.value, 1), dtype=torch.uint8, device=self.device)

    # -- solver ---------------------------------------------------------
    def solve(self, B: torch.Tensor, shift: float, rtol: float = 1e-6, max_iter: int = 1000, check_every: int = 8,
              out=None, workspace=None):
        """Conjugate-gradient solution A of (S + shift I) A = B for a square,
        symmetric positive semi-definite score (Task Map, Kernel ridge / GP
        mean row). Returns (A, info) with info's converged, status
        ("converged", "max_iter" or "breakdown"), iterations and
        max_rel_residual; check them before using A."""
        vec = B.dim() == 1
        B2 = B[:, None] if vec else B
        ldb = self._value(B2, "solve")
        C = B2.shape[1]
        A = torch.empty(self.N, C, dtype=self.dtype, device=self.device) if out is None else out
        if workspace is None:
            n = ctypes.c_size_t()
            check(self._lib.pw_cg_workspace_size(self._h, C, ctypes.byref(n)), "pw_cg_workspace_size")
            workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=self.device)
        info = _SolveInfo()
        check(self._lib.pw_cg_solve(self._h, float(shift), B2.data_ptr(), C, ldb, A.data_ptr(), _rows(A, "out"),
                                    int(max_iter), float(rtol), int(check_every), workspace.data_ptr(),
                                    workspace.numel(), _stream(self.device), ctypes.byref(info)), "pw_cg_solve")
        res = {"converged": bool(info.converged), "status": SOLVE_STATUS[info.status],
               "iterations": int(info.iterations), "max_rel_residual": float(info.max_rel_residual)}
        return (A[:, 0] if vec and out is None else A), res

    # -- views and derived reductions ----------------------------------
    def masked(self, mask) -> "LazyScores":
        """This score with more masks (op entries from the masks module)."""
        mask = [mask] if isinstance(mask, tuple) else list(mask)
        return LazyScores(self.X, self.Y, self.metric, self.gamma, list(self.ops) + mask)

    def mask_rows(self, keep) -> "LazyScores":
        return self.masked([("mask_rows", keep)])

    def mask_columns(self, keep) -> "LazyScores":
        return self.masked([("mask_columns", keep)])

    @property
    def T(self) -> "LazyScores":
        """The transposed score S^T[j, i] = S[i, j] (Y and X swapped, row and
        column ops and masks swapped; every built-in metric is symmetric).
        Column reductions such as min(-2) are row reductions of this view."""
        ops = [(_SWAP.get(n, n), a) for n, a in self.ops]
        return LazyScores(self.Y, self.X, self.metric, self.gamma, ops)

    def min(self, dim: int = -1):
        """Minimum over `dim` and its (lowest) index: top-k with k = 1 (Task
        Map, Chamfer row: D.min(-1) and D.min(-2))."""
        if dim in (-2, 0):
            return self.T.min(-1)
        v, i = self.topk(1)
        return v[:, 0], i[:, 0]

    def argmin(self, dim: int = -1):
        return self.min(dim)[1]

    def max(self, dim: int = -1):
        if dim in (-2, 0):
            return self.T.max(-1)
        v, i = self.topk(1, largest=True)
        return v[:, 0], i[:, 0]

    def sum(self, dim: int = -1) -> torch.Tensor:
        """Sum over `dim`: the kernel product with a column of ones."""
        if dim in (-2, 0):
            return self.T.sum(-1)
        ones = torch.ones(self.M, 1, dtype=self.dtype, device=self.device)
        return self.matmul(ones)[:, 0]

    def mean(self, dim: int = -1, inv_counts=None) -> torch.Tensor:
        """Mean over `dim` of the kept pairs (Features page, Native
        Deployment: reduce("mean", -1)); NaN for a row with none (pw_mean).
        With `inv_counts` (an [N] tensor) each row's 1 / kept count is
        written too. Under autograd the value still comes from pw_mean, and
        the backward replays the sum product weighted by those inverse
        counts."""
        if dim in (-2, 0):
            return self.T.mean(-1, inv_counts)
        if inv_counts is None and _needs_grad(self):
            return _replay(self, "mean")
        out = torch.empty(self.N, dtype=self.dtype, device=self.device)
        if inv_counts is not None and (inv_counts.dtype != self.dtype or inv_counts.device != self.device
                                       or inv_counts.numel() != self.N or not inv_counts.is_contiguous()):
            raise ValueError("inv_counts must be a contiguous [N] %s tensor on %s" % (self.dtype, self.device))
        n = ctypes.c_size_t()
        check(self._lib.pw_mean_workspace_size(self._h, ctypes.byref(n)), "pw_mean_workspace_size")
        ws = torch.empty(max(n.value, 1), dtype=torch.uint8, device=self.device)
        check(self._lib.pw_mean(self._h, out.data_ptr(), None if inv_counts is None else inv_counts.data_ptr(),
                                ws.data_ptr(), n.value, _stream(self.device)), "pw_mean")
        return out


from . import masks  # noqa: E402  (pair-mask helpers)

_VEC_OPS = ("add_rows", "weight_rows", "add_columns", "weight_columns")


class _Replay(torch.autograd.Function):
    """A consumer call whose backward replays the pairs with pw_backward.
    Inputs: a spec tuple, then X, Y, V (or None) and every op argument that
    is a tensor (op vectors, masks, group ids), in op order."""

    @staticmethod
    def forward(ctx, spec, X, Y, V, *tensors):
        metric, gamma, ops_spec, consumer, kw = spec
        it = iter(tensors)
        ops = [(n, next(it) if is_t else a) for n, a, is_t in ops_spec]
        e = LazyScores(X, Y, metric, gamma, ops)
        lse = torch.empty(0)
        if consumer == "softmax_matmul":
            lse = torch.empty(e.N, dtype=e.dtype, device=e.device)
            out = e.softmax_matmul(V, lse=lse)
            outs = (out,)
        elif consumer == "matmul":
            out = e.matmul(V)
            outs = (out,)
        elif consumer == "displacement":
            out = e.displacement()
            outs = (out,)
        elif consumer == "logsumexp":
            out = e.logsumexp(kw.get("exclude_self", False))
            outs = (out,)
        elif consumer == "mean":
            V = torch.empty(e.N, dtype=e.dtype, device=e.device)  # the rows' inverse kept counts
            out = e.mean(-1, inv_counts=V)
            outs = (out,)
        else:
            vals, idx = e.topk(kw["k"], kw.get("largest", False))
            ctx.mark_non_differentiable(idx)
            outs = (vals, idx)
            out = vals
        ctx.spec = spec
        ctx.save_for_backward(X, Y, V if V is not None else torch.empty(0), out, outs[-1], lse, *tensors)
        ctx.has_v = V is not None
        return outs if len(outs) > 1 else outs[0]

    @staticmethod
    def _mean_backward(ctx, e, G, inv, want):
        """The mean is the sum product of the scores weighted by the rows'
        inverse kept counts: replay that product's backward."""
        we = LazyScores(e.X, e.Y, e.metric, e.gamma, list(e.ops) + [("weight_rows", inv)])
        ones = torch.ones(e.M, 1, dtype=e.dtype, device=e.device)
        return we.backward("matmul", G.reshape(-1, 1).contiguous(), V=ones, want=tuple(want))

    @staticmethod
    def backward(ctx, *grads):
        metric, gamma, ops_spec, consumer, kw = ctx.spec
        X, Y, V, out, last, lse, *tensors = ctx.saved_tensors
        V = V if ctx.has_v else None
        it = iter(tensors)
        ops = [(n, next(it) if is_t else a) for n, a, is_t in ops_spec]
        e = LazyScores(X, Y, metric, gamma, ops)
        G = grads[0].contiguous()
        want = ["ops"]
        if ctx.needs_input_grad[1]:
            want.append("X")
        if ctx.needs_input_grad[2]:
            want.append("Y")
        if ctx.needs_input_grad[3] and consumer != "mean":
            want.append("V")
        if consumer == "mean":
            r = _Replay._mean_backward(ctx, e, G, V, want)
            r = dict(r, V=None)
        else:
            r = e.backward(consumer, G, V=V, out=out if consumer in ("softmax_matmul", "logsumexp") else None,
                           indices=last if consumer == "topk" else None, exclude_self=kw.get("exclude_self", False),
                           want=tuple(want), lse=lse if consumer == "softmax_matmul" else None)
        op_grads = []
        for t, (n, a, is_t) in enumerate(ops_spec):
            if is_t:
                op_grads.append(r["ops"][t] if n in _VEC_OPS else None)
        return (None, r["X"], r["Y"], r["V"], *op_grads)


def _needs_grad(e, V=None):
    if not torch.is_grad_enabled():
        return False
    ts = [e.X, e.Y] + ([V] if V is not None else []) + [a for n, a in e.ops if torch.is_tensor(a)]
    return any(t.requires_grad for t in ts)


def _replay(e, consumer, V=None, **kw):
    ops_spec = tuple((n, None if torch.is_tensor(a) else a, torch.is_tensor(a)) for n, a in e.ops)
    tensors = [a for n, a in e.ops if torch.is_tensor(a)]
    spec = (e.metric, e.gamma, ops_spec, consumer, kw)
    return _Replay.apply(spec, e.X, e.Y, V, *tensors)


class BatchedLazyScores:
    """Lazy scores over leading batch dimensions (Task Map, MMD row: one
    feature set per batch element; the Features page: a [1, N, *] input
    compares against every element of a [B, M, *] input). X is [B or 1,
    N, D], Y is [B or 1, M, D]; op vectors are either shared ([N] / [M]) or
    per element ([B, N] / [B, M]); masks are shared. A forward consumer call
    binds the whole batch (pw_bind_batched) and runs every element in one
    launch; outputs stack along a leading B axis. Calls that need autograd,
    per-element masks or the backward run element by element (each element
    a LazyScores; the slices carry autograd)."""

    def __init__(self, X, Y, metric="linear", gamma=1.0, ops=()):
        if X.dim() != 3 or Y.dim() != 3:
            raise ValueError("batched scores need [B, N, D] and [B, M, D] inputs")
        bx, by = X.shape[0], Y.shape[0]
        if bx != by and 1 not in (bx, by):
            raise ValueError("batch sizes %d and %d do not broadcast" % (bx, by))
        self.B = max(bx, by)
        self.X, self.Y, self.metric, self.gamma = X, Y, metric, float(gamma)
        self.ops = expand_ops(ops)
        self.N, self.M, self.D = X.shape[1], Y.shape[1], X.shape[2]
        self.dtype, self.device = X.dtype, X.device

    def element(self, b: int) -> LazyScores:
        X = self.X[b if self.X.shape[0] > 1 else 0]
        Y = self.Y[b if self.Y.shape[0] > 1 else 0]
        ops = []
        for n, a in self.ops:
            if torch.is_tensor(a) and a.dim() == 2:  # per-element vector [B, len]
                a = a[b]
            ops.append((n, a))
        return LazyScores(X, Y, self.metric, self.gamma, ops)

    # -- one launch for the whole batch ----------------------------------
    def _stride(self, t, what):
        """Elements between consecutive batch elements of t [B or 1, ...]
        (0 for a single shared one); rows of each element must be laid out
        with unit column stride."""
        if t.shape[0] == 1:
            return 0
        return t.stride(0)

    def _batched_ok(self, V=None):
        if _needs_grad(self, V):
            return False
        for n, a in self.ops:
            if n in MASK_OPS and torch.is_tensor(a) and a.dim() != 1:
                return False  # masks are shared by the batch
        return True

    def _bind(self, V=None):
        """A pw_expr over the whole batch, and the tensors it borrows."""
        lib = load_library()
        X, Y = self.X, self.Y
        if X.dtype not in DTYPES or Y.dtype != X.dtype or not X.is_cuda or Y.device != X.device:
            raise ValueError("X and Y must be float32 or float64 tensors on one GPU")
        ldx, ldy = _rows(X[0], "X"), _rows(Y[0], "Y")
        bt = _Batch()
        bt.B = self.B
        bt.sx, bt.sy = self._stride(X, "X"), self._stride(Y, "Y")
        bt.sv = 0 if V is None or V.dim() == 2 else self._stride(V, "V")
        keep = [X, Y]
        arr = (_Op * max(len(self.ops), 1))()
        for t, (name, arg) in enumerate(self.ops):
            arr[t].kind = OPS[name]
            if name in ("mul", "add", "band_upper", "band_lower"):
                arr[t].scalar = float(arg)
            elif name != "exp":
                n = self.N if name.endswith("_rows") else self.M
                v = arg
                per = v.dim() == 2
                if name in MASK_OPS:
                    want = (torch.bool, torch.uint8) if name.startswith("mask") else (torch.int64,)
                else:
                    want = (self.dtype,)
                if (v.dtype not in want or v.device != self.device or v.shape[-1] != n or v.stride(-1) != 1
                        or (per and v.shape[0] not in (1, self.B))):
                    raise ValueError("%s needs a %s vector of %d elements (or [B, %d]) on %s"
                                     % (name, " or ".join(str(w) for w in want), n, n, self.device))
                arr[t].vec = v.data_ptr()
                bt.op_stride[t] = v.stride(0) if per and v.shape[0] > 1 else 0
                keep.append(v)
        h = ctypes.c_void_p()
        check(lib.pw_bind_batched(ctypes.byref(h), DTYPES[X.dtype], METRICS[self.metric], self.gamma, X.data_ptr(),
                                  self.N, ldx, Y.data_ptr(), self.M, ldy, self.D, arr, len(self.ops),
                                  ctypes.byref(bt)), "pw_bind_batched")
        return _Handle(lib, h, keep)

    def plan(self, consumer: str, C: int = 0, k: int = 0) -> str:
        """The batched launch plan of a consumer (pw_plan_describe)."""
        return self._bind().plan(consumer, C, k)

    def _V3(self, V):
        V3 = V if V.dim() == 3 else V[None]
        if V3.dtype != self.dtype or V3.device != self.device or V3.shape[1] != self.M or \
                V3.shape[0] not in (1, self.B):
            raise ValueError("V must be [B or 1, M, C] (or [M, C]) %s on %s" % (self.dtype, self.device))
        return V3

    def _value_consumer(self, name, V):
        V3 = self._V3(V)
        h = self._bind(V)
        C = V3.shape[2]
        out = torch.empty(self.B, self.N, C, dtype=self.dtype, device=self.device)
        ws, nb = h.workspace(name, C)
        fn = h.lib.pw_matmul if name == "matmul" else h.lib.pw_softmax_matmul
        check(fn(h.h, V3.data_ptr(), C, _rows(V3[0], "V"), out.data_ptr(), C, ws.data_ptr(), nb,
                 _stream(self.device)), "pw_" + name)
        return out

    def _each(self, fn):
        outs = [fn(self.element(b)) for b in range(self.B)]
        if isinstance(outs[0], tuple):
            return tuple(torch.stack(parts) for parts in zip(*outs))
        return torch.stack(outs)

    def _V(self, V, b):
        return V[b if V.shape[0] > 1 else 0] if V.dim() == 3 else V

    def matmul(self, V, mask=None):
        if mask is not None:
            return self.masked(mask).matmul(V)
        if self._batched_ok(V):
            return self._value_consumer("matmul", V)
        return torch.stack([self.element(b).matmul(self._V(V, b)) for b in range(self.B)])

    __matmul__ = matmul

    def softmax_matmul(self, V, mask=None):
        if mask is not None:
            return self.masked(mask).softmax_matmul(V)
        if self._batched_ok(V):
            return self._value_consumer("softmax_matmul", V)
        return torch.stack([self.element(b).softmax_matmul(self._V(V, b)) for b in range(self.B)])

    def displacement(self, mask=None):
        if mask is not None:
            return self.masked(mask).displacement()
        if not self._batched_ok():
            return self._each(lambda e: e.displacement())
        h = self._bind()
        out = torch.empty(self.B, self.N, self.D, dtype=self.dtype, device=self.device)
        ws, nb = h.workspace("displacement")
        check(h.lib.pw_displacement(h.h, out.data_ptr(), self.D, ws.data_ptr(), nb, _stream(self.device)),
              "pw_displacement")
        return out

    def logsumexp(self, exclude_self=False, mask=None):
        if mask is not None:
            return self.masked(mask).logsumexp(exclude_self)
        if not self._batched_ok():
            return self._each(lambda e: e.logsumexp(exclude_self))
        h = self._bind()
        out = torch.empty(self.B, self.N, dtype=self.dtype, device=self.device)
        ws, nb = h.workspace("logsumexp")
        check(h.lib.pw_logsumexp(h.h, int(bool(exclude_self)), out.data_ptr(), ws.data_ptr(), nb,
                                 _stream(self.device)), "pw_logsumexp")
        return out

    def topk(self, k, largest=False, mask=None):
        if mask is not None:
            return self.masked(mask).topk(k, largest)
        if not self._batched_ok():
            return self._each(lambda e: e.topk(k, largest))
        h = self._bind()
        vals = torch.empty(self.B, self.N, k, dtype=self.dtype, device=self.device)
        idx = torch.empty(self.B, self.N, k, dtype=torch.int64, device=self.device)
        ws, nb = h.workspace("topk", 0, k)
        check(h.lib.pw_topk(h.h, int(k), int(bool(largest)), vals.data_ptr(), idx.data_ptr(), ws.data_ptr(), nb,
                            _stream(self.device)), "pw_topk")
        return vals, idx

    def min(self, dim=-1):
        if dim in (-2, 1):
            return self.T.min(-1)
        v, i = self.topk(1)
        return v[..., 0], i[..., 0]

    def max(self, dim=-1):
        if dim in (-2, 1):
            return self.T.max(-1)
        v, i = self.topk(1, largest=True)
        return v[..., 0], i[..., 0]

    def argmin(self, dim=-1):
        return self.min(dim)[1]

    def sum(self, dim=-1):
        """Sum over `dim`: the product with a column of ones."""
        if dim in (-2, 1):
            return self.T.sum(-1)
        ones = torch.ones(self.M, 1, dtype=self.dtype, device=self.device)
        return self.matmul(ones)[..., 0]

    def mean(self, dim=-1):
        """Mean over `dim` of the kept pairs, NaN for a row with none: one
        pw_mean call for the whole batch (element by element under autograd
        or with per-element masks)."""
        if dim in (-2, 1):
            return self.T.mean(-1)
        if not self._batched_ok():
            return self._each(lambda e: e.mean(-1))
        h = self._bind()
        out = torch.empty(self.B, self.N, dtype=self.dtype, device=self.device)
        n = ctypes.c_size_t()
        check(h.lib.pw_mean_workspace_size(h.h, ctypes.byref(n)), "pw_mean_workspace_size")
        ws = torch.empty(max(n.value, 1), dtype=torch.uint8, device=self.device)
        check(h.lib.pw_mean(h.h, out.data_ptr(), None, ws.data_ptr(), n.value, _stream(self.device)), "pw_mean")
        return out

    def masked(self, mask):
        mask = [mask] if isinstance(mask, tuple) else list(mask)
        return BatchedLazyScores(self.X, self.Y, self.metric, self.gamma, list(self.ops) + mask)

    @property
    def T(self):
        ops = [(_SWAP.get(n, n), a) for n, a in self.ops]
        return BatchedLazyScores(self.Y, self.X, self.metric, self.gamma, ops)


class _Handle:
    """A bound pw_expr that owns its handle and keeps the tensors it
    borrows alive."""

    def __init__(self, lib, h, keep):
        self.lib, self.h, self._keep = lib, h, keep
        self.device = keep[0].device

    def __del__(self):
        if self.h is not None and self.h.value:
            self.lib.pw_release(self.h)
            self.h = None

    def plan(self, consumer, C=0, k=0):
        buf = ctypes.create_string_buffer(512)
        check(self.lib.pw_plan_describe(self.h, CONSUMERS[consumer], int(C), int(k), buf, 512), "pw_plan_describe")
        return buf.value.decode()

    def workspace(self, consumer, C=0, k=0):
        n = ctypes.c_size_t()
        check(self.lib.pw_workspace_size(self.h, CONSUMERS[consumer], int(C), int(k), ctypes.byref(n)),
              "pw_workspace_size")
        ws = torch.empty(max(n.value, 1), dtype=torch.uint8, device=self.device)
        return ws, n.value


def lazy(X, Y=None, metric: str = "linear", gamma: float = 1.0, ops=()):
    """Bind S[i, j] = ops(metric(X[i], Y[j])); Y defaults to X. Inputs with
    a leading batch axis ([B, N, D]) give a BatchedLazyScores."""
    Y = X if Y is None else Y
    if X.dim() == 3 or Y.dim() == 3:
        return BatchedLazyScores(X if X.dim() == 3 else X[None], Y if Y.dim() == 3 else Y[None], metric, gamma, ops)
    return LazyScores(X, Y, metric, gamma, ops)


def _mmd_args(X3, Y3, kernel):
    if X3.dim() != 3 or Y3.dim() != 3 or X3.shape[2] != Y3.shape[2]:
        raise ValueError("clouds must be [B, n, D] and [B or 1, m, D]")
    if X3.dtype not in DTYPES or Y3.dtype != X3.dtype or not X3.is_cuda or Y3.device != X3.device:
        raise ValueError("X and Y must be float32 or float64 tensors on one GPU")
    if kernel not in METRICS:
        raise ValueError("unknown kernel %r" % kernel)
    B = max(X3.shape[0], Y3.shape[0])
    if X3.shape[0] not in (1, B) or Y3.shape[0] not in (1, B):
        raise ValueError("batch sizes %d and %d do not broadcast" % (X3.shape[0], Y3.shape[0]))
    sx = 0 if X3.shape[0] == 1 else X3.stride(0)
    sy = 0 if Y3.shape[0] == 1 else Y3.stride(0)
    return B, X3.shape[1], Y3.shape[1], X3.shape[2], sx, sy, DTYPES[X3.dtype], METRICS[kernel]


class _Mmd(torch.autograd.Function):
    """pw_mmd2 forward; pw_mmd2_backward for the clouds' gradients."""

    @staticmethod
    def forward(ctx, X3, Y3, kernel, gamma, unbiased):
        lib = load_library()
        B, n, m, D, sx, sy, dt, mt = _mmd_args(X3, Y3, kernel)
        nb = ctypes.c_size_t()
        check(lib.pw_mmd2_workspace_size(dt, mt, float(gamma), n, m, D, B, ctypes.byref(nb)), "pw_mmd2_workspace_size")
        ws = torch.empty(max(nb.value, 1), dtype=torch.uint8, device=X3.device)
        out = torch.empty(B, dtype=X3.dtype, device=X3.device)
        check(lib.pw_mmd2(dt, mt, float(gamma), X3.data_ptr(), n, _rows(X3[0], "X"), sx, Y3.data_ptr(), m,
                          _rows(Y3[0], "Y"), sy, D, B, int(bool(unbiased)), out.data_ptr(), ws.data_ptr(), nb.value,
                          _stream(X3.device)), "pw_mmd2")
        ctx.save_for_backward(X3, Y3)
        ctx.args = (kernel, float(gamma), bool(unbiased))
        return out

    @staticmethod
    def backward(ctx, g):
        lib = load_library()
        X3, Y3 = ctx.saved_tensors
        kernel, gamma, unbiased = ctx.args
        B, n, m, D, sx, sy, dt, mt = _mmd_args(X3, Y3, kernel)
        G = g.to(X3.dtype).contiguous()
        dX = torch.empty(X3.shape[0], n, D, dtype=X3.dtype, device=X3.device) if ctx.needs_input_grad[0] else None
        dY = torch.empty(Y3.shape[0], m, D, dtype=X3.dtype, device=X3.device) if ctx.needs_input_grad[1] else None
        nb = ctypes.c_size_t()
        check(lib.pw_mmd2_backward_workspace_size(dt, mt, gamma, n, m, D, ctypes.byref(nb)),
              "pw_mmd2_backward_workspace_size")
        ws = torch.empty(max(nb.value, 1), dtype=torch.uint8, device=X3.device)
        check(lib.pw_mmd2_backward(dt, mt, gamma, X3.data_ptr(), n, _rows(X3[0], "X"), sx, Y3.data_ptr(), m,
                                   _rows(Y3[0], "Y"), sy, D, B, int(unbiased), G.data_ptr(),
                                   None if dX is None else dX.data_ptr(), D, None if dY is None else dY.data_ptr(),
                                   D, ws.data_ptr(), nb.value, _stream(X3.device)), "pw_mmd2_backward")
        return dX, dY, None, None, None


def mmd_statistics(X: torch.Tensor, Y: torch.Tensor, kernel: str = "rbf", gamma: float = 1.0,
                   unbiased: bool = True) -> torch.Tensor:
    """Squared maximum mean discrepancy between point clouds (Task Map, MMD
    row: mmd_statistics(X[None], Y[None], kernel="rbf", gamma=g), unbiased by
    default; one feature set is one cloud): X [B, n, D] (or [n, D]) against
    Y [B or 1, m, D] (or [m, D]); returns [B] (a scalar for 2-D inputs).
    pw_mmd2 does every step on the device, and pw_mmd2_backward gives the
    clouds' gradients under autograd."""
    vec = X.dim() == 2 and Y.dim() == 2
    X3 = X[None] if X.dim() == 2 else X
    Y3 = Y[None] if Y.dim() == 2 else Y
    out = _Mmd.apply(X3, Y3, kernel, gamma, unbiased)
    return out[0] if vec else out


def svgd_direction(x: torch.Tensor, score: torch.Tensor, gamma: float, workspace=None) -> torch.Tensor:
    """(K @ score - 2 gamma K.displacement()) / n for K = rbf(x, x): one
    kernel product and one displacement, combined on the device."""
    K = lazy(x, x, "rbf", gamma=gamma)
    drive = K.matmul(score)
    rep = K.displacement()
    return (drive - 2.0 * gamma * rep) / x.shape[-2]
