"""Python binding of the FFF forward-pass library (libfff.so, C ABI in
include/fff.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Torch tensors supply device memory and the current stream.  If the
library has not been built this module raises on first use; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libfff.so")

# fff_dtype_t
DTYPE_F32 = 0
DTYPE_BF16 = 1
# fff_status_t
SUCCESS = 0
ERROR_INVALID_VALUE = 1
ERROR_NOT_SUPPORTED = 2
ERROR_WORKSPACE = 3
ERROR_HIP = 4
# fff_algo_t
ALGO_AUTO = 0
ALGO_GENERIC = 1
ALGO_PREFILL = 2
ALGO_DECODE = 3
ALGOS = {"auto": ALGO_AUTO, "generic": ALGO_GENERIC, "prefill": ALGO_PREFILL, "decode": ALGO_DECODE}
# fff_plan_t flags
PLAN_TEST_DECODE_NO_PUBLISH = 1
# fff_variant_t
VARIANT_FFF = 0
VARIANT_POST = 1
VARIANTS = {"fff": VARIANT_FFF, "post": VARIANT_POST}
MAX_DEPTH = 20


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("P", ctypes.c_int32),
                ("D", ctypes.c_int32), ("h", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("variant", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("algo", ctypes.c_int32), ("split_level", ctypes.c_int32),
                ("chunk_tokens", ctypes.c_int32), ("flags", ctypes.c_int32)]


class StageEvents(ctypes.Structure):
    """fff_stage_events_t: HIP events recorded at the stage boundaries."""
    _fields_ = [("start", ctypes.c_void_p), ("prepared", ctypes.c_void_p), ("top", ctypes.c_void_p),
                ("deep", ctypes.c_void_p), ("routed", ctypes.c_void_p), ("done", ctypes.c_void_p)]
    NAMES = ("start", "prepared", "top", "deep", "routed", "done")


class Pruning(ctypes.Structure):
    """fff_pruning_t: a prepared static-pruning table (device memory is the
    caller's; keep the tensor that holds it alive while the table is used)."""
    _fields_ = [("table", ctypes.c_void_p), ("P", ctypes.c_int32), ("D", ctypes.c_int32),
                ("d", ctypes.c_int32), ("split_level", ctypes.c_int32),
                ("col_tiles", ctypes.c_int32)]


class FFFError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


EXPORTS = ("fff_plan_default", "fff_plan_resolve", "fff_workspace_size", "fff_forward",
           "fff_route", "fff_project", "fff_project_workspace_size", "fff_project_ws",
           "fff_status_string", "fff_algo_name",
           "fff_prune_table_size", "fff_prune_prepare", "fff_forward_pruned",
           "fff_backward_workspace_size", "fff_backward", "fff_forward_static",
           "fff_backward_pruned_workspace_size", "fff_backward_pruned")
STATIC_SCRATCH_BYTES = 32 << 20  # FFF_STATIC_SCRATCH_BYTES

_lib: Optional[ctypes.CDLL] = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libfff.so; raises if it is missing (build it with build.py)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIBRARY
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python sparse_tree_structured_amd/build.py` "
                          "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(p)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    SP, PP = ctypes.POINTER(Shape), ctypes.POINTER(Plan)
    lib.fff_plan_default.argtypes = [SP, PP]
    lib.fff_plan_resolve.argtypes = [SP, PP, PP]
    lib.fff_workspace_size.argtypes = [SP, PP, ctypes.POINTER(sz)]
    lib.fff_forward.argtypes = [SP, PP, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                ctypes.POINTER(StageEvents)]
    lib.fff_route.argtypes = [SP, PP, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.fff_project.argtypes = [SP, ctypes.c_int32, vp, vp, vp, vp]
    lib.fff_project_workspace_size.argtypes = [SP, ctypes.c_int32, ctypes.POINTER(sz)]
    lib.fff_project_ws.argtypes = [SP, ctypes.c_int32, vp, vp, vp, vp, sz, vp]
    PrP = ctypes.POINTER(Pruning)
    lib.fff_prune_table_size.argtypes = [SP, PP, ctypes.POINTER(sz)]
    lib.fff_prune_prepare.argtypes = [SP, PP, vp, vp, vp, sz, vp, PrP]
    lib.fff_forward_pruned.argtypes = [SP, PP, PrP, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                       ctypes.POINTER(StageEvents)]
    lib.fff_backward_workspace_size.argtypes = [SP, PP, ctypes.POINTER(sz)]
    lib.fff_backward.argtypes = [SP, PP, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.fff_backward_pruned_workspace_size.argtypes = [SP, PP, PrP, ctypes.POINTER(sz)]
    lib.fff_backward_pruned.argtypes = [SP, PP, PrP, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        vp, sz, vp]
    lib.fff_forward_static.argtypes = [SP, PP, vp, vp, vp, vp, vp, vp, vp, vp,
                                       ctypes.POINTER(StageEvents)]
    lib.fff_status_string.argtypes = [ctypes.c_int]
    lib.fff_status_string.restype = ctypes.c_char_p
    lib.fff_algo_name.argtypes = [ctypes.c_int32]
    lib.fff_algo_name.restype = ctypes.c_char_p
    for name in ("fff_plan_default", "fff_plan_resolve", "fff_workspace_size", "fff_forward",
                 "fff_route", "fff_project", "fff_project_workspace_size", "fff_project_ws",
                 "fff_prune_table_size", "fff_prune_prepare",
                 "fff_forward_pruned", "fff_backward_workspace_size", "fff_backward",
                 "fff_forward_static"):
        getattr(lib, name).restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().fff_status_string(int(status)).decode()


def algo_name(algo: int) -> str:
    return load_library().fff_algo_name(int(algo)).decode()


def _variant_code(variant) -> int:
    return VARIANTS[variant] if isinstance(variant, str) else int(variant)


def make_shape(T: int, d: int, P: int, D: int, h: int, dtype: int, variant=VARIANT_FFF) -> Shape:
    return Shape(int(T), int(d), int(P), int(D), int(h), int(dtype), _variant_code(variant))


def make_plan(algo=ALGO_AUTO, split_level: int = -1, chunk_tokens: int = 0,
              flags: int = 0) -> Plan:
    if isinstance(algo, str):
        algo = ALGOS[algo]
    return Plan(int(algo), int(split_level), int(chunk_tokens), int(flags))


def plan_default(shape: Shape) -> Plan:
    p = Plan()
    st = load_library().fff_plan_default(ctypes.byref(shape), ctypes.byref(p))
    if st != SUCCESS:
        raise FFFError(st, "fff_plan_default")
    return p


def resolve_plan(shape: Shape, plan: Plan) -> Plan:
    """The plan as the library would run it ('choose by shape' fields filled in)."""
    out = Plan()
    st = load_library().fff_plan_resolve(ctypes.byref(shape), ctypes.byref(plan), ctypes.byref(out))
    if st != SUCCESS:
        raise FFFError(st, "fff_plan_resolve")
    return out


def workspace_size(shape: Shape, plan: Optional[Plan] = None) -> int:
    n = ctypes.c_size_t()
    st = load_library().fff_workspace_size(ctypes.byref(shape),
                                           ctypes.byref(plan) if plan is not None else None,
                                           ctypes.byref(n))
    if st != SUCCESS:
        raise FFFError(st, "fff_workspace_size")
    return int(n.value)


# ---- torch-facing helpers (device memory and streams only) ----

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dims(t, n, what):
    if t.dim() != n:
        raise ValueError(f"{what} must have {n} dimensions, got shape {tuple(t.shape)}")
    return tuple(int(v) for v in t.shape)


def shape_of(x, W_node, V_node, variant=VARIANT_FFF) -> Shape:
    T, d = _dims(x, 2, "x [T,d]")
    P, N, d2 = _dims(W_node, 3, "W_node [P,N,d]")
    _dims(V_node, 3, "V_node [P,N,h]")
    h = int(V_node.shape[2])
    D = N.bit_length() - 1
    if d2 != d or N < 1 or (1 << (D + 1)) - 1 != N:
        raise ValueError(f"W_node must be [P, 2^(D+1)-1, d={d}], got {tuple(W_node.shape)}")
    return make_shape(T, d, P, D, h, _dtype_code(x), variant)


def _want(t, shape, what):
    if tuple(int(v) for v in t.shape) != tuple(shape):
        raise ValueError(f"{what} must be {list(shape)}, got {list(t.shape)}")


def _check(tensors, dtype, device):
    """Every tensor contiguous, of `dtype`, on `device`, which must be a GPU
    (the library takes device pointers only)."""
    for t in tensors:
        if t.dtype != dtype or t.device != device or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous, on one device, of one dtype")
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, not {device}")


def _check_layer(shape: Shape, x, W_node, b_node, V_node, W_out=None, extra=(), y=None,
                 path_out=None, workspace=None):
    """Full shapes of the layer's tensors against `shape` (W_out in the
    library's [P*h, d] layout, not nn.Linear's [d, P*h]), of the optional
    outputs y [T,d], path_out [T,P] and a flat workspace; then dtype (the
    layer's, int32 for path_out, uint8 for the workspace), device and
    contiguity.  Raises ValueError before anything reaches the library."""
    torch = _torch()
    N = (1 << (shape.D + 1)) - 1
    _want(x, (shape.T, shape.d), "x [T,d]")
    _want(W_node, (shape.P, N, shape.d), "W_node [P,N,d]")
    _want(b_node, (shape.P, N), "b_node [P,N]")
    _want(V_node, (shape.P, N, shape.h), "V_node [P,N,h]")
    same = [x, W_node, b_node, V_node]
    if W_out is not None:
        _want(W_out, (shape.P * shape.h, shape.d), "W_out [P*h,d]")
        same.append(W_out)
    for t, want, what in extra:
        _want(t, want, what)
        same.append(t)
    if y is not None:
        _want(y, (shape.T, shape.d), "y [T,d]")
        same.append(y)
    if path_out is not None:
        _want(path_out, (shape.T, shape.P), "path_out [T,P]")
    if workspace is not None and workspace.dim() != 1:
        raise ValueError("workspace must be a flat uint8 tensor")
    _check(same, x.dtype, x.device)
    if path_out is not None:
        _check([path_out], torch.int32, x.device)
    if workspace is not None:
        _check([workspace], torch.uint8, x.device)


def _stream_handle(stream) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def alloc_workspace(shape: Shape, plan: Optional[Plan], device):
    torch = _torch()
    n = workspace_size(shape, plan)
    # torch's caching allocator returns blocks aligned to at least 512 bytes.
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device), n


def forward(x, W_node, b_node, V_node, W_out, *, algo=ALGO_AUTO, split_level: int = -1,
            chunk_tokens: int = 0, want_path: bool = True, workspace=None, y=None, path_out=None,
            stream=None, events: Optional[StageEvents] = None,
            variant=VARIANT_FFF, plan_flags: int = 0) -> Tuple[object, Optional[object]]:
    """y = FFF(x); returns (y, path_out[T,P] int32 or None).

    ``variant`` "fff" (0) applies GELU to each visited node's logit; "post"
    (1) applies it to each element of a tree's summed output instead.
    ``plan_flags``: fff_plan_t flags (PLAN_TEST_DECODE_NO_PUBLISH, tests only)."""
    torch = _torch()
    shape = shape_of(x, W_node, V_node, variant)
    _check_layer(shape, x, W_node, b_node, V_node, W_out, y=y, path_out=path_out,
                 workspace=workspace)
    plan = make_plan(algo, split_level, chunk_tokens, plan_flags)
    if workspace is None:
        workspace, nbytes = alloc_workspace(shape, plan, x.device)
    else:
        nbytes = workspace.numel() * workspace.element_size()
    if y is None:
        y = torch.empty((shape.T, shape.d), dtype=x.dtype, device=x.device)
    if want_path and path_out is None:
        path_out = torch.empty((shape.T, shape.P), dtype=torch.int32, device=x.device)
    st = load_library().fff_forward(
        ctypes.byref(shape), ctypes.byref(plan), x.data_ptr(), W_node.data_ptr(), b_node.data_ptr(),
        V_node.data_ptr(), W_out.data_ptr(), y.data_ptr(),
        path_out.data_ptr() if path_out is not None else None,
        workspace.data_ptr(), nbytes, _stream_handle(stream),
        ctypes.byref(events) if events is not None else None)
    if st != SUCCESS:
        raise FFFError(st, "fff_forward")
    return y, path_out


def forward_static(x, W_node, b_node, V_node, W_out, y, path_out=None, *, algo=ALGO_AUTO,
                   split_level: int = -1, chunk_tokens: int = 0, stream=None,
                   events: Optional[StageEvents] = None, variant=VARIANT_FFF,
                   plan_flags: int = 0):
    """fff_forward_static: the layer with the library's fixed scratch region
    as its workspace.  The caller passes y [T,d] (and path_out [T,P] int32,
    or None); nothing is allocated."""
    shape = shape_of(x, W_node, V_node, variant)
    _check_layer(shape, x, W_node, b_node, V_node, W_out, y=y, path_out=path_out)
    plan = make_plan(algo, split_level, chunk_tokens, plan_flags)
    st = load_library().fff_forward_static(
        ctypes.byref(shape), ctypes.byref(plan), x.data_ptr(), W_node.data_ptr(),
        b_node.data_ptr(), V_node.data_ptr(), W_out.data_ptr(), y.data_ptr(),
        path_out.data_ptr() if path_out is not None else None, _stream_handle(stream),
        ctypes.byref(events) if events is not None else None)
    if st != SUCCESS:
        raise FFFError(st, "fff_forward_static")
    return y, path_out


def route(x, W_node, b_node, V_node, *, algo=ALGO_AUTO, split_level: int = -1,
          chunk_tokens: int = 0, stream=None, variant=VARIANT_FFF):
    """Routing only: returns (H[T, P*h], path_out[T,P])."""
    torch = _torch()
    shape = shape_of(x, W_node, V_node, variant)
    _check_layer(shape, x, W_node, b_node, V_node)
    plan = make_plan(algo, split_level, chunk_tokens)
    workspace, nbytes = alloc_workspace(shape, plan, x.device)
    H = torch.empty((shape.T, shape.P * shape.h), dtype=x.dtype, device=x.device)
    path = torch.empty((shape.T, shape.P), dtype=torch.int32, device=x.device)
    st = load_library().fff_route(ctypes.byref(shape), ctypes.byref(plan), x.data_ptr(),
                                  W_node.data_ptr(), b_node.data_ptr(), V_node.data_ptr(),
                                  H.data_ptr(), path.data_ptr(), workspace.data_ptr(), nbytes,
                                  _stream_handle(stream))
    if st != SUCCESS:
        raise FFFError(st, "fff_route")
    return H, path


def project_workspace_size(shape: Shape, algo=ALGO_AUTO) -> int:
    """Workspace bytes of fff_project_ws (0 where it needs none)."""
    if isinstance(algo, str):
        algo = ALGOS[algo]
    n = ctypes.c_size_t()
    st = load_library().fff_project_workspace_size(ctypes.byref(shape), int(algo), ctypes.byref(n))
    if st != SUCCESS:
        raise FFFError(st, "fff_project_workspace_size")
    return n.value


def project(H, W_out, *, algo=ALGO_AUTO, stream=None, y=None, workspace=None,
            use_workspace: bool = True):
    """y = H . W_out (fp32 accumulation).

    With ``use_workspace`` (default) the call goes through fff_project_ws
    (whose workspace size is 0: it may be None), else through fff_project;
    both run the kernel fff_forward's projection uses for the same shape."""
    torch = _torch()
    T, K = _dims(H, 2, "H [T,K]")
    K2, d = _dims(W_out, 2, "W_out [K,d]")
    if K2 != K:
        raise ValueError(f"H {list(H.shape)} and W_out {list(W_out.shape)} disagree on K")
    if y is not None:
        _want(y, (T, d), "y [T,d]")
    _check([H, W_out] + ([y] if y is not None else []), H.dtype, H.device)
    if workspace is not None:
        _check([workspace], torch.uint8, H.device)
    # K = P*h with P=1, h=K describes the product for the library.
    shape = make_shape(T, d, 1, 0, K, _dtype_code(H))
    if y is None:
        y = torch.empty((T, d), dtype=H.dtype, device=H.device)
    if isinstance(algo, str):
        algo = ALGOS[algo]
    lib = load_library()
    if not use_workspace:
        st = lib.fff_project(ctypes.byref(shape), int(algo), H.data_ptr(), W_out.data_ptr(),
                             y.data_ptr(), _stream_handle(stream))
        if st != SUCCESS:
            raise FFFError(st, "fff_project")
        return y
    if workspace is None:
        nbytes = project_workspace_size(shape, algo)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=H.device) if nbytes else None
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.fff_project_ws(ctypes.byref(shape), int(algo), H.data_ptr(), W_out.data_ptr(),
                            y.data_ptr(), ws_ptr, ws_bytes, _stream_handle(stream))
    if st != SUCCESS:
        raise FFFError(st, "fff_project_ws")
    return y


def prune_table_size(shape: Shape, plan: Optional[Plan] = None) -> int:
    n = ctypes.c_size_t()
    st = load_library().fff_prune_table_size(ctypes.byref(shape),
                                             ctypes.byref(plan) if plan is not None else None,
                                             ctypes.byref(n))
    if st != SUCCESS:
        raise FFFError(st, "fff_prune_table_size")
    return int(n.value)


def prune_prepare(leaf_alive, W_node, V_node, *, algo=ALGO_AUTO, split_level: int = -1,
                  chunk_tokens: int = 0, T: Optional[int] = None, stream=None,
                  variant=VARIANT_FFF):
    """Static path pruning table for trees W_node [P,N,d] (device) and a leaf
    mask leaf_alive [P, 2^D] (host: numpy or CPU tensor, nonzero = alive).
    The plan is resolved for T tokens (default 65536, a prefill batch) and
    the given options; returns (Pruning, table tensor), the tensor owning the
    device memory."""
    import numpy as np
    torch = _torch()
    P, N, d = W_node.shape
    D = N.bit_length() - 1
    mask = np.ascontiguousarray(np.asarray(leaf_alive, dtype=np.uint8))
    if mask.shape != (P, 1 << D):
        raise ValueError("leaf_alive must be [P, 2^D]")
    shape = make_shape(T if T is not None else 65536, d, P, D, V_node.shape[2],
                       _dtype_code(W_node), variant)
    plan = make_plan(algo, split_level, chunk_tokens)
    n = prune_table_size(shape, plan)
    table = torch.empty(max(n, 1), dtype=torch.uint8, device=W_node.device)
    out = Pruning()
    st = load_library().fff_prune_prepare(
        ctypes.byref(shape), ctypes.byref(plan), mask.ctypes.data_as(ctypes.c_void_p),
        W_node.data_ptr(), table.data_ptr(), n, _stream_handle(stream), ctypes.byref(out))
    if st != SUCCESS:
        raise FFFError(st, "fff_prune_prepare")
    return out, table


def forward_pruned(x, W_node, b_node, V_node, W_out, pruning: Pruning, *, algo=ALGO_AUTO,
                   split_level: int = -1, chunk_tokens: int = 0, want_path: bool = True,
                   workspace=None, y=None, path_out=None, stream=None,
                   events: Optional[StageEvents] = None, variant=VARIANT_FFF):
    """fff_forward_pruned: y and path_out of the pruned trees."""
    torch = _torch()
    shape = shape_of(x, W_node, V_node, variant)
    _check_layer(shape, x, W_node, b_node, V_node, W_out, y=y, path_out=path_out,
                 workspace=workspace)
    plan = make_plan(algo, split_level, chunk_tokens)
    if workspace is None:
        workspace, nbytes = alloc_workspace(shape, plan, x.device)
    else:
        nbytes = workspace.numel() * workspace.element_size()
    if y is None:
        y = torch.empty((shape.T, shape.d), dtype=x.dtype, device=x.device)
    if want_path and path_out is None:
        path_out = torch.empty((shape.T, shape.P), dtype=torch.int32, device=x.device)
    st = load_library().fff_forward_pruned(
        ctypes.byref(shape), ctypes.byref(plan), ctypes.byref(pruning), x.data_ptr(),
        W_node.data_ptr(), b_node.data_ptr(), V_node.data_ptr(), W_out.data_ptr(), y.data_ptr(),
        path_out.data_ptr() if path_out is not None else None, workspace.data_ptr(), nbytes,
        _stream_handle(stream), ctypes.byref(events) if events is not None else None)
    if st != SUCCESS:
        raise FFFError(st, "fff_forward_pruned")
    return y, path_out


def backward_workspace_size(shape: Shape, plan: Optional[Plan] = None) -> int:
    n = ctypes.c_size_t()
    st = load_library().fff_backward_workspace_size(
        ctypes.byref(shape), ctypes.byref(plan) if plan is not None else None, ctypes.byref(n))
    if st != SUCCESS:
        raise FFFError(st, "fff_backward_workspace_size")
    return int(n.value)


def backward_pruned_workspace_size(shape: Shape, plan: Optional[Plan], pruning: Pruning) -> int:
    n = ctypes.c_size_t()
    st = load_library().fff_backward_pruned_workspace_size(
        ctypes.byref(shape), ctypes.byref(plan) if plan is not None else None,
        ctypes.byref(pruning), ctypes.byref(n))
    if st != SUCCESS:
        raise FFFError(st, "fff_backward_pruned_workspace_size")
    return int(n.value)


def backward(x, W_node, b_node, V_node, W_out, dy, *, algo=ALGO_AUTO, split_level: int = -1,
             workspace=None, out=None, stream=None, variant=VARIANT_FFF):
    """Gradients of sum(y * dy) with the forward's paths held fixed.  Returns
    a dict: dx (dtype of x), dW_node, db_node, dV_node, dW_out (float32)."""
    return _backward(x, W_node, b_node, V_node, W_out, dy, None, algo, split_level, workspace,
                     out, stream, variant)


def backward_pruned(x, W_node, b_node, V_node, W_out, dy, pruning: Pruning, *, algo=ALGO_AUTO,
                    split_level: int = -1, workspace=None, out=None, stream=None,
                    variant=VARIANT_FFF):
    """fff_backward_pruned: the gradients of backward() with the paths
    fff_forward_pruned takes on the prepared table."""
    return _backward(x, W_node, b_node, V_node, W_out, dy, pruning, algo, split_level, workspace,
                     out, stream, variant)


def _backward(x, W_node, b_node, V_node, W_out, dy, pruning, algo, split_level, workspace, out,
              stream, variant):
    torch = _torch()
    shape = shape_of(x, W_node, V_node, variant)
    N = (1 << (shape.D + 1)) - 1
    want = {"dx": ((shape.T, shape.d), x.dtype), "dW_node": ((shape.P, N, shape.d), torch.float32),
            "db_node": ((shape.P, N), torch.float32),
            "dV_node": ((shape.P, N, shape.h), torch.float32),
            "dW_out": ((shape.P * shape.h, shape.d), torch.float32)}
    if out is not None:
        for k, (shp, _) in want.items():
            _want(out[k], shp, k)
    _check_layer(shape, x, W_node, b_node, V_node, W_out,
                 extra=[(dy, (shape.T, shape.d), "dy [T,d]")], workspace=workspace)
    if out is not None:
        for k, (_, dt) in want.items():
            _check([out[k]], dt, x.device)
    plan = make_plan(algo, split_level, 0)
    if workspace is None:
        n = (backward_workspace_size(shape, plan) if pruning is None
             else backward_pruned_workspace_size(shape, plan, pruning))
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=x.device)
    nbytes = workspace.numel() * workspace.element_size()
    f32 = dict(dtype=torch.float32, device=x.device)
    g = out or {"dx": torch.empty_like(x), "dW_node": torch.empty(W_node.shape, **f32),
                "db_node": torch.empty(b_node.shape, **f32),
                "dV_node": torch.empty(V_node.shape, **f32),
                "dW_out": torch.empty(W_out.shape, **f32)}
    ptrs = (x.data_ptr(), W_node.data_ptr(), b_node.data_ptr(), V_node.data_ptr(),
            W_out.data_ptr(), dy.data_ptr(), g["dx"].data_ptr(), g["dW_node"].data_ptr(),
            g["db_node"].data_ptr(), g["dV_node"].data_ptr(), g["dW_out"].data_ptr(),
            workspace.data_ptr(), nbytes, _stream_handle(stream))
    lib = load_library()
    if pruning is None:
        st = lib.fff_backward(ctypes.byref(shape), ctypes.byref(plan), *ptrs)
        what = "fff_backward"
    else:
        st = lib.fff_backward_pruned(ctypes.byref(shape), ctypes.byref(plan),
                                     ctypes.byref(pruning), *ptrs)
        what = "fff_backward_pruned"
    if st != SUCCESS:
        raise FFFError(st, what)
    return g
