"""MI355X (gfx950) AVQ-Attention forward pass.

Thin Python binding of the C ABI in include/avq.h (libavq.so, built by
``python -m adaptive_vector_quantized_avq_amd.build``).  Each function checks
tensor shapes/devices, allocates outputs with torch and forwards raw device
pointers plus the current HIP stream to the library; every step of the
computation runs in the library's HIP kernels.  There is no fallback path:
if the library is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "AvqError", "library_path", "load_library", "abi_version",
    "build_tree3", "assign_aggregate3", "attention3_fwd", "attention3_workspace_size",
    "assign_aggregate3_workspace_size",
    "build_tree", "assign_aggregate", "attention_fwd", "exact_attention_fwd",
    "assign_aggregate_workspace_size", "attention_workspace_size", "forward",
    "assign_aggregate_noalloc", "NOALLOC_SCRATCH_BYTES", "codebook_diagnostics", "capture",
    "gilbert_order", "permute_tokens",
    "AVQ_FLAG_FORCE_CHILD", "AVQ_FLAG_UNFUSED",
]

AVQ_FLAG_FORCE_CHILD = 1
AVQ_FLAG_UNFUSED = 2
NOALLOC_SCRATCH_BYTES = 16 << 20   # AVQ_NOALLOC_SCRATCH_BYTES of include/avq.h
_DTYPES = {torch.float32: 0, torch.bfloat16: 1}
_PKG = os.path.dirname(os.path.abspath(__file__))
_lib = None


class AvqError(RuntimeError):
    pass


def library_path() -> str:
    return os.path.join(_PKG, "libavq.so")


def load_library():
    """Load libavq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise AvqError(f"{path} is missing: build it with "
                       "`python -m adaptive_vector_quantized_avq_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, u32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_float, ctypes.c_size_t
    lib.avq_abi_version.restype = i32
    lib.avq_status_string.restype = ctypes.c_char_p
    lib.avq_status_string.argtypes = [i32]
    lib.avq_last_error.restype = ctypes.c_char_p
    lib.avq_build_tree.restype = i32
    lib.avq_build_tree.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.avq_assign_aggregate_workspace_size.restype = sz
    lib.avq_assign_aggregate_workspace_size.argtypes = [i32] * 6
    lib.avq_assign_aggregate_noalloc.restype = i32
    lib.avq_assign_aggregate_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                                 u32, vp, vp, vp, vp]
    lib.avq_attention_workspace_size.restype = sz
    lib.avq_attention_workspace_size.argtypes = [i32] * 6
    lib.avq_assign_aggregate.restype = i32
    lib.avq_assign_aggregate.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, u32,
                                         vp, vp, vp, vp, sz, vp]
    lib.avq_attention_fwd.restype = i32
    lib.avq_attention_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                      f32, i32, vp, vp, vp, vp, sz, vp]
    lib.avq_diagnostics_workspace_size.restype = sz
    lib.avq_diagnostics_workspace_size.argtypes = [i32, i32, i32]
    lib.avq_codebook_diagnostics.restype = i32
    lib.avq_codebook_diagnostics.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                             vp, vp, vp, sz, vp]
    lib.avq_capture.restype = i32
    lib.avq_capture.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp, vp]
    lib.avq_gilbert_order.restype = i32
    lib.avq_gilbert_order.argtypes = [i32, i32, vp]
    lib.avq_permute_tokens.restype = i32
    lib.avq_permute_tokens.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.avq_exact_attention_fwd.restype = i32
    lib.avq_exact_attention_fwd.argtypes = [vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, vp]
    lib.avq_build_tree3.restype = i32
    lib.avq_build_tree3.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]
    lib.avq_assign_aggregate3_workspace_size.restype = sz
    lib.avq_assign_aggregate3_workspace_size.argtypes = [i32] * 6
    lib.avq_assign_aggregate3.restype = i32
    lib.avq_assign_aggregate3.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, u32,
                                          vp, vp, vp, vp, sz, vp]
    lib.avq_attention3_workspace_size.restype = sz
    lib.avq_attention3_workspace_size.argtypes = [i32] * 6
    lib.avq_attention3_fwd.restype = i32
    lib.avq_attention3_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                                       vp, vp, vp, vp, sz, vp]
    _lib = lib
    return lib


def abi_version() -> int:
    return load_library().avq_abi_version()


def _check(rc: int):
    if rc != 0:
        lib = load_library()
        raise AvqError(f"{lib.avq_status_string(rc).decode()}: {lib.avq_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _on(dev: torch.device):
    # the library launches on the given stream but reads per-device state
    # (CU count, kernel attributes) from the current device
    return torch.cuda.device(dev)


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise AvqError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")
    return _DTYPES[t.dtype]


def _need(t: torch.Tensor, name: str, ndim: int, dtype=None, dev=None):
    if not isinstance(t, torch.Tensor) or t.dim() != ndim:
        raise AvqError(f"{name} must be a {ndim}-d tensor")
    if not t.is_cuda:
        raise AvqError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise AvqError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise AvqError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if dev is not None and t.device != dev:
        raise AvqError(f"{name} is on {t.device}, expected {dev}")


def _tree_dims(children: torch.Tensor):
    """(H, M0, C, d) of a tree's children [H][M0][C][d], or of a flat
    codebook [H][M0][d] (C = 0)."""
    if not isinstance(children, torch.Tensor) or children.dim() not in (3, 4):
        raise AvqError("children must be [H][M0][C][d] (or a flat codebook [H][M0][d])")
    if children.dim() == 3:
        H, M0, d = children.shape
        return H, M0, 0, d
    return tuple(children.shape)


def build_tree(children: torch.Tensor):
    """children [H][M0][C][d] (or a flat codebook [H][M0][d], C = 0) ->
    (parents [H][M0][d], sqnorm [H][M0(1+C)] fp32, frame [H][d] fp32): the
    tree stage 1 reads (norms are in the frame)."""
    H, M0, C, d = _tree_dims(children)
    _need(children, "children", children.dim())
    parents = torch.empty((H, M0, d), dtype=children.dtype, device=children.device)
    sqnorm = torch.empty((H, M0 * (1 + C)), dtype=torch.float32, device=children.device)
    frame = torch.empty((H, d), dtype=torch.float32, device=children.device)
    with _on(children.device):
        _check(load_library().avq_build_tree(_ptr(children), H, M0, C, d, _dt(children), _ptr(parents),
                                             _ptr(sqnorm), _ptr(frame), _stream(children.device)))
    return parents, sqnorm, frame


def assign_aggregate_workspace_size(B, H, N, M0, C, d) -> int:
    return int(load_library().avq_assign_aggregate_workspace_size(B, H, N, M0, C, d))


def attention_workspace_size(B, H, M0, C, d, dtype) -> int:
    return int(load_library().avq_attention_workspace_size(B, H, M0, C, d, _DTYPES[dtype]))


def _workspace(ws, need: int, dev, name: str):
    if ws is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(ws, name, 1, torch.uint8, dev)
    if ws.numel() < need:
        raise AvqError(f"{name} too small: {ws.numel()} < {need} bytes")
    return ws


def assign_aggregate(K, V, parents, children, sqnorm, frame, force_child: bool = False,
                     want_leaf: bool = False, workspace: Optional[torch.Tensor] = None,
                     out: Optional[tuple] = None, unfused: bool = False):
    """Stage 1.  K, V [B][H][N][d] -> (vsum [B][H][S_tot][d] fp32,
    count [B][H][S_tot] int32, leaf [B][H][N] int32 or None).  `unfused`
    (flat codebooks only) runs the separate assign-then-scatter comparison
    path."""
    _need(K, "K", 4)
    dev, dt = K.device, K.dtype
    _need(V, "V", 4, dt, dev)
    Hc, M0, C, dc = _tree_dims(children)
    _need(children, "children", children.dim(), dt, dev)
    _need(parents, "parents", 3, dt, dev)
    _need(sqnorm, "sqnorm", 2, torch.float32, dev)
    _need(frame, "frame", 2, torch.float32, dev)
    B, H, N, d = K.shape
    if V.shape != K.shape or Hc != H or dc != d or \
            parents.shape != (H, M0, d) or sqnorm.shape != (H, M0 * (1 + C)) or frame.shape != (H, d):
        raise AvqError("inconsistent shapes")
    S = M0 * (1 + C)
    lib = load_library()
    workspace = _workspace(workspace, int(lib.avq_assign_aggregate_workspace_size(B, H, N, M0, C, d)),
                           dev, "workspace")
    if out is None:
        vsum = torch.empty((B, H, S, d), dtype=torch.float32, device=dev)
        count = torch.empty((B, H, S), dtype=torch.int32, device=dev)
    else:
        vsum, count = out
        _need(vsum, "vsum", 4, torch.float32, dev)
        _need(count, "count", 3, torch.int32, dev)
        if vsum.shape != (B, H, S, d) or count.shape != (B, H, S):
            raise AvqError("output buffers do not match the shape")
    leaf = torch.empty((B, H, N), dtype=torch.int32, device=dev) if want_leaf else None
    with _on(dev):
        _check(lib.avq_assign_aggregate(
            _ptr(K), _ptr(V), _ptr(parents), _ptr(children), _ptr(sqnorm), _ptr(frame), B, H, N, d, M0, C, _dt(K),
            (AVQ_FLAG_FORCE_CHILD if force_child else 0) | (AVQ_FLAG_UNFUSED if unfused else 0),
            _ptr(vsum), _ptr(count), _ptr(leaf), _ptr(workspace), workspace.numel(), _stream(dev)))
    return vsum, count, leaf


def assign_aggregate_noalloc(K, V, parents, children, sqnorm, frame, out, force_child: bool = False,
                             leaf: Optional[torch.Tensor] = None):
    """Stage 1 through the allocation-free entry point: the caller passes the
    outputs out = (vsum [B][H][S_tot][d] fp32, count [B][H][S_tot] int32) and
    optionally leaf [B][H][N] int32; the library uses its own static device
    scratch (calls that overlap on one device race).  Returns out."""
    _need(K, "K", 4)
    dev, dt = K.device, K.dtype
    _need(V, "V", 4, dt, dev)
    Hc, M0, C, dc = _tree_dims(children)
    _need(children, "children", children.dim(), dt, dev)
    _need(parents, "parents", 3, dt, dev)
    _need(sqnorm, "sqnorm", 2, torch.float32, dev)
    _need(frame, "frame", 2, torch.float32, dev)
    B, H, N, d = K.shape
    if V.shape != K.shape or Hc != H or dc != d or \
            parents.shape != (H, M0, d) or sqnorm.shape != (H, M0 * (1 + C)) or frame.shape != (H, d):
        raise AvqError("inconsistent shapes")
    S = M0 * (1 + C)
    vsum, count = out
    _need(vsum, "vsum", 4, torch.float32, dev)
    _need(count, "count", 3, torch.int32, dev)
    if vsum.shape != (B, H, S, d) or count.shape != (B, H, S):
        raise AvqError("output buffers do not match the shape")
    if leaf is not None:
        _need(leaf, "leaf", 3, torch.int32, dev)
        if leaf.shape != (B, H, N):
            raise AvqError("leaf does not match the shape")
    with _on(dev):
        _check(load_library().avq_assign_aggregate_noalloc(
            _ptr(K), _ptr(V), _ptr(parents), _ptr(children), _ptr(sqnorm), _ptr(frame), B, H, N, d, M0, C, _dt(K),
            AVQ_FLAG_FORCE_CHILD if force_child else 0, _ptr(vsum), _ptr(count), _ptr(leaf),
            _stream(dev)))
    return vsum, count


def attention_fwd(Q, parents, children, vsum, count, P: int, tile: int, scale: float,
                  want_sel: bool = False, want_importance: bool = False,
                  workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """Stage 2.  Q [B][H][N][d] and the aggregates vsum [B][H][S_tot][d] fp32,
    count [B][H][S_tot] int32 -> (Y [B][H][N][d], sel [B][H][ntiles][P] or
    None, importance [B][H][ntiles][M0] or None)."""
    _need(Q, "Q", 4)
    dev, dt = Q.device, Q.dtype
    Hc, M0, C, dc = _tree_dims(children)
    _need(children, "children", children.dim(), dt, dev)
    _need(parents, "parents", 3, dt, dev)
    _need(vsum, "vsum", 4, torch.float32, dev)
    _need(count, "count", 3, torch.int32, dev)
    B, H, N, d = Q.shape
    S = M0 * (1 + C)
    if parents.shape != (H, M0, d) or Hc != H or dc != d:
        raise AvqError("inconsistent shapes")
    if vsum.shape != (B, H, S, d) or count.shape != (B, H, S):
        raise AvqError("vsum / count do not match the shape")
    lib = load_library()
    workspace = _workspace(workspace, int(lib.avq_attention_workspace_size(B, H, M0, C, d, _dt(Q))),
                           dev, "workspace")
    nt = -(-N // tile) if tile > 0 else 0
    Y = torch.empty_like(Q) if out is None else out
    _need(Y, "out", 4, dt, dev)
    if Y.shape != Q.shape:
        raise AvqError("out must have Q's shape")
    sel = torch.empty((B, H, nt, P), dtype=torch.int32, device=dev) if want_sel else None
    imp = torch.empty((B, H, nt, M0), dtype=torch.float32, device=dev) if want_importance else None
    with _on(dev):
        _check(lib.avq_attention_fwd(
            _ptr(Q), _ptr(parents), _ptr(children), _ptr(vsum), _ptr(count), B, H, N, d, M0, C, P,
            tile, float(scale), _dt(Q), _ptr(Y), _ptr(sel), _ptr(imp), _ptr(workspace),
            workspace.numel(), _stream(dev)))
    return Y, sel, imp


def codebook_diagnostics(K, parents, children, leaf, count, commitment: bool = True, active: bool = True):
    """Commitment loss E||k - k_hat||^2 [B][H] (needs K and leaf) and active
    ratio [B][H] (needs count) -> (commit or None, active or None)."""
    _need(K, "K", 4)
    dev, dt = K.device, K.dtype
    H, M0, C, d = _tree_dims(children)
    _need(children, "children", children.dim(), dt, dev)
    _need(parents, "parents", 3, dt, dev)
    _need(leaf, "leaf", 3, torch.int32, dev)
    _need(count, "count", 3, torch.int32, dev)
    B, Hk, N, dk = K.shape
    if Hk != H or dk != d or parents.shape != (H, M0, d) or leaf.shape != (B, H, N) or \
            count.shape != (B, H, M0 * (1 + C)):
        raise AvqError("inconsistent shapes")
    lib = load_library()
    ws = _workspace(None, int(lib.avq_diagnostics_workspace_size(B, H, N)), dev, "workspace")
    cm = torch.empty((B, H), dtype=torch.float32, device=dev) if commitment else None
    ac = torch.empty((B, H), dtype=torch.float32, device=dev) if active else None
    with _on(dev):
        _check(lib.avq_codebook_diagnostics(_ptr(K), _ptr(parents), _ptr(children), _ptr(leaf), _ptr(count),
                                            B, H, N, d, M0, C, _dt(K), _ptr(cm), _ptr(ac), _ptr(ws),
                                            ws.numel(), _stream(dev)))
    return cm, ac


def capture(Q, K, children, leaf, sel, tile: int, scale: float):
    """Per-query capture [B][H][N]: the fraction of exact softmax weight on
    keys whose parent the query's tile selected (sel from attention_fwd)."""
    _need(Q, "Q", 4)
    dev, dt = Q.device, Q.dtype
    _need(K, "K", 4, dt, dev)
    H, M0, C, d = _tree_dims(children)
    _need(leaf, "leaf", 3, torch.int32, dev)
    _need(sel, "sel", 4, torch.int32, dev)
    B, Hq, N, dq = Q.shape
    nt = -(-N // tile) if tile > 0 else 0
    if K.shape != Q.shape or Hq != H or dq != d or leaf.shape != (B, H, N) or sel.shape[:3] != (B, H, nt):
        raise AvqError("inconsistent shapes")
    P = sel.shape[3]
    out = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    with _on(dev):
        _check(load_library().avq_capture(_ptr(Q), _ptr(K), _ptr(leaf), _ptr(sel) if P > 0 else None, B, H, N,
                                          d, M0, C, P, tile, float(scale), _dt(Q), _ptr(out), _stream(dev)))
    return out


def gilbert_order(W: int, H: int) -> torch.Tensor:
    """Row-major cell indices of a W x H grid along the Gilbert curve, as a
    CPU int32 tensor (host computation in the library)."""
    out = torch.empty(W * H, dtype=torch.int32)
    _check(load_library().avq_gilbert_order(W, H, _ptr(out)))
    return out


def permute_tokens(x: torch.Tensor, order: torch.Tensor, inverse: bool = False,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x [B][H][N][d] -> rows moved into the order (out[:, :, i] =
    x[:, :, order[i]]) or, with inverse, back out of it."""
    _need(x, "x", 4)
    _need(order, "order", 1, torch.int32, x.device)
    B, H, N, d = x.shape
    if order.numel() != N:
        raise AvqError("order must have N entries")
    y = torch.empty_like(x) if out is None else out
    _need(y, "out", 4, x.dtype, x.device)
    if y.shape != x.shape:
        raise AvqError("out must have x's shape")
    with _on(x.device):
        _check(load_library().avq_permute_tokens(_ptr(x), _ptr(order), B, H, N, d, _dt(x), 1 if inverse else 0,
                                                 _ptr(y), _stream(x.device)))
    return y


def exact_attention_fwd(Q, K, V, scale: float, out: Optional[torch.Tensor] = None):
    """Exact softmax attention, Q/K/V [B][H][N][d] -> Y."""
    _need(Q, "Q", 4)
    _need(K, "K", 4, Q.dtype, Q.device)
    _need(V, "V", 4, Q.dtype, Q.device)
    if K.shape != Q.shape or V.shape != Q.shape:
        raise AvqError("Q, K, V must have the same shape")
    B, H, N, d = Q.shape
    Y = torch.empty_like(Q) if out is None else out
    _need(Y, "out", 4, Q.dtype, Q.device)
    if Y.shape != Q.shape:
        raise AvqError("out must have Q's shape")
    with _on(Q.device):
        _check(load_library().avq_exact_attention_fwd(_ptr(Q), _ptr(K), _ptr(V), B, H, N, d, float(scale),
                                                      _dt(Q), _ptr(Y), _stream(Q.device)))
    return Y


# ---------------------------------------------------------------------------
# three-level tree (roots -> children -> leaves)

def _tree3_dims(leaves: torch.Tensor):
    if not isinstance(leaves, torch.Tensor) or leaves.dim() != 5 or leaves.shape[2] != leaves.shape[3]:
        raise AvqError("leaves must be [H][M0][C][C][d]")
    H, M0, C, _, d = leaves.shape
    return H, M0, C, d


def build_tree3(leaves: torch.Tensor):
    """leaves [H][M0][C][C][d] -> (level0 [H][M0][d], level1 [H][M0][C][d],
    sqnorm [H][M0(1+C+C^2)] fp32, frame [H][d] fp32)."""
    H, M0, C, d = _tree3_dims(leaves)
    _need(leaves, "leaves", 5)
    dev = leaves.device
    l0 = torch.empty((H, M0, d), dtype=leaves.dtype, device=dev)
    l1 = torch.empty((H, M0, C, d), dtype=leaves.dtype, device=dev)
    sq = torch.empty((H, M0 * (1 + C + C * C)), dtype=torch.float32, device=dev)
    fr = torch.empty((H, d), dtype=torch.float32, device=dev)
    with _on(dev):
        _check(load_library().avq_build_tree3(_ptr(leaves), H, M0, C, d, _dt(leaves), _ptr(l0), _ptr(l1),
                                              _ptr(sq), _ptr(fr), _stream(dev)))
    return l0, l1, sq, fr


def assign_aggregate3_workspace_size(B, H, N, M0, C, d) -> int:
    return int(load_library().avq_assign_aggregate3_workspace_size(B, H, N, M0, C, d))


def assign_aggregate3(K, V, level0, level1, leaves, sqnorm, frame, force_child: bool = False,
                      want_leaf: bool = False, workspace: Optional[torch.Tensor] = None,
                      out: Optional[tuple] = None):
    """Stage 1 on a three-level tree: (vsum [B][H][S3][d] fp32, count
    [B][H][S3] int32, leaf [B][H][N] int32 or None); `out` = (vsum, count)
    buffers to write into."""
    _need(K, "K", 4)
    dev, dt = K.device, K.dtype
    _need(V, "V", 4, dt, dev)
    H, M0, C, d = _tree3_dims(leaves)
    _need(leaves, "leaves", 5, dt, dev)
    _need(level0, "level0", 3, dt, dev)
    _need(level1, "level1", 4, dt, dev)
    _need(sqnorm, "sqnorm", 2, torch.float32, dev)
    _need(frame, "frame", 2, torch.float32, dev)
    B, Hk, N, dk = K.shape
    S = M0 * (1 + C + C * C)
    if V.shape != K.shape or Hk != H or dk != d or level0.shape != (H, M0, d) or \
            level1.shape != (H, M0, C, d) or sqnorm.shape != (H, S) or frame.shape != (H, d):
        raise AvqError("inconsistent shapes")
    lib = load_library()
    workspace = _workspace(workspace, int(lib.avq_assign_aggregate3_workspace_size(B, H, N, M0, C, d)),
                           dev, "workspace")
    if out is None:
        vsum = torch.empty((B, H, S, d), dtype=torch.float32, device=dev)
        count = torch.empty((B, H, S), dtype=torch.int32, device=dev)
    else:
        vsum, count = out
        _need(vsum, "vsum", 4, torch.float32, dev)
        _need(count, "count", 3, torch.int32, dev)
        if vsum.shape != (B, H, S, d) or count.shape != (B, H, S):
            raise AvqError("output buffers do not match the shape")
    leaf = torch.empty((B, H, N), dtype=torch.int32, device=dev) if want_leaf else None
    with _on(dev):
        _check(lib.avq_assign_aggregate3(
            _ptr(K), _ptr(V), _ptr(level0), _ptr(level1), _ptr(leaves), _ptr(sqnorm), _ptr(frame), B, H, N, d,
            M0, C, _dt(K), AVQ_FLAG_FORCE_CHILD if force_child else 0, _ptr(vsum), _ptr(count), _ptr(leaf),
            _ptr(workspace), workspace.numel(), _stream(dev)))
    return vsum, count, leaf


def attention3_workspace_size(B, H, M0, C, d, dtype) -> int:
    return int(load_library().avq_attention3_workspace_size(B, H, M0, C, d, _DTYPES[dtype]))


def attention3_fwd(Q, level0, level1, leaves, vsum, count, P: int, tile: int, scale: float,
                   want_sel: bool = False, workspace: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None):
    """Stage 2 on a three-level tree -> (Y, sel0 [B][H][ntiles][P] or None,
    sel1 [B][H][ntiles][P] or None: selected roots and children, ascending)."""
    _need(Q, "Q", 4)
    dev, dt = Q.device, Q.dtype
    H, M0, C, d = _tree3_dims(leaves)
    _need(leaves, "leaves", 5, dt, dev)
    _need(level0, "level0", 3, dt, dev)
    _need(level1, "level1", 4, dt, dev)
    _need(vsum, "vsum", 4, torch.float32, dev)
    _need(count, "count", 3, torch.int32, dev)
    B, Hq, N, dq = Q.shape
    S = M0 * (1 + C + C * C)
    if Hq != H or dq != d or level0.shape != (H, M0, d) or level1.shape != (H, M0, C, d):
        raise AvqError("inconsistent shapes")
    if vsum.shape != (B, H, S, d) or count.shape != (B, H, S):
        raise AvqError("vsum / count do not match the shape")
    lib = load_library()
    workspace = _workspace(workspace, int(lib.avq_attention3_workspace_size(B, H, M0, C, d, _dt(Q))),
                           dev, "workspace")
    nt = -(-N // tile) if tile > 0 else 0
    Y = torch.empty_like(Q) if out is None else out
    _need(Y, "out", 4, dt, dev)
    if Y.shape != Q.shape:
        raise AvqError("out must have Q's shape")
    s0 = torch.empty((B, H, nt, P), dtype=torch.int32, device=dev) if want_sel else None
    s1 = torch.empty((B, H, nt, P), dtype=torch.int32, device=dev) if want_sel else None
    with _on(dev):
        _check(lib.avq_attention3_fwd(
            _ptr(Q), _ptr(level0), _ptr(level1), _ptr(leaves), _ptr(vsum), _ptr(count), B, H, N, d, M0, C, P,
            tile, float(scale), _dt(Q), _ptr(Y), _ptr(s0), _ptr(s1), _ptr(workspace), workspace.numel(),
            _stream(dev)))
    return Y, s0, s1


def forward(Q, K, V, children, P: int, tile: int, scale: float, tree=None, force_child=False):
    """Whole AVQ-Attention forward: build (or reuse) the tree, stage 1,
    stage 2.  Returns Y."""
    parents, sqnorm, frame = tree if tree is not None else build_tree(children)
    vsum, count, _ = assign_aggregate(K, V, parents, children, sqnorm, frame, force_child=force_child)
    Y, _, _ = attention_fwd(Q, parents, children, vsum, count, P, tile, scale)
    return Y
