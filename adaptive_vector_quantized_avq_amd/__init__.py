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
    "build_tree", "assign_aggregate", "attention_fwd", "exact_attention_fwd",
    "assign_aggregate_workspace_size", "operand_pack_size", "forward",
    "AVQ_FLAG_FORCE_CHILD",
]

AVQ_FLAG_FORCE_CHILD = 1
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
    lib.avq_build_tree.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.avq_assign_aggregate_workspace_size.restype = sz
    lib.avq_assign_aggregate_workspace_size.argtypes = [i32] * 6
    lib.avq_assign_aggregate.restype = i32
    lib.avq_operand_pack_size.restype = sz
    lib.avq_operand_pack_size.argtypes = [i32] * 6
    lib.avq_assign_aggregate.restype = i32
    lib.avq_assign_aggregate.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, u32,
                                         vp, vp, vp, vp, vp, sz, vp]
    lib.avq_attention_fwd.restype = i32
    lib.avq_attention_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                      f32, i32, vp, vp, vp, vp]
    lib.avq_exact_attention_fwd.restype = i32
    lib.avq_exact_attention_fwd.argtypes = [vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, vp]
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


def build_tree(children: torch.Tensor):
    """children [H][M0][C][d] -> (parents [H][M0][d], sqnorm [H][M0(1+C)] fp32)."""
    _need(children, "children", 4)
    H, M0, C, d = children.shape
    parents = torch.empty((H, M0, d), dtype=children.dtype, device=children.device)
    sqnorm = torch.empty((H, M0 * (1 + C)), dtype=torch.float32, device=children.device)
    with _on(children.device):
        _check(load_library().avq_build_tree(_ptr(children), H, M0, C, d, _dt(children), _ptr(parents),
                                             _ptr(sqnorm), _stream(children.device)))
    return parents, sqnorm


def assign_aggregate_workspace_size(B, H, N, M0, C, d) -> int:
    return int(load_library().avq_assign_aggregate_workspace_size(B, H, N, M0, C, d))


def operand_pack_size(B, H, M0, C, d, dtype) -> int:
    return int(load_library().avq_operand_pack_size(B, H, M0, C, d, _DTYPES[dtype]))


def assign_aggregate(K, V, parents, children, sqnorm, force_child: bool = False,
                     want_leaf: bool = False, workspace: Optional[torch.Tensor] = None,
                     out: Optional[tuple] = None):
    """Stage 1.  K, V [B][H][N][d] -> (vsum [B][H][S_tot][d] fp32,
    count [B][H][S_tot] int32, leaf [B][H][N] int32 or None, pack uint8: the
    same aggregates laid out as stage-2 operands)."""
    _need(K, "K", 4)
    dev, dt = K.device, K.dtype
    _need(V, "V", 4, dt, dev)
    _need(children, "children", 4, dt, dev)
    _need(parents, "parents", 3, dt, dev)
    _need(sqnorm, "sqnorm", 2, torch.float32, dev)
    B, H, N, d = K.shape
    M0, C = children.shape[1], children.shape[2]
    if V.shape != K.shape or children.shape[0] != H or children.shape[3] != d or \
            parents.shape != (H, M0, d) or sqnorm.shape != (H, M0 * (1 + C)):
        raise AvqError("inconsistent shapes")
    S = M0 * (1 + C)
    lib = load_library()
    need = int(lib.avq_assign_aggregate_workspace_size(B, H, N, M0, C, d))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if out is None:
        vsum = torch.empty((B, H, S, d), dtype=torch.float32, device=dev)
        count = torch.empty((B, H, S), dtype=torch.int32, device=dev)
        pack = torch.empty(int(lib.avq_operand_pack_size(B, H, M0, C, d, _dt(K))), dtype=torch.uint8,
                           device=dev)
    else:
        vsum, count, pack = out
        _need(vsum, "vsum", 4, torch.float32, dev)
        _need(count, "count", 3, torch.int32, dev)
        _need(pack, "pack", 1, torch.uint8, dev)
        if vsum.shape != (B, H, S, d) or count.shape != (B, H, S) or \
                pack.numel() < int(lib.avq_operand_pack_size(B, H, M0, C, d, _dt(K))):
            raise AvqError("output buffers do not match the shape")
    _need(workspace, "workspace", 1, torch.uint8, dev)
    leaf = torch.empty((B, H, N), dtype=torch.int32, device=dev) if want_leaf else None
    with _on(dev):
        _check(lib.avq_assign_aggregate(
            _ptr(K), _ptr(V), _ptr(parents), _ptr(children), _ptr(sqnorm), B, H, N, d, M0, C, _dt(K),
            AVQ_FLAG_FORCE_CHILD if force_child else 0, _ptr(vsum), _ptr(count), _ptr(leaf), _ptr(pack),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev)))
    return vsum, count, leaf, pack


def attention_fwd(Q, parents, children, pack, P: int, tile: int, scale: float,
                  want_sel: bool = False, want_importance: bool = False,
                  out: Optional[torch.Tensor] = None):
    """Stage 2.  Q [B][H][N][d] and the operand pack of stage 1 ->
    (Y [B][H][N][d], sel [B][H][ntiles][P] or None,
    importance [B][H][ntiles][M0] or None)."""
    _need(Q, "Q", 4)
    dev, dt = Q.device, Q.dtype
    _need(children, "children", 4, dt, dev)
    _need(parents, "parents", 3, dt, dev)
    _need(pack, "pack", 1, torch.uint8, dev)
    B, H, N, d = Q.shape
    M0, C = children.shape[1], children.shape[2]
    if parents.shape != (H, M0, d) or children.shape[0] != H or children.shape[3] != d:
        raise AvqError("inconsistent shapes")
    if pack.numel() < int(load_library().avq_operand_pack_size(B, H, M0, C, d, _dt(Q))):
        raise AvqError("operand pack too small for this shape")
    nt = -(-N // tile) if tile > 0 else 0
    Y = torch.empty_like(Q) if out is None else out
    _need(Y, "out", 4, dt, dev)
    if Y.shape != Q.shape:
        raise AvqError("out must have Q's shape")
    sel = torch.empty((B, H, nt, P), dtype=torch.int32, device=dev) if want_sel else None
    imp = torch.empty((B, H, nt, M0), dtype=torch.float32, device=dev) if want_importance else None
    with _on(dev):
        _check(load_library().avq_attention_fwd(
            _ptr(Q), _ptr(parents), _ptr(children), _ptr(pack), B, H, N, d, M0, C, P, tile,
            float(scale), _dt(Q), _ptr(Y), _ptr(sel), _ptr(imp), _stream(dev)))
    return Y, sel, imp


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


def forward(Q, K, V, children, P: int, tile: int, scale: float, tree=None, force_child=False):
    """Whole AVQ-Attention forward: build (or reuse) the tree, stage 1,
    stage 2.  Returns Y."""
    parents, sqnorm = tree if tree is not None else build_tree(children)
    _, _, _, pack = assign_aggregate(K, V, parents, children, sqnorm, force_child=force_child)
    Y, _, _ = attention_fwd(Q, parents, children, pack, P, tile, scale)
    return Y
