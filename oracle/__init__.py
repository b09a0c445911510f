"""CPU oracle for the AVQ-Attention forward pass.

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package.  The GPU library never
uses it.

The arithmetic lives in avq_oracle.c (float64, one (batch, head) unit per
call, written straight from the steps on the pages); this module compiles it
with gcc, converts arrays and runs independent (batch, head) units -- and,
for the attention, independent tile ranges -- on a thread pool (ctypes
releases the GIL during each call).  No arithmetic of the method happens in
Python here.

Parity pins: every function below is checked against closed forms, brute
force and invariants in tests/test_oracle_pins.py.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "avq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libavq_oracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build() -> str:
    """Compile avq_oracle.c into oracle/libavq_oracle.so (strict IEEE fp64:
    no fast-math, no FMA contraction)."""
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off",
                           "-fno-fast-math", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if (not os.path.exists(_LIB_PATH)
                    or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
                build()
            lib = ctypes.CDLL(_LIB_PATH)
            lib.avqo_round_bf16.restype = ctypes.c_double
            lib.avqo_round_bf16.argtypes = [ctypes.c_double]
            lib.avqo_round.argtypes = [_dp, ctypes.c_int64, ctypes.c_int, _dp]
            lib.avqo_build_tree.argtypes = [_dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, _dp]
            lib.avqo_sqnorm.argtypes = [_dp, ctypes.c_int64, ctypes.c_int, _dp]
            lib.avqo_assign.argtypes = [_dp, ctypes.c_int64, ctypes.c_int, _dp, _dp,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        _i32p, _i32p, _dp, _dp]
            lib.avqo_aggregate.argtypes = [_dp, ctypes.c_int64, ctypes.c_int, _i32p,
                                           ctypes.c_int, ctypes.c_int, _dp, _i64p]
            lib.avqo_attention.restype = ctypes.c_int
            lib.avqo_attention.argtypes = [_dp, ctypes.c_int64, ctypes.c_int, _dp, _dp,
                                           ctypes.c_int, ctypes.c_int, _dp, _i64p,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_double, _i32p,
                                           ctypes.c_int64, ctypes.c_int64,
                                           _dp, _dp, _i32p]
            lib.avqo_commitment.restype = ctypes.c_double
            lib.avqo_commitment.argtypes = [_dp, ctypes.c_int64, ctypes.c_int, _dp, _dp,
                                            ctypes.c_int, ctypes.c_int, _i32p]
            lib.avqo_active_ratio.restype = ctypes.c_double
            lib.avqo_active_ratio.argtypes = [_i64p, ctypes.c_int, ctypes.c_int64, ctypes.c_double]
            lib.avqo_capture.restype = ctypes.c_int
            lib.avqo_capture.argtypes = [_dp, _dp, ctypes.c_int64, ctypes.c_int, _i32p, _i32p,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                         _dp]
            lib.avqo_gilbert_order.argtypes = [ctypes.c_int, ctypes.c_int, _i32p]
            lib.avqo_build_tree3.argtypes = [_dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, _dp, _dp]
            lib.avqo_assign3.argtypes = [_dp, ctypes.c_int64, ctypes.c_int, _dp, _dp, _dp,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         _i32p, _i32p, _dp, _dp, _dp]
            lib.avqo_aggregate3.argtypes = [_dp, ctypes.c_int64, ctypes.c_int, _i32p,
                                            ctypes.c_int, ctypes.c_int, _dp, _i64p]
            lib.avqo_attention3.restype = ctypes.c_int
            lib.avqo_attention3.argtypes = [_dp, ctypes.c_int64, ctypes.c_int, _dp, _dp, _dp,
                                            ctypes.c_int, ctypes.c_int, _dp, _i64p,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                            _i32p, _i32p, ctypes.c_int64, ctypes.c_int64,
                                            _dp, _dp, _i32p, _dp, _i32p]
            _lib = lib
    return _lib


def _p(a, t):
    return a.ctypes.data_as(t) if a is not None else ctypes.cast(None, t)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def default_threads() -> int:
    """Host threads for independent units: the CPUs this process may use,
    at most 16 (one GPU's share of a GPU host)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def _run(fn, units, threads):
    threads = threads or default_threads()
    if threads == 1 or len(units) == 1:
        for u in units:
            fn(u)
        return
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fn, units))


# ---------------------------------------------------------------------------

def round_to(x, dtype: str) -> np.ndarray:
    """Round float64 values to the storage dtype ('f32' or 'bf16'), ties to even."""
    lib = _load()
    x = _f64(x)
    out = np.empty_like(x)
    lib.avqo_round(_p(x, _dp), x.size, 1 if dtype == "bf16" else 0, _p(out, _dp))
    return out


def build_tree(children, dtype: str):
    """children [H][M0][C][d] float64 -> (parents [H][M0][d] rounded to dtype,
    sqnorm [H][M0(1+C)] float64: parents first, then children).

    A flat codebook (plain VQ, no children) is passed as [H][M0][d]: its
    codewords are the parents, C = 0."""
    lib = _load()
    children = _f64(children)
    if children.ndim == 3:
        H, M0, d = children.shape
        sq = np.empty((H, M0))
        for h in range(H):
            lib.avqo_sqnorm(_p(children[h], _dp), M0, d, _p(sq[h], _dp))
        return children.copy(), sq
    H, M0, C, d = children.shape
    parents = np.empty((H, M0, d))
    sq = np.empty((H, M0 * (1 + C)))
    for h in range(H):
        lib.avqo_build_tree(_p(children[h], _dp), M0, C, d, 1 if dtype == "bf16" else 0,
                            _p(parents[h], _dp))
        lib.avqo_sqnorm(_p(parents[h], _dp), M0, d, _p(sq[h, :M0], _dp))
        tmp = np.empty(M0 * C)
        lib.avqo_sqnorm(_p(children[h], _dp), M0 * C, d, _p(tmp, _dp))
        sq[h, M0:] = tmp
    return parents, sq


def _tree_shape(children):
    """(M0, C) of a tree's children array, C = 0 for a flat [H][M0][d] codebook."""
    return (children.shape[1], 0) if children.ndim == 3 else (children.shape[1], children.shape[2])


def assign(K, parents, children, force_child: bool = False, threads: Optional[int] = None):
    """K [B][H][N][d] -> dict of [B][H][N] arrays: pstar, leaf (int32),
    gap_parent, gap_leaf (float64 relative top-2 gaps)."""
    lib = _load()
    K, parents, children = _f64(K), _f64(parents), _f64(children)
    B, H, N, d = K.shape
    M0, C = _tree_shape(children)
    out = {k: np.empty((B, H, N), dtype=np.int32) for k in ("pstar", "leaf")}
    out.update({k: np.empty((B, H, N)) for k in ("gap_parent", "gap_leaf")})

    def unit(bh):
        b, h = bh
        lib.avqo_assign(_p(K[b, h], _dp), N, d, _p(parents[h], _dp), _p(children[h], _dp),
                        M0, C, 1 if force_child else 0,
                        _p(out["pstar"][b, h], _i32p), _p(out["leaf"][b, h], _i32p),
                        _p(out["gap_parent"][b, h], _dp), _p(out["gap_leaf"][b, h], _dp))

    _run(unit, [(b, h) for b in range(B) for h in range(H)], threads)
    return out


def aggregate(V, leaf, M0: int, C: int, threads: Optional[int] = None):
    """V [B][H][N][d], leaf [B][H][N] -> (vsum [B][H][S_tot][d] float64,
    count [B][H][S_tot] int64)."""
    lib = _load()
    V = _f64(V)
    leaf = np.ascontiguousarray(leaf, dtype=np.int32)
    B, H, N, d = V.shape
    S = M0 * (1 + C)
    vsum = np.empty((B, H, S, d))
    count = np.empty((B, H, S), dtype=np.int64)

    def unit(bh):
        b, h = bh
        lib.avqo_aggregate(_p(V[b, h], _dp), N, d, _p(leaf[b, h], _i32p), M0, C,
                           _p(vsum[b, h], _dp), _p(count[b, h], _i64p))

    _run(unit, [(b, h) for b in range(B) for h in range(H)], threads)
    return vsum, count


def attention(Q, parents, children, vsum, count, P: int, T: int, scale: float,
              forced_sel=None, tiles=None, threads: Optional[int] = None):
    """Q [B][H][N][d] -> (Y [B][H][N][d], importance [B][H][ntiles][M0],
    sel [B][H][ntiles][P]).  `tiles` = (t_begin, t_end) restricts the work
    to those query tiles (other rows of Y are NaN).  `forced_sel`
    [B][H][ntiles][P] replaces the top-P choice."""
    lib = _load()
    Q, parents, children, vsum = _f64(Q), _f64(parents), _f64(children), _f64(vsum)
    count = np.ascontiguousarray(count, dtype=np.int64)
    B, H, N, d = Q.shape
    M0, C = _tree_shape(children)
    nt = -(-N // T)
    t0, t1 = tiles if tiles is not None else (0, nt)
    Y = np.full((B, H, N, d), np.nan)
    imp = np.zeros((B, H, nt, M0))
    sel = np.zeros((B, H, nt, max(P, 0)), dtype=np.int32)
    fs = None if forced_sel is None else np.ascontiguousarray(forced_sel, dtype=np.int32)
    threads = threads or default_threads()
    nunits_bh = B * H
    # split tiles so that every thread has work
    per = max(1, -(-(t1 - t0) * nunits_bh // (4 * threads)))
    units = [(b, h, a, min(a + per, t1)) for b in range(B) for h in range(H)
             for a in range(t0, t1, per)]

    def unit(u):
        b, h, a, e = u
        rc = lib.avqo_attention(_p(Q[b, h], _dp), N, d, _p(parents[h], _dp),
                                _p(children[h], _dp), M0, C, _p(vsum[b, h], _dp),
                                _p(count[b, h], _i64p), P, T, float(scale),
                                _p(fs[b, h] if fs is not None else None, _i32p),
                                a, e, _p(Y[b, h], _dp), _p(imp[b, h], _dp),
                                _p(sel[b, h], _i32p))
        if rc != 0:
            raise MemoryError("oracle attention allocation failed")

    _run(unit, units, threads)
    return Y, imp, sel


def commitment(K, parents, children, leaf, threads: Optional[int] = None):
    """K [B][H][N][d], leaf [B][H][N] -> [B][H]: mean over the keys of the
    squared distance to the assigned leaf codeword (Table 7's E||k - k_hat||^2)."""
    lib = _load()
    K, parents, children = _f64(K), _f64(parents), _f64(children)
    leaf = np.ascontiguousarray(leaf, dtype=np.int32)
    B, H, N, d = K.shape
    M0, C = _tree_shape(children)
    out = np.empty((B, H))

    def unit(bh):
        b, h = bh
        out[b, h] = lib.avqo_commitment(_p(K[b, h], _dp), N, d, _p(parents[h], _dp),
                                        _p(children[h], _dp), M0, C, _p(leaf[b, h], _i32p))

    _run(unit, [(b, h) for b in range(B) for h in range(H)], threads)
    return out


def active_ratio(count, N: int, share: float = 0.01):
    """count [B][H][S_tot] -> [B][H]: fraction of codewords whose count
    exceeds share * N / S_tot (Table 9's active ratio, share = 1 %)."""
    lib = _load()
    count = np.ascontiguousarray(count, dtype=np.int64)
    B, H, S = count.shape
    out = np.empty((B, H))
    for b in range(B):
        for h in range(H):
            out[b, h] = lib.avqo_active_ratio(_p(count[b, h], _i64p), S, N, share)
    return out


def capture(Q, K, pstar, sel, T: int, scale: float, M0: int, threads: Optional[int] = None):
    """Q, K [B][H][N][d], pstar [B][H][N], sel [B][H][ntiles][P] -> [B][H][N]:
    each query's fraction of exact softmax weight on keys whose parent its
    tile selected (Sec. 5.2, Table 6 "capture").  O(N^2 d): small N only."""
    lib = _load()
    Q, K = _f64(Q), _f64(K)
    pstar = np.ascontiguousarray(pstar, dtype=np.int32)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    B, H, N, d = Q.shape
    P = sel.shape[-1]
    out = np.empty((B, H, N))

    def unit(bh):
        b, h = bh
        rc = lib.avqo_capture(_p(Q[b, h], _dp), _p(K[b, h], _dp), N, d, _p(pstar[b, h], _i32p),
                              _p(sel[b, h], _i32p), P, T, float(scale), M0, _p(out[b, h], _dp))
        if rc != 0:
            raise MemoryError("oracle capture allocation failed")

    _run(unit, [(b, h) for b in range(B) for h in range(H)], threads)
    return out


def gilbert_order(W: int, H: int) -> np.ndarray:
    """Row-major cell indices y*W + x of a W x H grid in the order of the
    generalized Hilbert curve (the pages' token reordering, ref. [4])."""
    lib = _load()
    out = np.empty(W * H, dtype=np.int32)
    lib.avqo_gilbert_order(W, H, _p(out, _i32p))
    return out


# ---------------------------------------------------------------------------
# three-level tree (roots -> children -> leaves)

def build_tree3(leaves, dtype: str):
    """leaves [H][M0][C][C][d] float64 -> (level0 [H][M0][d], level1
    [H][M0][C][d], sqnorm [H][M0(1+C+C^2)]: roots, children, leaves), the two
    upper levels rounded to dtype."""
    lib = _load()
    leaves = _f64(leaves)
    H, M0, C, _, d = leaves.shape
    l0 = np.empty((H, M0, d))
    l1 = np.empty((H, M0, C, d))
    n1 = M0 * C
    sq = np.empty((H, M0 + n1 + n1 * C))
    for h in range(H):
        lib.avqo_build_tree3(_p(leaves[h], _dp), M0, C, d, 1 if dtype == "bf16" else 0,
                             _p(l1[h], _dp), _p(l0[h], _dp))
        for lo, rows, n in ((0, l0[h], M0), (M0, l1[h], n1), (M0 + n1, leaves[h], n1 * C)):
            tmp = np.empty(n)
            lib.avqo_sqnorm(_p(np.ascontiguousarray(rows), _dp), n, d, _p(tmp, _dp))
            sq[h, lo:lo + n] = tmp
    return l0, l1, sq


def assign3(K, level0, level1, leaves, force_child: bool = False, threads: Optional[int] = None):
    """K [B][H][N][d] -> dict of [B][H][N] arrays: pstar, leaf (int32, slot
    in the three-level layout), gap0, gap1, gap2 (relative top-2 gaps at
    each level; gap2 is +inf for keys that stayed at their root)."""
    lib = _load()
    K, level0, level1, leaves = _f64(K), _f64(level0), _f64(level1), _f64(leaves)
    B, H, N, d = K.shape
    M0, C = leaves.shape[1], leaves.shape[2]
    out = {k: np.empty((B, H, N), dtype=np.int32) for k in ("pstar", "leaf")}
    out.update({k: np.empty((B, H, N)) for k in ("gap0", "gap1", "gap2")})

    def unit(bh):
        b, h = bh
        lib.avqo_assign3(_p(K[b, h], _dp), N, d, _p(level0[h], _dp), _p(level1[h], _dp),
                         _p(leaves[h], _dp), M0, C, 1 if force_child else 0,
                         _p(out["pstar"][b, h], _i32p), _p(out["leaf"][b, h], _i32p),
                         _p(out["gap0"][b, h], _dp), _p(out["gap1"][b, h], _dp),
                         _p(out["gap2"][b, h], _dp))

    _run(unit, [(b, h) for b in range(B) for h in range(H)], threads)
    return out


def aggregate3(V, leaf, M0: int, C: int, threads: Optional[int] = None):
    """V [B][H][N][d], leaf [B][H][N] (three-level slots) -> (vsum
    [B][H][S3][d], count [B][H][S3]) with every slot holding its whole cell."""
    lib = _load()
    V = _f64(V)
    leaf = np.ascontiguousarray(leaf, dtype=np.int32)
    B, H, N, d = V.shape
    S = M0 * (1 + C + C * C)
    vsum = np.empty((B, H, S, d))
    count = np.empty((B, H, S), dtype=np.int64)

    def unit(bh):
        b, h = bh
        lib.avqo_aggregate3(_p(V[b, h], _dp), N, d, _p(leaf[b, h], _i32p), M0, C,
                            _p(vsum[b, h], _dp), _p(count[b, h], _i64p))

    _run(unit, [(b, h) for b in range(B) for h in range(H)], threads)
    return vsum, count


def attention3(Q, level0, level1, leaves, vsum, count, P: int, T: int, scale: float,
               forced_sel0=None, forced_sel1=None, tiles=None, threads: Optional[int] = None):
    """Q [B][H][N][d] -> dict: Y [B][H][N][d]; imp0 [B][H][ntiles][M0] and
    sel0 [B][H][ntiles][P] (roots, sel0 in importance order); imp1
    [B][H][ntiles][P*C] (children of the selected roots by ascending index)
    and sel1 [B][H][ntiles][P] (selected children p*C + a, ascending).
    `tiles` = (t_begin, t_end) restricts the work (other rows of Y are NaN)."""
    lib = _load()
    Q, level0, level1, leaves, vsum = _f64(Q), _f64(level0), _f64(level1), _f64(leaves), _f64(vsum)
    count = np.ascontiguousarray(count, dtype=np.int64)
    B, H, N, d = Q.shape
    M0, C = leaves.shape[1], leaves.shape[2]
    nt = -(-N // T)
    t0, t1 = tiles if tiles is not None else (0, nt)
    Y = np.full((B, H, N, d), np.nan)
    imp0 = np.zeros((B, H, nt, M0))
    sel0 = np.zeros((B, H, nt, P), dtype=np.int32)
    imp1 = np.zeros((B, H, nt, P * C))
    sel1 = np.zeros((B, H, nt, P), dtype=np.int32)
    f0 = None if forced_sel0 is None else np.ascontiguousarray(forced_sel0, dtype=np.int32)
    f1 = None if forced_sel1 is None else np.ascontiguousarray(forced_sel1, dtype=np.int32)
    threads = threads or default_threads()
    per = max(1, -(-(t1 - t0) * B * H // (4 * threads)))
    units = [(b, h, a, min(a + per, t1)) for b in range(B) for h in range(H)
             for a in range(t0, t1, per)]

    def unit(u):
        b, h, a, e = u
        rc = lib.avqo_attention3(_p(Q[b, h], _dp), N, d, _p(level0[h], _dp), _p(level1[h], _dp),
                                 _p(leaves[h], _dp), M0, C, _p(vsum[b, h], _dp),
                                 _p(count[b, h], _i64p), P, T, float(scale),
                                 _p(f0[b, h] if f0 is not None else None, _i32p),
                                 _p(f1[b, h] if f1 is not None else None, _i32p),
                                 a, e, _p(Y[b, h], _dp), _p(imp0[b, h], _dp), _p(sel0[b, h], _i32p),
                                 _p(imp1[b, h], _dp), _p(sel1[b, h], _i32p))
        if rc != 0:
            raise MemoryError("oracle attention allocation failed")

    _run(unit, units, threads)
    return dict(Y=Y, imp0=imp0, sel0=sel0, imp1=imp1, sel1=sel1)


def forward3(inp, P: Optional[int] = None, T: Optional[int] = None, force_child=False,
             threads: Optional[int] = None, tiles=None):
    """Whole three-level forward pass on a `synth.Inputs` workload whose
    `children` holds the leaves [H][M0][C][C][d]."""
    from synth import storage_to_f64
    lv = storage_to_f64(inp.children, inp.dtype)
    l0, l1, sq = build_tree3(lv, inp.dtype)
    P = inp.P if P is None else P
    T = inp.T if T is None else T
    a = assign3(storage_to_f64(inp.K, inp.dtype), l0, l1, lv, force_child, threads)
    vsum, count = aggregate3(storage_to_f64(inp.V, inp.dtype), a["leaf"], inp.M0, inp.C, threads)
    att = attention3(storage_to_f64(inp.Q, inp.dtype), l0, l1, lv, vsum, count, P, T, inp.scale,
                     tiles=tiles, threads=threads)
    return dict(level0=l0, level1=l1, sqnorm=sq, vsum=vsum, count=count, **a, **att)


def forward(inp, P: Optional[int] = None, T: Optional[int] = None, force_child=False,
            threads: Optional[int] = None, forced_sel=None, parents=None):
    """Whole forward pass on an `synth.Inputs` workload.  `parents` (float64,
    [H][M0][d]) may be given to run steps O2-O8 on an externally supplied
    tree; by default the oracle's own O1 tree is used."""
    from synth import storage_to_f64
    ch = storage_to_f64(inp.children, inp.dtype)
    par, sq = build_tree(ch, inp.dtype)
    if parents is not None:
        par = _f64(parents)
    P = inp.P if P is None else P
    T = inp.T if T is None else T
    a = assign(storage_to_f64(inp.K, inp.dtype), par, ch, force_child, threads)
    vsum, count = aggregate(storage_to_f64(inp.V, inp.dtype), a["leaf"], inp.M0, inp.C, threads)
    Y, imp, sel = attention(storage_to_f64(inp.Q, inp.dtype), par, ch, vsum, count, P, T,
                            inp.scale, forced_sel=forced_sel, threads=threads)
    return dict(parents=par, sqnorm=sq, vsum=vsum, count=count, Y=Y, importance=imp,
                sel=sel, **a)
