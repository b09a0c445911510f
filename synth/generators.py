"""Seeded synthetic workloads shaped like the vision-transformer layers the
AVQ-Attention pages time and evaluate.

The pages ("AVQ-Attention: Adaptive Vector-Quantized Attention", Sec. 5 and
Table 2) run ViT-B (N=785), DPT-L (N=901), SD1.5 U-Nets (N up to ~16k) and a
kernel timing sweep (B=4, H=12, D=64, N up to 65,536).  None of those datasets
or trained codebooks exist here, so each workload below draws a frozen
parent/child codebook and Q/K/V from fixed distributions (NumPy PCG64,
fixed seed) with the same shapes.

Draw order is fixed: first the codebook of every head (parents, child
offsets, and the per-head Zipf ranking or per-leaf scales when used), then
for every (b, h) in row-major order: key leaves, key noise, query parents,
query noise, values.  Everything is drawn in float64 and rounded once to the
storage dtype (round-to-nearest-even).

Storage convention: "f32" tensors are numpy float32; "bf16" tensors are numpy
uint16 arrays holding the bf16 bit patterns.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

# name -> shape and distribution recipe.  The seed is 1000 + position in
# WORKLOAD_ORDER.
WORKLOADS = {
    # fp32, small enough for the CPU oracle in well under a second.
    "tiny-f32": dict(B=1, H=1, N=1024, d=64, M0=16, C=4, P=4, T=64,
                     dtype="f32", keys="uniform", queries="parent"),
    # ViT-B-like layer on a 64x64 patch grid.
    "vit-b": dict(B=1, H=12, N=4096, d=64, M0=64, C=8, P=8, T=128,
                  dtype="bf16", keys="uniform", queries="clustered"),
    # Segmentation-resolution layer with Zipf(1.1)-skewed leaf occupancy;
    # swept over P in {0, 4, 16, 128}.
    "seg-zipf": dict(B=2, H=16, N=16384, d=64, M0=128, C=8, P=16, T=128,
                     dtype="bf16", keys="zipf", queries="clustered",
                     P_sweep=(0, 4, 16, 128)),
    # Long-sequence layer on a 256x256 token grid (the headline shape).
    "long-64k": dict(B=1, H=8, N=65536, d=64, M0=256, C=8, P=16, T=128,
                     dtype="bf16", keys="uniform", queries="clustered"),
    # Wide-head diffusion-like layer: d=128, 16 children per parent,
    # anisotropic per-leaf key spread.
    "wide-d128": dict(B=2, H=10, N=32768, d=128, M0=256, C=16, P=32, T=64,
                      dtype="bf16", keys="anisotropic", queries="clustered"),
    # Flat VQ-attention (no children, C = 0) at the long-sequence shape: the
    # pages' fixed-codebook baseline with M = 256 codewords (Table 2).
    "flat-64k": dict(B=1, H=8, N=65536, d=64, M0=256, C=0, P=0, T=128,
                     dtype="bf16", keys="uniform", queries="clustered"),
    # Three-level tree (roots -> children -> leaves, the deeper hierarchy
    # the pages propose as the next step, Sec. 6) at the long-sequence
    # shape, with the pages' 64/16/8 root configuration: 64 roots, 512
    # children, 4096 leaves per head; P = 16 refinements at each level.
    "deep-64k": dict(B=1, H=8, N=65536, d=64, M0=64, C=8, P=16, T=128,
                     dtype="bf16", keys="uniform", queries="clustered", levels=3),
}
WORKLOAD_ORDER = ["tiny-f32", "vit-b", "seg-zipf", "long-64k", "wide-d128"]
# further workloads (not among the five the parity suite sweeps by name)
EXTRA_WORKLOADS = ["flat-64k", "deep-64k"]

CHILD_SPREAD = 0.3      # std of child offsets around their parent
LEAF_SPREAD = 0.15      # std of leaf offsets around their child (three-level trees)
KEY_SPREAD = 0.1        # std of key noise around its generating leaf
QUERY_SPREAD = 0.5      # std of query noise around its parent
ZIPF_EXPONENT = 1.1
ANISO_RANGE = (0.05, 0.3)
QUERY_PARENTS_PER_TILE = 4


# ---------------------------------------------------------------------------
# storage-format conversions (bit manipulation only)
# ---------------------------------------------------------------------------

def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bf16 (ties to even) and return the bit patterns
    as uint16.  Values are assumed to lie in bf16's normal range or be zero."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    b = x.view(np.uint64)
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    r = (b + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    f = r.view(np.float64).astype(np.float32)          # exact: r fits in bf16
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(u) -> np.ndarray:
    u = np.ascontiguousarray(np.asarray(u, dtype=np.uint16))
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x64, dtype=np.float32)
    if dtype == "bf16":
        return f64_to_bf16_bits(x64)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# workload container
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Inputs:
    name: str
    B: int
    H: int
    N: int
    d: int
    M0: int
    C: int
    P: int
    T: int
    dtype: str
    scale: float
    seed: int
    children: np.ndarray      # [H][M0][C][d] storage dtype ([H][M0][d] for a flat codebook, C = 0;
                              # the leaves [H][M0][C][C][d] of a three-level tree)
    Q: np.ndarray             # [B][H][N][d]
    K: np.ndarray
    V: np.ndarray
    true_leaf: np.ndarray     # [B][H][N] int32: slot of the generating leaf (M0 + p*C + c; p if C = 0;
                              # M0 + M0*C + (p*C + a)*C + b for a three-level tree)
    levels: int = 2

    @property
    def S_tot(self) -> int:
        if self.levels == 3:
            return self.M0 * (1 + self.C + self.C * self.C)
        return self.M0 * (1 + self.C)

    @property
    def ntiles(self) -> int:
        return -(-self.N // self.T)

    def f64(self, field: str) -> np.ndarray:
        return storage_to_f64(getattr(self, field), self.dtype)


def _zipf_probs(L: int) -> np.ndarray:
    w = np.arange(1, L + 1, dtype=np.float64) ** (-ZIPF_EXPONENT)
    return w / w.sum()


def _clustered_query_parents(rng, N, T, M0):
    ntiles = -(-N // T)
    k = min(QUERY_PARENTS_PER_TILE, M0)
    # k distinct parents per tile: first k entries of a random permutation
    cand = np.argsort(rng.random((ntiles, M0)), axis=1)[:, :k]
    pick = rng.integers(0, k, size=N)
    tile = np.arange(N) // T
    return cand[tile, pick]


def generate(name: str, seed: Optional[int] = None, **overrides) -> Inputs:
    """Draw the named workload.  `overrides` may change any shape field
    (B, H, N, d, M0, C, P, T, dtype, keys, queries) to get a smaller instance
    with the same structure."""
    spec = dict(WORKLOADS[name])
    spec.pop("P_sweep", None)
    spec.update(overrides)
    if seed is None:
        seed = 1000 + (WORKLOAD_ORDER + EXTRA_WORKLOADS).index(name)
    B, H, N, d = spec["B"], spec["H"], spec["N"], spec["d"]
    M0, C, P, T = spec["M0"], spec["C"], spec["P"], spec["T"]
    dtype = spec["dtype"]
    levels = spec.get("levels", 2)
    rng = np.random.Generator(np.random.PCG64(seed))
    flat_vq = C == 0          # a flat codebook: the M0 codewords are the leaves
    deep = levels == 3        # roots -> children -> leaves
    if deep and flat_vq:
        raise ValueError("a three-level tree needs C > 0")
    L = M0 if flat_vq else M0 * C * (C if deep else 1)

    parents64 = np.empty((H, M0, d))
    children64 = np.empty((H, M0, C, d))
    leaves64 = np.empty((H, M0, C, C, d)) if deep else None
    zipf_perm = [None] * H
    aniso = [None] * H
    for h in range(H):
        par = rng.standard_normal((M0, d))
        parents64[h] = par
        if not flat_vq:
            off = rng.normal(0.0, CHILD_SPREAD, size=(M0, C, d))
            off -= off.mean(axis=1, keepdims=True)
            children64[h] = par[:, None, :] + off
        if deep:
            off2 = rng.normal(0.0, LEAF_SPREAD, size=(M0, C, C, d))
            off2 -= off2.mean(axis=2, keepdims=True)
            leaves64[h] = children64[h][:, :, None, :] + off2
        if spec["keys"] == "zipf":
            zipf_perm[h] = rng.permutation(L)
        elif spec["keys"] == "anisotropic":
            aniso[h] = rng.uniform(ANISO_RANGE[0], ANISO_RANGE[1], size=(L, d))

    st = np.uint16 if dtype == "bf16" else np.float32
    Q = np.empty((B, H, N, d), dtype=st)
    K = np.empty((B, H, N, d), dtype=st)
    V = np.empty((B, H, N, d), dtype=st)
    true_leaf = np.empty((B, H, N), dtype=np.int32)
    zp = _zipf_probs(L) if spec["keys"] == "zipf" else None

    for b in range(B):
        for h in range(H):
            flat = (parents64[h] if flat_vq else
                    leaves64[h].reshape(L, d) if deep else children64[h].reshape(L, d))
            if spec["keys"] == "zipf":
                rank = rng.choice(L, size=N, p=zp)
                leaf = zipf_perm[h][rank]
            else:
                leaf = rng.integers(0, L, size=N)
            noise = rng.standard_normal((N, d))
            if spec["keys"] == "anisotropic":
                k64 = flat[leaf] + aniso[h][leaf] * noise
            else:
                k64 = flat[leaf] + KEY_SPREAD * noise
            if spec["queries"] == "clustered":
                qp = _clustered_query_parents(rng, N, T, M0)
            else:
                qp = rng.integers(0, M0, size=N)
            q64 = parents64[h][qp] + QUERY_SPREAD * rng.standard_normal((N, d))
            v64 = rng.standard_normal((N, d))
            K[b, h] = to_storage(k64, dtype)
            Q[b, h] = to_storage(q64, dtype)
            V[b, h] = to_storage(v64, dtype)
            true_leaf[b, h] = (leaf if flat_vq else
                               M0 + M0 * C + leaf if deep else M0 + leaf)

    # a flat codebook is passed as [H][M0][d]: its codewords are the parents;
    # a three-level tree as its leaves [H][M0][C][C][d]
    codebook = parents64 if flat_vq else leaves64 if deep else children64
    return Inputs(name=name, B=B, H=H, N=N, d=d, M0=M0, C=C, P=P, T=T,
                  dtype=dtype, scale=1.0 / math.sqrt(d), seed=seed,
                  children=to_storage(codebook, dtype), Q=Q, K=K, V=V,
                  true_leaf=true_leaf, levels=levels)


def generate_dyadic(seed: int, B=1, H=1, N=256, d=64, M0=8, C=4, P=2, T=64,
                    dtype="bf16") -> Inputs:
    """Codebook whose coordinates are multiples of 1/8 with |x| < 32, the last
    child of every parent chosen so the children average exactly to the
    parent.  Every coordinate is then exact in bf16 and fp32, and so is the
    mean.  Keys, queries and values are drawn as in `generate` (uniform
    leaves, queries around a random parent)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    L = M0 * C
    children64 = np.empty((H, M0, C, d))
    parents64 = np.empty((H, M0, d))
    for h in range(H):
        par = np.clip(np.round(rng.standard_normal((M0, d)) * 8) / 8, -8, 8)
        off = np.clip(np.round(rng.normal(0, CHILD_SPREAD, (M0, C, d)) * 8) / 8, -2, 2)
        off[:, C - 1, :] = -off[:, : C - 1, :].sum(axis=1)
        parents64[h] = par
        children64[h] = par[:, None, :] + off
    st = np.uint16 if dtype == "bf16" else np.float32
    Q = np.empty((B, H, N, d), dtype=st)
    K = np.empty_like(Q)
    V = np.empty_like(Q)
    true_leaf = np.empty((B, H, N), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            flat = children64[h].reshape(L, d)
            leaf = rng.integers(0, L, size=N)
            k64 = flat[leaf] + KEY_SPREAD * rng.standard_normal((N, d))
            qp = rng.integers(0, M0, size=N)
            q64 = parents64[h][qp] + QUERY_SPREAD * rng.standard_normal((N, d))
            v64 = rng.standard_normal((N, d))
            K[b, h] = to_storage(k64, dtype)
            Q[b, h] = to_storage(q64, dtype)
            V[b, h] = to_storage(v64, dtype)
            true_leaf[b, h] = M0 + leaf
    return Inputs(name="dyadic", B=B, H=H, N=N, d=d, M0=M0, C=C, P=P, T=T,
                  dtype=dtype, scale=1.0 / math.sqrt(d), seed=seed,
                  children=to_storage(children64, dtype), Q=Q, K=K, V=V,
                  true_leaf=true_leaf)


def generate_one_key_per_leaf(seed: int, B=1, H=1, d=64, M0=8, C=4, T=64,
                              dtype="bf16", dyadic=True) -> Inputs:
    """N = M0*C keys, key l placed exactly on child l (leaf order), so every
    leaf holds exactly one key.  With a dyadic codebook the parent is the
    exact mean of its children."""
    base = generate_dyadic(seed, B=B, H=H, N=M0 * C, d=d, M0=M0, C=C, P=M0,
                           T=T, dtype=dtype) if dyadic else None
    if base is None:
        raise NotImplementedError("only the dyadic codebook is supported")
    L = M0 * C
    for b in range(B):
        for h in range(H):
            base.K[b, h] = base.children[h].reshape(L, d)
            base.true_leaf[b, h] = M0 + np.arange(L, dtype=np.int32)
    base.name = "one-key-per-leaf"
    return base


def generate_dyadic3(seed: int, B=1, H=1, N=256, d=64, M0=4, C=4, P=2, T=64,
                     dtype="bf16", one_key_per_leaf=False, upper_share=0.25) -> Inputs:
    """Three-level tree whose coordinates are multiples of 1/8 with |x| < 32:
    the last child of every root and the last leaf of every child are chosen
    so that each level averages exactly to the one above.  Every coordinate,
    and every mean, is then exact in bf16 and fp32.  Keys are drawn around
    uniformly chosen leaves, except that a share `upper_share` of them is
    drawn around a random root or a random child (half each), so that some
    keys stay above the leaf level (or, with one_key_per_leaf, N = M0*C*C
    keys are placed exactly on the leaves in leaf order); queries around a
    random root; values standard normal."""
    rng = np.random.Generator(np.random.PCG64(seed))
    L = M0 * C * C
    leaves64 = np.empty((H, M0, C, C, d))
    mids64 = np.empty((H, M0, C, d))
    roots64 = np.empty((H, M0, d))
    for h in range(H):
        root = np.clip(np.round(rng.standard_normal((M0, d)) * 8) / 8, -4, 4)
        off = np.clip(np.round(rng.normal(0, CHILD_SPREAD, (M0, C, d)) * 8) / 8, -1, 1)
        off[:, C - 1, :] = -off[:, : C - 1, :].sum(axis=1)
        off2 = np.clip(np.round(rng.normal(0, LEAF_SPREAD, (M0, C, C, d)) * 8) / 8, -1, 1)
        off2[:, :, C - 1, :] = -off2[:, :, : C - 1, :].sum(axis=2)
        roots64[h] = root
        mids64[h] = root[:, None, :] + off
        leaves64[h] = mids64[h][:, :, None, :] + off2
    if one_key_per_leaf:
        N = L
    st = np.uint16 if dtype == "bf16" else np.float32
    Q = np.empty((B, H, N, d), dtype=st)
    K = np.empty_like(Q)
    V = np.empty_like(Q)
    true_leaf = np.empty((B, H, N), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            flat = leaves64[h].reshape(L, d)
            if one_key_per_leaf:
                leaf = np.arange(L)
                k64 = flat.copy()
            else:
                leaf = rng.integers(0, L, size=N)
                centre = flat[leaf]
                kind = rng.random(N)
                up_root = kind < upper_share / 2
                up_child = (kind >= upper_share / 2) & (kind < upper_share)
                centre[up_root] = roots64[h][leaf[up_root] // (C * C)]
                centre[up_child] = mids64[h].reshape(M0 * C, d)[leaf[up_child] // C]
                k64 = centre + KEY_SPREAD * rng.standard_normal((N, d))
            qp = rng.integers(0, M0, size=N)
            q64 = roots64[h][qp] + QUERY_SPREAD * rng.standard_normal((N, d))
            v64 = rng.standard_normal((N, d))
            K[b, h] = to_storage(k64, dtype)
            Q[b, h] = to_storage(q64, dtype)
            V[b, h] = to_storage(v64, dtype)
            true_leaf[b, h] = M0 + M0 * C + leaf
    return Inputs(name="dyadic3", B=B, H=H, N=N, d=d, M0=M0, C=C, P=P, T=T,
                  dtype=dtype, scale=1.0 / math.sqrt(d), seed=seed,
                  children=to_storage(leaves64, dtype), Q=Q, K=K, V=V,
                  true_leaf=true_leaf, levels=3)
