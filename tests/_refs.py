"""Independent reference formulations used to pin the oracle (tests only).

These are *different* formulations of what the oracle computes, not copies of
it: the oracle works on aggregated codewords (value sums and counts) with an
online max and a child-for-parent correction, while the references below work
key by key on the quantised keys, or are textbook softmax attention.
"""

import numpy as np


def softmax_attention(Q, K, V, scale):
    """Textbook softmax attention for one head: Q [n][d], K, V [N][d]
    ("AVQ-Attention", Sec. 3.1)."""
    S = scale * Q @ K.T
    S -= S.max(axis=1, keepdims=True)
    A = np.exp(S)
    return (A @ V) / A.sum(axis=1, keepdims=True)


def key_level_vq_attention(Q, parents, children, V, pstar, leaf, sel, T, scale):
    """Softmax attention of each query over the *keys*, every key replaced by
    its representative codeword (Sec. 3.2: attention with K_hat).  In a tile
    whose selection contains the key's parent the representative is the key's
    leaf (child or the parent itself); otherwise it is the parent.
    Q [N][d], parents [M0][d], children [M0][C][d], sel [ntiles][P]."""
    N, d = Q.shape
    M0, C = children.shape[0], children.shape[1]
    flat = children.reshape(M0 * C, d)
    Y = np.empty((N, d))
    for t in range(-(-N // T)):
        i0, i1 = t * T, min(N, (t + 1) * T)
        refined = np.isin(pstar, np.asarray(sel[t], dtype=np.int64))
        rep = np.where((leaf >= M0)[:, None] & refined[:, None],
                       flat[np.maximum(leaf - M0, 0)], parents[pstar])
        Y[i0:i1] = softmax_attention(Q[i0:i1], rep, V, scale)
    return Y


def brute_force_assign(keys, parents, children, force_child=False):
    """Pure-Python two-stage assignment for tiny inputs: parents ranked by
    (distance, index); then the chosen parent's children ranked the same way;
    a child wins only when strictly closer (or always with force_child)."""
    M0 = len(parents)
    C = len(children[0])

    def dist(a, b):
        return sum((x - y) * (x - y) for x, y in zip(a, b))

    out = []
    for k in keys:
        p = sorted(range(M0), key=lambda j: (dist(k, parents[j]), j))[0]
        c = sorted(range(C), key=lambda j: (dist(k, children[p][j]), j))[0]
        if force_child or dist(k, children[p][c]) < dist(k, parents[p]):
            out.append((p, M0 + p * C + c))
        else:
            out.append((p, p))
    return out


def key_level_vq_attention3(Q, level0, level1, leaves, V, pstar, leaf, sel0, sel1, T, scale):
    """Three-level tree, key by key: in each tile every key is represented by
    the deepest *active* codeword on its path -- its root; its child if the
    tile refined that root (sel0); its leaf if the tile also refined that
    child (sel1).  With every codeword the exact mean of the ones below it
    (a recovered logit then equals the direct one), the corrected
    attention over aggregates is exactly softmax attention over these
    representatives.  Q [N][d], level0 [M0][d], level1 [M0][C][d], leaves
    [M0][C][C][d], leaf in the three-level slot layout."""
    N, d = Q.shape
    M0, C = leaves.shape[0], leaves.shape[1]
    n1 = M0 * C
    l1 = level1.reshape(n1, d)
    lv = leaves.reshape(n1 * C, d)
    child = np.where(leaf >= M0 + n1, (leaf - M0 - n1) // C, np.where(leaf >= M0, leaf - M0, -1))
    gidx = np.where(leaf >= M0 + n1, leaf - M0 - n1, -1)
    Y = np.empty((N, d))
    for t in range(-(-N // T)):
        i0, i1 = t * T, min(N, (t + 1) * T)
        on1 = (child >= 0) & np.isin(pstar, np.asarray(sel0[t], dtype=np.int64))
        on2 = on1 & (gidx >= 0) & np.isin(child, np.asarray(sel1[t], dtype=np.int64))
        rep = level0[pstar]
        rep = np.where(on1[:, None], l1[np.maximum(child, 0)], rep)
        rep = np.where(on2[:, None], lv[np.maximum(gidx, 0)], rep)
        Y[i0:i1] = softmax_attention(Q[i0:i1], rep, V, scale)
    return Y


def brute_force_assign3(keys, level0, level1, leaves, force_child=False):
    """Pure-Python descent for tiny inputs: nearest root by (distance, index);
    then its children the same way, taken only when strictly closer than the
    root (always with force_child); then, from a child, its leaves the same
    way against the child.  Returns (root, slot) per key in the three-level
    slot layout."""
    M0, C = len(level0), len(level1[0])

    def dist(a, b):
        return sum((x - y) * (x - y) for x, y in zip(a, b))

    def nearest(cands, k):
        return sorted(range(len(cands)), key=lambda j: (dist(k, cands[j]), j))[0]

    out = []
    for k in keys:
        p = nearest(level0, k)
        a = nearest(level1[p], k)
        if not (force_child or dist(k, level1[p][a]) < dist(k, level0[p])):
            out.append((p, p))
            continue
        b = nearest(leaves[p][a], k)
        if force_child or dist(k, leaves[p][a][b]) < dist(k, level1[p][a]):
            out.append((p, M0 + M0 * C + (p * C + a) * C + b))
        else:
            out.append((p, M0 + p * C + a))
    return out
