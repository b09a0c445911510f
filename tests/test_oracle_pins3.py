"""Pins for the oracle's three-level tree (roots -> children -> leaves, the
deeper hierarchy the AVQ-Attention pages propose in Sec. 6): hand-computed
trees and assignments, brute force, the key-level form of the corrected
attention, and the reduction to the two-level tree when the leaf level adds
nothing."""

import numpy as np
import pytest

import oracle
import synth
from _refs import brute_force_assign3, key_level_vq_attention3


def test_tree3_hand_example():
    # one root, two children of two leaves each, d = 2
    leaves = np.array([[[[[0.0, 0.0], [2.0, 0.0]], [[4.0, 4.0], [6.0, 0.0]]]]])
    l0, l1, sq = oracle.build_tree3(leaves, "f32")
    np.testing.assert_array_equal(l1[0, 0], [[1.0, 0.0], [5.0, 2.0]])
    np.testing.assert_array_equal(l0[0, 0], [3.0, 1.0])
    # slots: root, child 0, child 1, four leaves
    np.testing.assert_array_equal(sq[0], [10.0, 1.0, 29.0, 0.0, 4.0, 32.0, 36.0])
    # the root is the mean of all leaves, rounded once: 1/3 in bf16
    leaves = np.zeros((1, 1, 2, 2, 1))
    leaves[0, 0, 0, 0, 0] = 4.0 / 3.0
    l0, l1, _ = oracle.build_tree3(leaves, "bf16")
    assert l0[0, 0, 0] == oracle.round_to(np.array([1.0 / 3.0]), "bf16")[0]
    assert l1[0, 0, 0, 0] == oracle.round_to(np.array([2.0 / 3.0]), "bf16")[0]


def _line_tree():
    # 1-D: root 0 has children -9 (leaves -10, -8) and -1 (leaves -2, 0);
    # root 1 has children 9 (leaves 8, 10) and 21 (leaves 20, 22)
    leaves = np.array([[[[-10.0], [-8.0]], [[-2.0], [0.0]]],
                       [[[8.0], [10.0]], [[20.0], [22.0]]]])[None]
    return leaves, oracle.build_tree3(leaves, "f32")


def test_assign3_hand_geometry():
    leaves, (l0, l1, _) = _line_tree()
    np.testing.assert_array_equal(l0[0, :, 0], [-5.0, 15.0])
    np.testing.assert_array_equal(l1[0, :, :, 0], [[-9.0, -1.0], [9.0, 21.0]])
    keys = np.array([-5.0, -7.0, -8.5, -8.0, 11.0, 15.5])
    K = keys.reshape(1, 1, -1, 1)
    a = oracle.assign3(K, l0, l1, leaves[0][None] if leaves.ndim == 6 else leaves)
    # -5: at its root; -7: child -9 is only as close as the root (4 = 4), so
    # it stays; -8.5: child -9 (0.25 < 12.25), leaf -8 only ties (0.25), so
    # it stays at the child; -8: child, then leaf -8 (0 < 1); 11: child 9
    # (4 < 16), then leaf 10 (1 < 4); 15.5: root 1 (children 42.25, 30.25)
    M0, C = 2, 2
    n1 = M0 * C
    expect = [0, 0, M0 + 0, M0 + n1 + 1, M0 + n1 + (1 * C + 0) * C + 1, 1]
    np.testing.assert_array_equal(a["leaf"][0, 0], expect)
    np.testing.assert_array_equal(a["pstar"][0, 0], [0, 0, 0, 0, 1, 1])
    assert a["gap1"][0, 0, 1] == 0.0 and a["gap2"][0, 0, 2] == 0.0
    assert np.isinf(a["gap2"][0, 0, 0]) and np.isinf(a["gap2"][0, 0, 5])
    # force_child descends regardless: -5 ties between its children (16, 16)
    # and takes child 0, then leaf -8 (9 < 25)
    f = oracle.assign3(K, l0, l1, leaves, force_child=True)
    assert f["leaf"][0, 0, 0] == M0 + n1 + 1
    assert f["leaf"][0, 0, 5] == M0 + n1 + (1 * C + 1) * C + 0


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("force", [False, True])
def test_assign3_brute_force_tiny(seed, force):
    rng = np.random.default_rng(seed)
    M0, C, d = 3, 3, 2
    # a small integer grid makes exact ties common
    leaves = rng.integers(-3, 4, size=(1, M0, C, C, d)).astype(np.float64)
    l0, l1, _ = oracle.build_tree3(leaves, "f32")
    keys = rng.integers(-4, 5, size=(40, d)).astype(np.float64)
    a = oracle.assign3(keys.reshape(1, 1, 40, d), l0, l1, leaves, force_child=force)
    ref = brute_force_assign3(keys.tolist(), l0[0].tolist(), l1[0].tolist(), leaves[0].tolist(), force)
    np.testing.assert_array_equal(a["pstar"][0, 0], [r[0] for r in ref])
    np.testing.assert_array_equal(a["leaf"][0, 0], [r[1] for r in ref])


def test_aggregate3_whole_cells():
    inp = synth.generate_dyadic3(3, N=600, M0=4, C=4)
    lv = inp.f64("children")
    l0, l1, _ = oracle.build_tree3(lv, inp.dtype)
    a = oracle.assign3(inp.f64("K"), l0, l1, lv)
    V = inp.f64("V")
    vsum, count = oracle.aggregate3(V, a["leaf"], 4, 4)
    leaf, v = a["leaf"][0, 0], V[0, 0]
    M0, C, n1 = 4, 4, 16
    root = a["pstar"][0, 0]
    child = np.where(leaf >= M0 + n1, (leaf - M0 - n1) // C, np.where(leaf >= M0, leaf - M0, -1))
    for p in range(M0):
        np.testing.assert_allclose(vsum[0, 0, p], v[root == p].sum(0), atol=1e-12)
        assert count[0, 0, p] == (root == p).sum()
    for c in range(n1):
        np.testing.assert_allclose(vsum[0, 0, M0 + c], v[child == c].sum(0), atol=1e-12)
        assert count[0, 0, M0 + c] == (child == c).sum()
    for g in range(n1 * C):
        assert count[0, 0, M0 + n1 + g] == (leaf == M0 + n1 + g).sum()
    # a child's cell contains its leaves' cells; a root's its children's
    assert (count[0, 0, M0:M0 + n1] >= count[0, 0, M0 + n1:].reshape(n1, C).sum(1)).all()
    assert (count[0, 0, :M0] >= count[0, 0, M0:M0 + n1].reshape(M0, C).sum(1)).all()
    assert count[0, 0, :M0].sum() == 600


def _pipeline3(inp, P=None, T=None):
    lv = inp.f64("children")
    l0, l1, _ = oracle.build_tree3(lv, inp.dtype)
    a = oracle.assign3(inp.f64("K"), l0, l1, lv)
    vsum, count = oracle.aggregate3(inp.f64("V"), a["leaf"], inp.M0, inp.C)
    P = inp.P if P is None else P
    T = inp.T if T is None else T
    r = oracle.attention3(inp.f64("Q"), l0, l1, lv, vsum, count, P, T, inp.scale)
    return dict(l0=l0, l1=l1, lv=lv, a=a, vsum=vsum, count=count, P=P, T=T, **r)


@pytest.mark.parametrize("P", [1, 2, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attention3_equals_key_level_form(P, dtype):
    inp = synth.generate_dyadic3(11, H=2, N=700, M0=6, C=4, T=64, dtype=dtype)
    r = _pipeline3(inp, P=P)
    # some keys stay at a root or a child, so every branch of the form is used
    leaf = r["a"]["leaf"]
    assert (leaf < 6).any() and ((leaf >= 6) & (leaf < 30)).any() and (leaf >= 30).any()
    for h in range(2):
        ref = key_level_vq_attention3(inp.f64("Q")[0, h], r["l0"][h], r["l1"][h], r["lv"][h],
                                      inp.f64("V")[0, h], r["a"]["pstar"][0, h], leaf[0, h],
                                      r["sel0"][0, h], r["sel1"][0, h], 64, inp.scale)
        np.testing.assert_allclose(r["Y"][0, h], ref, atol=1e-12, rtol=0)


def test_attention3_one_key_per_leaf_full_roots():
    # every root refined (P = M0) and P of the children: keys on leaves
    inp = synth.generate_dyadic3(12, H=1, M0=4, C=2, P=4, T=8, dtype="f32", one_key_per_leaf=True)
    r = _pipeline3(inp)
    assert (r["count"][0, 0, 4 + 8:] == 1).all()
    ref = key_level_vq_attention3(inp.f64("Q")[0, 0], r["l0"][0], r["l1"][0], r["lv"][0],
                                  inp.f64("V")[0, 0], r["a"]["pstar"][0, 0], r["a"]["leaf"][0, 0],
                                  r["sel0"][0, 0], r["sel1"][0, 0], 8, inp.scale)
    np.testing.assert_allclose(r["Y"][0, 0], ref, atol=1e-12, rtol=0)


def test_level1_importance_key_level_form_and_selection():
    inp = synth.generate_dyadic3(13, H=1, N=900, M0=6, C=4, T=128, dtype="f32")
    r = _pipeline3(inp, P=3)
    M0, C, n1, d = 6, 4, 24, inp.d
    Q, scale = inp.f64("Q")[0, 0], inp.scale
    leaf, root = r["a"]["leaf"][0, 0], r["a"]["pstar"][0, 0]
    child = np.where(leaf >= M0 + n1, (leaf - M0 - n1) // C, np.where(leaf >= M0, leaf - M0, -1))
    l1 = r["l1"][0].reshape(n1, d)
    n_child = np.bincount(child[child >= 0], minlength=n1)
    for t in range(r["imp1"].shape[2]):
        i0, i1 = t * 128, min(900, (t + 1) * 128)
        sel0 = np.sort(r["sel0"][0, 0, t])
        on1 = (child >= 0) & np.isin(root, sel0)
        rep = np.where(on1[:, None], l1[np.maximum(child, 0)], r["l0"][0][root])
        S = scale * Q[i0:i1] @ rep.T
        sh = S.max(axis=1, keepdims=True)
        Z1 = np.exp(S - sh).sum(axis=1)                       # key by key
        cands = (sel0[:, None] * C + np.arange(C)[None, :]).ravel()
        Sc = scale * Q[i0:i1] @ l1[cands].T
        w1 = (np.exp(Sc - sh) / Z1[:, None]).sum(axis=0) * n_child[cands]
        np.testing.assert_allclose(r["imp1"][0, 0, t], w1, rtol=1e-11, atol=0)
        # the selection is the P largest, ties to the lower child index
        order = np.lexsort((cands, -r["imp1"][0, 0, t]))
        np.testing.assert_array_equal(r["sel1"][0, 0, t], np.sort(cands[order[:3]]))


def test_attention3_with_copied_leaves_is_the_two_level_tree():
    base = synth.generate_dyadic(14, H=2, N=800, M0=8, C=4, T=64, dtype="bf16")
    ch = base.f64("children")                                   # [H][M0][C][d]
    leaves = np.repeat(ch[:, :, :, None, :], 4, axis=3)         # every leaf = its child
    l0, l1, _ = oracle.build_tree3(leaves, "bf16")
    par, _ = oracle.build_tree(ch, "bf16")
    np.testing.assert_array_equal(l1, ch)
    np.testing.assert_array_equal(l0, par)
    K, V, Q = base.f64("K"), base.f64("V"), base.f64("Q")
    a3 = oracle.assign3(K, l0, l1, leaves)
    a2 = oracle.assign(K, par, ch)
    np.testing.assert_array_equal(a3["leaf"], a2["leaf"])      # no key ever reaches a leaf
    v3, c3 = oracle.aggregate3(V, a3["leaf"], 8, 4)
    v2, c2 = oracle.aggregate(V, a2["leaf"], 8, 4)
    np.testing.assert_array_equal(c3[..., :40], c2)
    assert (c3[..., 40:] == 0).all()
    np.testing.assert_allclose(v3[..., :40, :], v2, atol=1e-12)
    for P in (1, 3):
        r3 = oracle.attention3(Q, l0, l1, leaves, v3, c3, P, 64, base.scale)
        Y2, _, s2 = oracle.attention(Q, par, ch, v2, c2, P, 64, base.scale)
        np.testing.assert_allclose(r3["Y"], Y2, atol=1e-12, rtol=0)
        np.testing.assert_array_equal(np.sort(r3["sel0"], -1), np.sort(s2, -1))


def test_deep_workload_recovers_generating_leaf():
    inp = synth.generate("deep-64k", H=1, N=2000)
    lv = inp.f64("children")
    l0, l1, _ = oracle.build_tree3(lv, inp.dtype)
    a = oracle.assign3(inp.f64("K"), l0, l1, lv)
    assert (a["leaf"] == inp.true_leaf).mean() > 0.95
