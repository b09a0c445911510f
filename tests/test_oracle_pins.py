"""Pins for the CPU oracle: closed forms, key-level reformulations, brute
force and invariants fixed by the AVQ-Attention pages and by mathematics.
None of these re-types the oracle's own formulas."""

import json
import os
import random

import numpy as np
import pytest

import oracle
import synth
from _refs import brute_force_assign, key_level_vq_attention, softmax_attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- rounding

def test_round_bf16_hand_values():
    cases = {
        1.0 + 2 ** -8: 1.0,                      # halfway, even neighbour 1.0
        1.0 + 3 * 2 ** -8: 1.0 + 2 ** -6,        # halfway, even neighbour above
        1.0 + 2 ** -8 + 2 ** -30: 1.0 + 2 ** -7,  # just above halfway
        -(1.0 + 2 ** -8): -1.0,
        1.0 / 3.0: 0.333984375,
        0.0: 0.0,
        2.0 ** -130: 2.0 ** -130,                # bf16 subnormal, exact
        255.0 / 8: 255.0 / 8,                    # 8 significant bits, exact
    }
    x = np.array(list(cases.keys()))
    np.testing.assert_array_equal(oracle.round_to(x, "bf16"), np.array(list(cases.values())))


def test_round_bf16_agrees_with_bitwise_rounding():
    # two independent implementations: frexp-based (oracle) and integer
    # bit arithmetic (input generator)
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        (rng.integers(-2 ** 12, 2 ** 12, 4000) + 0.5) * 2.0 ** -7])
    ref = synth.bf16_bits_to_f64(synth.f64_to_bf16_bits(x))
    np.testing.assert_array_equal(oracle.round_to(x, "bf16"), ref)


def test_round_f32_is_ieee_single():
    x = np.random.default_rng(1).standard_normal(10000) * 1e3
    np.testing.assert_array_equal(oracle.round_to(x, "f32"), x.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------- tree (O1)

def test_tree_hand_example():
    # two parents, two children each, d = 2
    ch = np.array([[[1.0, 2.0], [1.0 + 2 ** -7, 6.0]],
                   [[1.0 + 2 ** -7, -3.0], [1.0 + 2 ** -6, 5.0]]])[None]
    par, sq = oracle.build_tree(ch, "bf16")
    # means: (1 + 2^-8, 4) -> ties to 1.0 ; (1 + 3*2^-8, 1) -> ties to 1 + 2^-6
    np.testing.assert_array_equal(par[0], [[1.0, 4.0], [1.0 + 2 ** -6, 1.0]])
    np.testing.assert_array_equal(sq[0, :2], [1.0 + 16.0, (1.0 + 2 ** -6) ** 2 + 1.0])
    np.testing.assert_array_equal(sq[0, 2:], [5.0, (1 + 2 ** -7) ** 2 + 36.0,
                                              (1 + 2 ** -7) ** 2 + 9.0, (1 + 2 ** -6) ** 2 + 25.0])


def test_tree_dyadic_mean_is_exact_and_recovers_parent_logit():
    inp = synth.generate_dyadic(3, H=2, M0=8, C=4, d=64)
    ch = inp.f64("children")
    par, _ = oracle.build_tree(ch, "bf16")
    q = np.random.default_rng(2).integers(-64, 64, size=(16, 64)) / 8.0
    # Child attention identity: q.C_p equals the mean over c of q.C_pc, exactly
    lhs = np.einsum("qd,hpd->hqp", q, par)
    rhs = np.einsum("qd,hpcd->hqpc", q, ch).sum(axis=3) / 4
    np.testing.assert_array_equal(lhs, rhs)


def test_tree_invariances():
    rng = np.random.default_rng(4)
    ch = rng.standard_normal((2, 5, 8, 16))
    par, _ = oracle.build_tree(ch, "f32")
    par2, _ = oracle.build_tree(ch[:, :, rng.permutation(8), :], "f32")
    np.testing.assert_array_equal(par, par2)
    const = np.repeat(rng.standard_normal((1, 3, 1, 16)), 4, axis=2)
    p3, _ = oracle.build_tree(const, "f32")
    np.testing.assert_array_equal(p3[0], const[0, :, 0, :].astype(np.float32))


# ---------------------------------------------------------------- assignment (O2)

@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_assign_recovers_generating_leaf(name):
    small = dict(B=1, H=2, N=2048)
    if name == "wide-d128":
        small["N"] = 1024
    inp = synth.generate(name, **small)
    ch = inp.f64("children")
    par, _ = oracle.build_tree(ch, inp.dtype)
    a = oracle.assign(inp.f64("K"), par, ch)
    assert (a["leaf"] == inp.true_leaf).all()
    assert (a["pstar"] == (inp.true_leaf - inp.M0) // inp.C).all()
    assert a["gap_parent"].min() > 1e-2 and a["gap_leaf"].min() > 1e-2


def test_assign_hand_geometry():
    # d = 2; parent 0 at the origin with children (+-1, 0); parent 1 at (10, 0)
    # with children (11, 0), (9, 0).  Slots: 0, 1 parents; 2, 3 children of
    # parent 0; 4, 5 children of parent 1.
    ch = np.array([[[[1.0, 0.0], [-1.0, 0.0]], [[11.0, 0.0], [9.0, 0.0]]]])
    par, _ = oracle.build_tree(ch, "f32")
    np.testing.assert_array_equal(par[0], [[0, 0], [10, 0]])
    keys = np.array([[0.9, 0.0],    # nearest parent 0, child 0 closer -> slot 2
                     [0.0, 0.0],    # on the parent -> stays (residual) -> slot 0
                     [0.0, 1.0],    # parent dist 1 < children dist 2 -> slot 0
                     [5.0, 0.0],    # tie between parents -> parent 0, child 0 -> 2
                     [5.5, 0.0],    # parent 1, its child (9,0) -> slot 5
                     [0.5, 0.0],    # child ties with parent: not strictly closer -> 0
                     [-3.0, 0.0]])  # parent 0, child 1 -> slot 3
    a = oracle.assign(keys[None, None], par, ch)
    assert a["leaf"][0, 0].tolist() == [2, 0, 0, 2, 5, 0, 3]
    assert a["pstar"][0, 0].tolist() == [0, 0, 0, 0, 1, 0, 0]
    f = oracle.assign(keys[None, None], par, ch, force_child=True)
    assert f["leaf"][0, 0].tolist() == [2, 2, 2, 2, 5, 2, 3]
    # the tie cases report a zero gap
    assert a["gap_parent"][0, 0, 3] == 0.0 and a["gap_leaf"][0, 0, 5] == 0.0


def test_assign_relative_gap_hand_values():
    # The near-tie measure is (D_(2) - D_(1)) / D_(2), normalised by the
    # second-smallest distance.  Key at the origin, d = 2; parents at squared
    # distances 4, 1, 9 (best not listed first), each with two children at
    # +-0.5 across the parent, i.e. 0.25 farther than it.
    ch = np.array([[[[2.0, 0.5], [2.0, -0.5]],
                    [[1.0, 0.5], [1.0, -0.5]],
                    [[3.0, 0.5], [3.0, -0.5]]]])
    par, _ = oracle.build_tree(ch, "f32")
    np.testing.assert_array_equal(par[0], [[2, 0], [1, 0], [3, 0]])
    a = oracle.assign(np.zeros((1, 1, 1, 2)), par, ch)
    assert a["pstar"][0, 0, 0] == 1 and a["leaf"][0, 0, 0] == 1
    assert a["gap_parent"][0, 0, 0] == 0.75          # (4 - 1) / 4, not (4 - 1) / 1
    assert a["gap_leaf"][0, 0, 0] == 0.2             # {1, 1.25, 1.25}: (1.25 - 1) / 1.25
    # parents at squared distances 1, 2, 5 give (2 - 1) / 2
    ch2 = np.array([[[[1.0, 0.5], [1.0, -0.5]],
                     [[1.0, 1.5], [1.0, 0.5]],
                     [[2.0, 1.5], [2.0, 0.5]]]])
    par2, _ = oracle.build_tree(ch2, "f32")
    b = oracle.assign(np.zeros((1, 1, 1, 2)), par2, ch2)
    assert b["gap_parent"][0, 0, 0] == 0.5
    # with the parent excluded (force_child) the two children tie: gap 0
    f = oracle.assign(np.zeros((1, 1, 1, 2)), par, ch, force_child=True)
    assert f["leaf"][0, 0, 0] == 3 + 1 * 2 and f["gap_leaf"][0, 0, 0] == 0.0


@pytest.mark.parametrize("seed", range(6))
def test_assign_brute_force_tiny(seed):
    rnd = random.Random(seed)
    M0, C, d, N = rnd.randint(1, 4), rnd.randint(1, 3), rnd.randint(1, 4), 64
    # small integer grid: many exact ties
    ch = [[[rnd.randint(-3, 3) for _ in range(d)] for _ in range(C)] for _ in range(M0)]
    par, _ = oracle.build_tree(np.array(ch, dtype=np.float64)[None], "f32")
    keys = [[rnd.randint(-4, 4) for _ in range(d)] for _ in range(N)]
    for force in (False, True):
        a = oracle.assign(np.array(keys, dtype=np.float64)[None, None], par, np.array(ch, float)[None],
                          force_child=force)
        ref = brute_force_assign(keys, par[0].tolist(), ch, force_child=force)
        assert list(zip(a["pstar"][0, 0].tolist(), a["leaf"][0, 0].tolist())) == ref


# ---------------------------------------------------------------- aggregation (O3)

def test_aggregate_conservation_and_brute_force():
    inp = synth.generate("seg-zipf", B=1, H=2, N=4096)
    ch = inp.f64("children")
    par, _ = oracle.build_tree(ch, inp.dtype)
    a = oracle.assign(inp.f64("K"), par, ch)
    V = inp.f64("V")
    vsum, count = oracle.aggregate(V, a["leaf"], inp.M0, inp.C)
    M0, C = inp.M0, inp.C
    for h in range(2):
        n_par = count[0, h, :M0]
        n_ch = count[0, h, M0:].reshape(M0, C)
        assert n_par.sum() == inp.N
        resid = n_par - n_ch.sum(axis=1)
        assert (resid >= 0).all()
        np.testing.assert_allclose(vsum[0, h, :M0].sum(axis=0), V[0, h].sum(axis=0), atol=1e-9)
        # every slot against a masked sum over its keys
        for slot in list(range(M0)) + list(range(M0, M0 * (1 + C), 7)):
            if slot < M0:
                mask = a["pstar"][0, h] == slot
            else:
                mask = a["leaf"][0, h] == slot
            assert count[0, h, slot] == mask.sum()
            np.testing.assert_allclose(vsum[0, h, slot], V[0, h][mask].sum(axis=0), atol=1e-9)
    # Zipf skew: the fullest leaf holds a large share of the keys
    assert count[0, :, M0:].max() > 0.1 * inp.N


# ---------------------------------------------------------------- attention (O4-O8)

def _pipeline(inp, P=None, T=None, V=None):
    ch = inp.f64("children")
    par, _ = oracle.build_tree(ch, inp.dtype)
    a = oracle.assign(inp.f64("K"), par, ch)
    V = inp.f64("V") if V is None else V
    vsum, count = oracle.aggregate(V, a["leaf"], inp.M0, inp.C)
    P = inp.P if P is None else P
    T = inp.T if T is None else T
    Y, w, sel = oracle.attention(inp.f64("Q"), par, ch, vsum, count, P, T, inp.scale)
    return dict(par=par, ch=ch, a=a, vsum=vsum, count=count, Y=Y, w=w, sel=sel, V=V, P=P, T=T)


def test_P0_equals_parent_level_vq_attention():
    inp = synth.generate("vit-b", H=2, N=1000, T=128)
    r = _pipeline(inp, P=0)
    for h in range(2):
        ref = key_level_vq_attention(inp.f64("Q")[0, h], r["par"][h], r["ch"][h], r["V"][0, h],
                                     r["a"]["pstar"][0, h], r["a"]["leaf"][0, h],
                                     np.zeros((r["w"].shape[2], 0), int), 128, inp.scale)
        np.testing.assert_allclose(r["Y"][0, h], ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("P", [1, 3, 8])
def test_dyadic_tree_equals_key_level_form(P):
    inp = synth.generate_dyadic(7, H=2, N=700, M0=8, C=4, T=64)
    r = _pipeline(inp, P=P)
    for h in range(2):
        ref = key_level_vq_attention(inp.f64("Q")[0, h], r["par"][h], r["ch"][h], r["V"][0, h],
                                     r["a"]["pstar"][0, h], r["a"]["leaf"][0, h],
                                     r["sel"][0, h], 64, inp.scale)
        np.testing.assert_allclose(r["Y"][0, h], ref, atol=1e-12, rtol=0)


def test_full_spawning_equals_child_level_vq_attention():
    inp = synth.generate_dyadic(8, H=1, N=500, M0=6, C=4, T=32, dtype="f32")
    r = _pipeline(inp, P=6)
    M0, C = 6, 4
    leaf = r["a"]["leaf"][0, 0]
    flat = r["ch"][0].reshape(M0 * C, -1)
    rep = np.where((leaf >= M0)[:, None], flat[np.maximum(leaf - M0, 0)],
                   r["par"][0][np.minimum(leaf, M0 - 1)])
    ref = softmax_attention(inp.f64("Q")[0, 0], rep, r["V"][0, 0], inp.scale)
    np.testing.assert_allclose(r["Y"][0, 0], ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_key_per_leaf_is_exact_softmax_attention(dtype):
    inp = synth.generate_one_key_per_leaf(9, H=2, M0=8, C=4, d=64, T=16, dtype=dtype)
    r = _pipeline(inp, P=8)
    assert (r["count"][0, :, 8:] == 1).all()
    for h in range(2):
        ref = softmax_attention(inp.f64("Q")[0, h], inp.f64("K")[0, h], r["V"][0, h], inp.scale)
        np.testing.assert_allclose(r["Y"][0, h], ref, atol=1e-12, rtol=0)


def test_importance_mass_and_empty_parents():
    inp = synth.generate("vit-b", H=1, N=1000, T=128)
    # keys only around the first 16 parents' children -> parents 16.. are empty
    K = inp.f64("K")
    ch = inp.f64("children")
    rng = np.random.default_rng(5)
    leafs = rng.integers(0, 16 * inp.C, size=1000)
    K[0, 0] = ch[0].reshape(-1, inp.d)[leafs] + 0.1 * rng.standard_normal((1000, inp.d))
    par, _ = oracle.build_tree(ch, inp.dtype)
    a = oracle.assign(K, par, ch)
    vsum, count = oracle.aggregate(inp.f64("V"), a["leaf"], inp.M0, inp.C)
    Y, w, sel = oracle.attention(inp.f64("Q"), par, ch, vsum, count, 8, 128, inp.scale)
    sizes = [128] * 7 + [1000 - 7 * 128]
    np.testing.assert_allclose(w[0, 0].sum(axis=1), sizes, rtol=1e-12)
    assert (w >= 0).all()
    empty = count[0, 0, :inp.M0] == 0
    assert empty.sum() >= 40 and (w[0, 0][:, empty] == 0).all()
    assert not np.isin(sel[0, 0], np.nonzero(empty)[0]).any()


def test_selection_is_top_P_and_nested():
    inp = synth.generate("seg-zipf", B=1, H=2, N=2048)
    sels = {}
    for P in (0, 4, 16, 128):
        r = _pipeline(inp, P=P)
        w = r["w"]
        for h in range(2):
            for t in range(w.shape[2]):
                order = sorted(range(inp.M0), key=lambda j: (-w[0, h, t, j], j))
                assert r["sel"][0, h, t].tolist() == order[:P]
        sels[P] = r["sel"]
    for t in range(sels[4].shape[2]):
        for h in range(2):
            assert set(sels[4][0, h, t]) <= set(sels[16][0, h, t]) <= set(sels[128][0, h, t])
    assert sels[128].shape[-1] == 128


@pytest.mark.parametrize("P", [0, 2, 16])
def test_constant_values_give_constant_output(P):
    inp = synth.generate("tiny-f32", N=512, M0=16, C=4, T=64)
    V = np.full((1, 1, 512, 64), 0.375)
    r = _pipeline(inp, P=P, V=V)
    np.testing.assert_allclose(r["Y"], 0.375, atol=1e-12)


def test_linearity_in_values():
    inp = synth.generate("tiny-f32", N=512)
    rng = np.random.default_rng(6)
    V1, V2 = rng.standard_normal((2, 1, 1, 512, 64))
    r1 = _pipeline(inp, V=V1)
    r2 = _pipeline(inp, V=V2)
    r3 = _pipeline(inp, V=2.0 * V1 - 3.0 * V2)
    assert (r1["sel"] == r3["sel"]).all()
    np.testing.assert_allclose(r3["Y"], 2.0 * r1["Y"] - 3.0 * r2["Y"], atol=1e-10)


def test_key_permutation_and_tile_independence():
    inp = synth.generate("vit-b", H=1, N=1024, T=128)
    r = _pipeline(inp)
    perm = np.random.default_rng(7).permutation(1024)
    inp2 = synth.generate("vit-b", H=1, N=1024, T=128)
    inp2.K = inp.K[:, :, perm]
    inp2.V = inp.V[:, :, perm]
    r2 = _pipeline(inp2)
    assert (r["count"] == r2["count"]).all() and (r["sel"] == r2["sel"]).all()
    np.testing.assert_allclose(r2["Y"], r["Y"], atol=1e-10)
    # tiles 3..5 alone
    Y, w, sel = oracle.attention(inp.f64("Q"), r["par"], r["ch"], r["vsum"], r["count"],
                                 inp.P, 128, inp.scale, tiles=(3, 6))
    np.testing.assert_array_equal(Y[:, :, 384:768], r["Y"][:, :, 384:768])
    assert np.isnan(Y[:, :, :384]).all()


def test_forced_selection_reproduces_natural_selection():
    inp = synth.generate("vit-b", H=1, N=512, T=128)
    r = _pipeline(inp)
    Y, w, sel = oracle.attention(inp.f64("Q"), r["par"], r["ch"], r["vsum"], r["count"],
                                 inp.P, 128, inp.scale, forced_sel=r["sel"][:, :, :, ::-1])
    np.testing.assert_allclose(Y, r["Y"], atol=1e-12)


def test_worked_example_codeword_counts():
    """The pages' worked example: a 64/16/8 tree stores 576 codewords and a
    query interacts with 64 parents plus 128 children = 192 of them."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example_64_16_8.json")))
    inp = synth.generate("vit-b", H=1, N=256, T=128, M0=g["M0"], C=g["C"], P=g["P"])
    r = _pipeline(inp)
    assert r["count"].shape[-1] == g["stored_codewords"]
    # perturb the aggregates of one codeword at a time: the output of tile 0
    # changes exactly for the 64 parents and the 16*8 children of the
    # selected parents -- 192 codewords
    base = r["Y"][0, 0, :128]
    influential = 0
    for slot in range(g["stored_codewords"]):
        vs = r["vsum"].copy()
        vs[0, 0, slot] += 1.0
        Y, _, _ = oracle.attention(inp.f64("Q"), r["par"], r["ch"], vs, r["count"], g["P"], 128,
                                   inp.scale, tiles=(0, 1), threads=1)
        if np.abs(Y[0, 0, :128] - base).max() > 0:
            influential += 1
    assert influential == g["interactions_per_query"]
    assert len(r["sel"][0, 0, 0]) * g["C"] == g["refining_children"]


def test_scale_argument_is_applied():
    inp = synth.generate_dyadic(11, H=1, N=300, M0=4, C=2, d=64, T=64, P=2)
    inp.scale = 0.05
    r = _pipeline(inp)
    ref = key_level_vq_attention(inp.f64("Q")[0, 0], r["par"][0], r["ch"][0], r["V"][0, 0],
                                 r["a"]["pstar"][0, 0], r["a"]["leaf"][0, 0], r["sel"][0, 0],
                                 64, 0.05)
    np.testing.assert_allclose(r["Y"][0, 0], ref, atol=1e-12)
    assert np.isfinite(r["Y"]).all()


# ---------------------------------------------------------------- inputs

@pytest.mark.parametrize("name", ["tiny-f32", "vit-b", "seg-zipf", "wide-d128"])
def test_generators_are_deterministic_per_seed(name):
    # the same seed reproduces every tensor bit for bit; another seed does not
    small = dict(B=1, H=1, N=300)
    a, b = synth.generate(name, seed=5, **small), synth.generate(name, seed=5, **small)
    c = synth.generate(name, seed=6, **small)
    for f in ("children", "Q", "K", "V", "true_leaf"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
        assert not np.array_equal(getattr(a, f), getattr(c, f)), f
    d1 = synth.generate_dyadic(3, N=100)
    d2 = synth.generate_dyadic(3, N=100)
    for f in ("children", "Q", "K", "V"):
        np.testing.assert_array_equal(getattr(d1, f), getattr(d2, f))


# ---------------------------------------------------------------- flat VQ (C = 0)

@pytest.mark.parametrize("seed", range(4))
def test_flat_vq_assignment_brute_force(seed):
    # plain VQ (Sec. 3.2): every key goes to its nearest codeword, ties to the
    # lowest index; small integer grids make exact ties common
    rnd = random.Random(100 + seed)
    M0, d, N = rnd.randint(1, 6), rnd.randint(1, 4), 80
    cb = [[rnd.randint(-3, 3) for _ in range(d)] for _ in range(M0)]
    keys = [[rnd.randint(-4, 4) for _ in range(d)] for _ in range(N)]
    par, _ = oracle.build_tree(np.array(cb, dtype=np.float64)[None], "f32")
    a = oracle.assign(np.array(keys, dtype=np.float64)[None, None], par, par)
    dist = lambda x, y: sum((u - v) ** 2 for u, v in zip(x, y))
    ref = [min(range(M0), key=lambda j: (dist(k, cb[j]), j)) for k in keys]
    assert a["leaf"][0, 0].tolist() == ref and a["pstar"][0, 0].tolist() == ref
    assert np.isinf(a["gap_leaf"]).all()


def test_flat_vq_recovers_generating_codeword():
    inp = synth.generate("flat-64k", H=2, N=2048)
    par, _ = oracle.build_tree(inp.f64("children"), inp.dtype)
    a = oracle.assign(inp.f64("K"), par, inp.f64("children"))
    assert (a["leaf"] == inp.true_leaf).all()


def test_flat_vq_attention_is_key_level_vq_attention():
    # Sec. 3.2: attention with every key replaced by its nearest codeword,
    # summed over keys (no aggregation), equals the count-weighted attention
    # over the codewords
    inp = synth.generate("flat-64k", B=1, H=2, N=700, M0=24, T=64, seed=9)
    r = oracle.forward(inp)
    cb, Q, V = inp.f64("children"), inp.f64("Q"), inp.f64("V")
    for h in range(inp.H):
        ref = softmax_attention(Q[0, h], cb[h][r["pstar"][0, h]], V[0, h], inp.scale)
        assert np.abs(r["Y"][0, h] - ref).max() < 1e-10
    # constant-rank invariants: counts sum to N, the value sums to the total
    assert (r["count"].sum(axis=-1) == inp.N).all()
    np.testing.assert_allclose(r["vsum"].sum(axis=2), V.sum(axis=2), rtol=1e-12, atol=1e-9)


def test_flat_codebook_is_the_parent_level_of_a_tree():
    # a flat codebook made of a tree's parents gives the tree's P = 0 result
    tree = synth.generate_dyadic(12, B=1, H=2, N=900, d=64, M0=8, C=4, P=0, T=64, dtype="f32")
    t = oracle.forward(tree, P=0)
    flat = synth.Inputs(**{**tree.__dict__})
    flat.C = 0
    flat.children = synth.to_storage(t["parents"], "f32")
    f = oracle.forward(flat, P=0)
    assert (f["pstar"] == t["pstar"]).all()
    np.testing.assert_array_equal(f["count"], t["count"][..., :tree.M0])
    assert np.abs(f["Y"] - t["Y"]).max() < 1e-12


# ---------------------------------------------------------------- diagnostics

def test_commitment_hand_values_and_zero_on_codewords():
    # d = 2, one parent at the origin with children (+-1, 0): key (0.75, 0)
    # -> child (1, 0) at 0.0625; key (0, 2) -> stays at the parent at 4
    # (children at 5); mean 2.03125
    ch = np.array([[[[1.0, 0.0], [-1.0, 0.0]]]])
    par, _ = oracle.build_tree(ch, "f32")
    keys = np.array([[0.75, 0.0], [0.0, 2.0]])[None, None]
    a = oracle.assign(keys, par, ch)
    assert a["leaf"][0, 0].tolist() == [1, 0]
    assert oracle.commitment(keys, par, ch, a["leaf"])[0, 0] == 2.03125
    # keys placed exactly on leaves: zero loss
    inp = synth.generate_one_key_per_leaf(7, H=2, d=64, M0=8, C=4, dtype="f32")
    r = oracle.forward(inp)
    assert (oracle.commitment(inp.f64("K"), r["parents"], inp.f64("children"), r["leaf"]) == 0).all()


def test_commitment_flat_is_mean_nearest_distance():
    # flat codebook: the loss is the mean squared distance to the nearest
    # codeword, by brute force
    rng = np.random.default_rng(5)
    cb = rng.standard_normal((1, 7, 3))
    K = rng.standard_normal((1, 1, 50, 3))
    par, _ = oracle.build_tree(cb, "f32")
    a = oracle.assign(K, par, cb)
    ref = np.mean([min(((k - c) ** 2).sum() for c in cb[0]) for k in K[0, 0]])
    assert abs(oracle.commitment(K, par, cb, a["leaf"])[0, 0] - ref) < 1e-12


def test_active_ratio_hand_values():
    # 4 codewords, N = 400: fair share 100, threshold 1 key; counts {0, 1, 2, 397}
    c = np.array([[[0, 1, 2, 397]]])
    assert oracle.active_ratio(c, 400)[0, 0] == 0.5          # only counts > 1
    assert oracle.active_ratio(c, 400, share=0.0)[0, 0] == 0.75


def test_capture_limits_and_softmax_reformulation():
    inp = synth.generate("vit-b", B=1, H=2, N=300, M0=12, C=4, P=3, T=64, dtype="f32", seed=17)
    r = oracle.forward(inp)
    Q, K = inp.f64("Q"), inp.f64("K")
    cap = oracle.capture(Q, K, r["pstar"], r["sel"], inp.T, inp.scale, inp.M0)
    # the same fraction from an explicit softmax matrix
    for h in range(inp.H):
        S = inp.scale * Q[0, h] @ K[0, h].T
        A = np.exp(S - S.max(axis=1, keepdims=True))
        A /= A.sum(axis=1, keepdims=True)
        for t in range(inp.ntiles):
            rows = slice(t * inp.T, min(inp.N, (t + 1) * inp.T))
            on = np.isin(r["pstar"][0, h], r["sel"][0, h, t])
            np.testing.assert_allclose(cap[0, h, rows], A[rows][:, on].sum(axis=1), rtol=1e-12, atol=1e-14)
    # every parent selected -> all the weight; none -> nothing
    all_sel = np.broadcast_to(np.arange(inp.M0, dtype=np.int32), (1, 2, inp.ntiles, inp.M0))
    assert np.abs(oracle.capture(Q, K, r["pstar"], all_sel, inp.T, inp.scale, inp.M0) - 1).max() < 1e-12
    none = np.zeros((1, 2, inp.ntiles, 0), dtype=np.int32)
    assert (oracle.capture(Q, K, r["pstar"], none, inp.T, inp.scale, inp.M0) == 0).all()


# ---------------------------------------------------------------- Gilbert order

def _hilbert_d2xy(n, dist):
    """Classical Hilbert curve on an n x n grid (n a power of two), index ->
    (x, y), by the textbook quadrant-rotation recursion written iteratively."""
    x = y = 0
    t = dist
    s = 1
    while s < n:
        rx = 1 & (t // 2)
        ry = 1 & (t ^ rx)
        if ry == 0:
            if rx == 1:
                x, y = s - 1 - x, s - 1 - y
            x, y = y, x
        x += s * rx
        y += s * ry
        t //= 4
        s *= 2
    return x, y


@pytest.mark.parametrize("W,H", [(1, 1), (1, 7), (9, 1), (2, 2), (4, 4), (3, 5), (5, 3), (6, 4), (7, 7),
                                 (10, 3), (28, 28), (30, 30), (64, 64), (13, 40), (256, 256), (33, 18)])
def test_gilbert_order_is_a_path_over_the_grid(W, H):
    o = oracle.gilbert_order(W, H)
    assert sorted(o.tolist()) == list(range(W * H))               # a permutation of the cells
    x, y = o % W, o // W
    step = np.abs(np.diff(x)) + np.abs(np.diff(y))
    cheb = np.maximum(np.abs(np.diff(x)), np.abs(np.diff(y)))
    assert (cheb == 1).all() if W * H > 1 else True               # every step to a touching cell
    assert (step == 2).sum() <= 1                                 # at most one diagonal step
    if W * H > 1:                                                 # corner to corner along the long side
        assert (x[0], y[0]) == (0, 0)
        assert ((x[-1], y[-1]) == (W - 1, 0)) if W >= H else ((x[-1], y[-1]) == (0, H - 1))


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32])
def test_gilbert_on_power_of_two_squares_is_the_hilbert_curve(n):
    o = oracle.gilbert_order(n, n)
    ref = [_hilbert_d2xy(n, i) for i in range(n * n)]
    assert [(int(v % n), int(v // n)) for v in o] == ref


def test_gilbert_tiles_are_compact():
    # 64 x 64 grid in tiles of 128 cells: every tile's bounding box is far
    # smaller than a raster tile's (2 rows x 64 columns)
    o = oracle.gilbert_order(64, 64)
    x, y = o % 64, o // 64
    spans = [(x[t:t + 128].max() - x[t:t + 128].min() + 1) * (y[t:t + 128].max() - y[t:t + 128].min() + 1)
             for t in range(0, 64 * 64, 128)]
    assert max(spans) <= 256
