"""Parity of the three-level tree (roots -> children -> leaves, the deeper
hierarchy the AVQ-Attention pages propose in Sec. 6) on the GPU, through the
C ABI, against the oracle's three-level functions.  The bars are those of
the two-level path (tests/_protocol.py), applied at every level: leaves
bit-exact outside the near-tie band at any of the three descents, counts
exact, value sums inside the fp32 summation bound, selections equal on
every tile (and every level) whose importance gap is at least 1e-4, Y
within 2e-2 (bf16) / 1e-4 (fp32)."""

import sys

import numpy as np
import pytest

import oracle
import synth
from _protocol import AMBIG, Y_TOL, check_selection, tensor_to_f64, tile_ambiguity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"


def _say(msg):
    sys.stdout.write(f"\n[case] {msg}\n")
    sys.stdout.flush()


@pytest.fixture(scope="module")
def avq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import adaptive_vector_quantized_avq_amd as m
    m.load_library()
    return m


def to_dev(arr, dtype):
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(DEV)


def run_gpu3(avq, inp, P, T, force_child=False):
    lv = to_dev(inp.children, inp.dtype)
    K, V, Q = (to_dev(x, inp.dtype) for x in (inp.K, inp.V, inp.Q))
    l0, l1, sq, fr = avq.build_tree3(lv)
    vsum, count, leaf = avq.assign_aggregate3(K, V, l0, l1, lv, sq, fr, force_child=force_child, want_leaf=True)
    Y, s0, s1 = avq.attention3_fwd(Q, l0, l1, lv, vsum, count, P, T, inp.scale, want_sel=True)
    torch.cuda.synchronize()
    return dict(l0=tensor_to_f64(l0, inp.dtype), l1=tensor_to_f64(l1, inp.dtype), sqnorm=sq.cpu().numpy(),
                frame=fr.cpu().numpy().astype(np.float64), vsum=vsum.cpu().numpy().astype(np.float64),
                count=count.cpu().numpy(), leaf=leaf.cpu().numpy(), Y=tensor_to_f64(Y, inp.dtype),
                sel0=s0.cpu().numpy(), sel1=s1.cpu().numpy())


def check_tree3(inp, g, l0, l1):
    np.testing.assert_array_equal(g["l0"], l0)
    np.testing.assert_array_equal(g["l1"], l1)
    H, M0, C, d = inp.H, inp.M0, inp.C, inp.d
    rows = np.concatenate([l0, l1.reshape(H, M0 * C, d), inp.f64("children").reshape(H, M0 * C * C, d)], axis=1)
    diff = rows - g["frame"][:, None, :]
    exact = oracle.round_to(diff, inp.dtype) == diff
    assert (exact | (g["frame"] == 0.0)[:, None, :]).all()
    ref = np.sum(diff * diff, axis=-1)
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert (np.abs(g["sqnorm"].astype(np.float64) - ref) <= ulp).all()


def check_stage1_3(inp, g, l0, l1, force_child):
    lv = inp.f64("children")
    a = oracle.assign3(inp.f64("K"), l0, l1, lv, force_child=force_child)
    amb = (a["gap0"] < AMBIG) | (a["gap1"] < AMBIG) | (a["gap2"] < AMBIG)
    bad = (g["leaf"] != a["leaf"]) & ~amb
    assert not bad.any(), f"{bad.sum()} non-ambiguous keys assigned differently, first at {np.argwhere(bad)[:5]}"
    M0, C = inp.M0, inp.C
    S3 = M0 * (1 + C + C * C)
    assert ((g["leaf"] >= 0) & (g["leaf"] < S3)).all()
    leaf = np.where(amb, g["leaf"], a["leaf"])
    V = inp.f64("V")
    vsum, count = oracle.aggregate3(V, leaf, M0, C)
    np.testing.assert_array_equal(g["count"], count)
    absum, _ = oracle.aggregate3(np.abs(V), leaf, M0, C)
    bound = np.maximum(count - 1, 0)[..., None] * 2.0 ** -24 * absum + 2.0 ** -23 * np.abs(vsum) + 1e-30
    err = np.abs(g["vsum"] - vsum)
    assert (err <= bound).all(), f"vsum outside the fp32 bound: max excess {(err - bound).max()}"
    return int(amb.sum()), vsum, count


def check_level1_selection(imp1, sel0_sorted, sel1_orc, sel1_gpu, C, P):
    """Level-1 selections: candidates are the children of the tile's roots
    (ascending), imp1 their importance in that order."""
    amb = tile_ambiguity(imp1, P)
    B, H, nt = imp1.shape[:3]
    for b in range(B):
        for h in range(H):
            for t in range(nt):
                g = set(sel1_gpu[b, h, t].tolist())
                o = set(sel1_orc[b, h, t].tolist())
                assert len(g) == P, f"tile {(b, h, t)}: duplicate level-1 selections {sorted(g)}"
                roots = sel0_sorted[b, h, t]
                cands = (roots[:, None] * C + np.arange(C)[None, :]).ravel()
                assert g <= set(cands.tolist()), f"tile {(b, h, t)}: level-1 pick outside the candidates"
                if not amb[b, h, t]:
                    assert g == o, f"tile {(b, h, t)}: level 1 gpu {sorted(g)} oracle {sorted(o)}"
                else:
                    w = imp1[b, h, t]
                    inside = np.isin(cands, sorted(g))
                    wp = -np.sort(-w)[P - 1]
                    if (~inside).any():
                        assert w[inside].min() >= w[~inside].max() - AMBIG * wp - 1e-30
    return int(amb.sum())


def check_all3(avq, inp, P=None, T=None, force_child=False):
    P = inp.P if P is None else P
    T = inp.T if T is None else T
    _say(f"three-level {inp.name} dtype={inp.dtype} B={inp.B} H={inp.H} N={inp.N} d={inp.d} M0={inp.M0} "
         f"C={inp.C} P={P} T={T} force_child={force_child} seed={inp.seed}")
    g = run_gpu3(avq, inp, P, T, force_child)
    lv = inp.f64("children")
    l0, l1, _ = oracle.build_tree3(lv, inp.dtype)
    check_tree3(inp, g, l0, l1)
    nkeys, vsum, count = check_stage1_3(inp, g, l0, l1, force_child)
    Q = inp.f64("Q")
    r = oracle.attention3(Q, l0, l1, lv, vsum, count, P, T, inp.scale)
    namb0 = check_selection(r["imp0"], r["sel0"], g["sel0"], P)
    same0 = (np.sort(g["sel0"], -1) == np.sort(r["sel0"], -1)).all()
    if not same0:   # level 1 is judged on the GPU's roots
        r = oracle.attention3(Q, l0, l1, lv, vsum, count, P, T, inp.scale, forced_sel0=g["sel0"])
    namb1 = check_level1_selection(r["imp1"], np.sort(g["sel0"], -1), r["sel1"], g["sel1"], inp.C, P)
    same1 = (g["sel1"] == r["sel1"]).all()
    if not (same0 and same1):
        r = oracle.attention3(Q, l0, l1, lv, vsum, count, P, T, inp.scale, forced_sel0=g["sel0"],
                              forced_sel1=g["sel1"])
    err = float(np.abs(g["Y"] - r["Y"]).max())
    _say(f"  max|dY|={err:.3e} ambiguous keys={nkeys} tiles={namb0}+{namb1} "
         f"keys at roots={int((g['leaf'] < inp.M0).sum())} "
         f"at children={int(((g['leaf'] >= inp.M0) & (g['leaf'] < inp.M0 * (1 + inp.C))).sum())}")
    assert err <= Y_TOL[inp.dtype], err
    return err


def test_deep_workload_reduced(avq):
    check_all3(avq, synth.generate("deep-64k", H=2, N=9000))


def test_deep_workload_full_size(avq):
    """deep-64k at its own shape (B=1, H=8, N=65536, M0=64, C=8, P=16):
    stage 1 on every key, stage 2 on every query tile."""
    check_all3(avq, synth.generate("deep-64k"))


def test_step_ranges_across_heads(avq):
    """bf16 at d = 128 runs one 8-wave work-group per CU; 20 heads of 25
    256-query steps do not divide the CUs, so each work-group takes a
    contiguous range of the (head, step) list and stages the next head's
    codebook where its range crosses into it.  Every key and every tile."""
    check_all3(avq, synth.generate("deep-64k", B=2, H=10, N=6400, d=128))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M0,C,P,T,d", [(6, 4, 2, 64, 64), (32, 8, 8, 128, 64), (100, 2, 40, 32, 64),
                                        (16, 16, 16, 256, 64), (24, 8, 5, 128, 128), (64, 4, 64, 64, 128)])
def test_dyadic_shapes(avq, dtype, M0, C, P, T, d):
    """Exact-mean trees across shapes: padded root counts, every C, tile
    sizes, d = 128, ragged last tiles, keys at all three levels."""
    inp = synth.generate_dyadic3(21 + M0 + C, H=2, N=1000 + 7 * M0, d=d, M0=M0, C=C, T=T, dtype=dtype)
    check_all3(avq, inp, P=P, T=T)


@pytest.mark.parametrize("P", [0, 1, 32])
def test_P_edges(avq, P):
    """P = 0 (root-level VQ-attention only), P = 1, and P*C = 256
    level-1 candidates (the largest a tile takes)."""
    check_all3(avq, synth.generate("deep-64k", H=1, N=3000), P=P)


def test_force_child(avq):
    check_all3(avq, synth.generate("deep-64k", H=1, N=5000), force_child=True)


def test_one_key_per_leaf_and_tiny_N(avq):
    check_all3(avq, synth.generate_dyadic3(31, H=1, M0=8, C=4, T=32, dtype="f32", one_key_per_leaf=True), P=8)
    check_all3(avq, synth.generate_dyadic3(32, H=1, N=5, M0=4, C=2, T=32, dtype="bf16"), P=2)


def test_repeatable_bits(avq):
    inp = synth.generate("deep-64k", H=1, N=4000)
    a = run_gpu3(avq, inp, 16, 128)
    b = run_gpu3(avq, inp, 16, 128)
    for k in ("vsum", "count", "leaf", "Y", "sel0", "sel1"):
        np.testing.assert_array_equal(a[k], b[k])


def test_argument_errors(avq):
    inp = synth.generate("deep-64k", H=1, N=256)
    lv = to_dev(inp.children, inp.dtype)
    l0, l1, sq, fr = avq.build_tree3(lv)
    K, V, Q = (to_dev(x, inp.dtype) for x in (inp.K, inp.V, inp.Q))
    vsum, count, _ = avq.assign_aggregate3(K, V, l0, l1, lv, sq, fr)
    with pytest.raises(avq.AvqError):   # P*C = 264 level-1 candidates
        avq.attention3_fwd(Q, l0, l1, lv, vsum, count, 33, 128, inp.scale)
    with pytest.raises(avq.AvqError):
        avq.attention3_fwd(Q, l0, l1, lv, vsum, count, 65, 128, inp.scale)
    with pytest.raises(avq.AvqError):
        avq.attention3_fwd(Q, l0, l1, lv, vsum, count, 4, 100, inp.scale)
