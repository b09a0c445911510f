"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Every case prints what it runs before touching the GPU."""

import sys

import numpy as np
import pytest

import oracle
import synth
from _protocol import Y_TOL, check_selection, check_stage1, tensor_to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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


DEV = "cuda:0"


def to_dev(arr, dtype):
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(DEV)


def run_gpu(avq, inp, P, T, force_child=False):
    ch = to_dev(inp.children, inp.dtype)
    K, V, Q = (to_dev(x, inp.dtype) for x in (inp.K, inp.V, inp.Q))
    parents, sq = avq.build_tree(ch)
    vsum, count, leaf, pack = avq.assign_aggregate(K, V, parents, ch, sq, force_child=force_child,
                                                   want_leaf=True)
    Y, sel, imp = avq.attention_fwd(Q, parents, ch, pack, P, T, inp.scale,
                                    want_sel=True, want_importance=True)
    torch.cuda.synchronize()
    return dict(parents=tensor_to_f64(parents, inp.dtype), sqnorm=sq.cpu().numpy(),
                vsum=vsum.cpu().numpy().astype(np.float64), count=count.cpu().numpy(),
                leaf=leaf.cpu().numpy(), Y=tensor_to_f64(Y, inp.dtype),
                sel=sel.cpu().numpy(), imp=imp.cpu().numpy().astype(np.float64))


def check_all(avq, inp, P=None, T=None, force_child=False, tile_ranges=None):
    """Run the whole forward on the GPU once, check stage 1 on every key and
    stage 2 on the given query-tile ranges (default: every tile)."""
    P = inp.P if P is None else P
    T = inp.T if T is None else T
    _say(f"{inp.name} dtype={inp.dtype} B={inp.B} H={inp.H} N={inp.N} d={inp.d} M0={inp.M0} "
         f"C={inp.C} P={P} T={T} force_child={force_child} seed={inp.seed}")
    g = run_gpu(avq, inp, P, T, force_child)
    ch64 = inp.f64("children")
    par64, sq64 = oracle.build_tree(ch64, inp.dtype)
    np.testing.assert_array_equal(g["parents"], par64)
    np.testing.assert_array_equal(g["sqnorm"], sq64.astype(np.float32))
    a, vsum, count = check_stage1(inp, par64, g["leaf"], g["vsum"], g["count"], force_child)
    Q64 = inp.f64("Q")
    nt = -(-inp.N // T)
    errs, namb = [], 0
    for (t0, t1) in (tile_ranges or [(0, nt)]):
        _, w, sel = oracle.attention(Q64, par64, ch64, vsum, count, P, T, inp.scale, tiles=(t0, t1))
        namb += check_selection(w[:, :, t0:t1], sel[:, :, t0:t1], g["sel"][:, :, t0:t1], P)
        np.testing.assert_allclose(g["imp"][:, :, t0:t1], w[:, :, t0:t1], rtol=2e-4, atol=1e-7 * T)
        Yf, _, _ = oracle.attention(Q64, par64, ch64, vsum, count, P, T, inp.scale,
                                    forced_sel=g["sel"], tiles=(t0, t1))
        rows = slice(t0 * T, min(inp.N, t1 * T))
        errs.append(float(np.abs(g["Y"][:, :, rows] - Yf[:, :, rows]).max()))
    err = max(errs)
    _say(f"  max|dY|={err:.3e} ambiguous keys={a['n_ambiguous']} tiles={namb} "
         f"residual keys={int(count[..., :inp.M0].sum() - count[..., inp.M0:].sum())}")
    assert err <= Y_TOL[inp.dtype], err
    return dict(err=err, g=g, vsum=vsum, count=count)


# ------------------------------------------------------------------ workloads


@pytest.mark.parametrize("name,N", [("tiny-f32", 1024), ("vit-b", 3000), ("seg-zipf", 5000),
                                    ("long-64k", 9000), ("wide-d128", 3000)])
def test_workload_reduced(avq, name, N):
    inp = synth.generate(name, B=1, H=2, N=N)
    check_all(avq, inp)


@pytest.mark.parametrize("P", [0, 4, 16, 128])
def test_seg_zipf_P_sweep(avq, P):
    inp = synth.generate("seg-zipf", B=2, H=2, N=4100)
    check_all(avq, inp, P=P)


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_workload_full_size_sampled_tiles(avq, name):
    """Full size of every workload; stage 1 checked on every key, stage 2
    on the first, a middle and the last query tile of every (b, h)."""
    inp = synth.generate(name)
    nt = inp.ntiles
    check_all(avq, inp, tile_ranges=[(0, 1), (nt // 2, nt // 2 + 1), (nt - 1, nt)])


def test_maximum_sequence_length(avq):
    """N = 2^20, the largest supported: 1024 assignment chunks per head (the
    refinement kernel's chunk table at its largest).  Stage 1 on every key,
    stage 2 on three tiles."""
    inp = synth.generate("long-64k", H=1, N=1 << 20)
    nt = inp.ntiles
    check_all(avq, inp, tile_ranges=[(0, 1), (nt // 2, nt // 2 + 1), (nt - 1, nt)])


# ------------------------------------------------------------------ edge shapes

EDGE = [
    # dtype, d, M0, C, P, T, N, force_child
    ("bf16", 64, 1, 4, 1, 64, 1, False),
    ("bf16", 64, 1, 4, 0, 32, 37, False),
    ("f32", 64, 5, 2, 3, 32, 300, False),
    ("bf16", 64, 100, 4, 9, 256, 1300, False),
    ("bf16", 128, 256, 8, 40, 32, 700, False),
    ("bf16", 64, 17, 8, 17, 32, 777, False),
    ("bf16", 64, 33, 16, 5, 128, 2049, False),
    ("f32", 128, 24, 4, 7, 64, 1500, False),
    ("bf16", 128, 64, 16, 64, 128, 1025, False),
    ("bf16", 64, 256, 8, 256, 128, 2100, False),
    ("bf16", 64, 40, 8, 6, 64, 3000, True),
    ("f32", 64, 16, 4, 4, 64, 1024, True),
    # d = 128: 256-query tiles over 8-wave work-groups, C = 2, 30 parents
    ("bf16", 128, 30, 2, 5, 256, 1500, False),
    # d = 128 with C = 16 (refinement groups of two parents), fp32, and a
    # ragged last group (129 parents)
    ("f32", 128, 48, 16, 3, 32, 900, False),
    ("bf16", 128, 129, 16, 20, 64, 777, True),
    # fp32 at d = 128 with 256-query tiles (8 waves, value sums from L2)
    ("f32", 128, 200, 4, 8, 256, 1100, False),
    # fewer non-empty parents than P (5 keys, 40 parents, P = 12): the top-P
    # threshold is 0 and the empty parents tie there, lowest indices first
    ("bf16", 64, 40, 4, 12, 64, 5, False),
    ("f32", 64, 40, 8, 12, 32, 3, False),
]


@pytest.mark.parametrize("dtype,d,M0,C,P,T,N,force", EDGE)
def test_edge_shapes(avq, dtype, d, M0, C, P, T, N, force):
    inp = synth.generate("vit-b", B=1, H=2, N=N, d=d, M0=M0, C=C, P=P, T=T, dtype=dtype,
                         seed=77 + M0 + N)
    check_all(avq, inp, force_child=force)


def _random_shapes(n, seed=2024):
    """n shapes drawn from the supported space (fp32 at d = 128 keeps M0 <=
    128 so that its parents fit in LDS for every tile)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dtype = str(rng.choice(["bf16", "f32"]))
        d = int(rng.choice([64, 128]))
        M0 = int(rng.integers(1, 129 if (dtype == "f32" and d == 128) else 257))
        C = int(rng.choice([2, 4, 8, 16]))
        P = int(rng.integers(0, M0 + 1))
        T = int(rng.choice([32, 64, 128, 256]))
        if dtype == "f32" and T == 256 and M0 > 128:
            P = min(P, 150)   # past that, the shape does not fit in LDS
        N = int(rng.integers(1, 2500))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        out.append((dtype, d, M0, C, P, T, N, B, H, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("dtype,d,M0,C,P,T,N,B,H,force", _random_shapes(40))
def test_random_shapes(avq, dtype, d, M0, C, P, T, N, B, H, force):
    inp = synth.generate("vit-b", B=B, H=H, N=N, d=d, M0=M0, C=C, P=P, T=T, dtype=dtype,
                         seed=500 + N + M0)
    check_all(avq, inp, force_child=force)


def test_scale_one_and_dyadic_tree(avq):
    inp = synth.generate_dyadic(5, B=2, H=2, N=700, d=64, M0=8, C=4, P=3, T=32)
    inp.scale = 1.0 / 64.0
    check_all(avq, inp)


@pytest.mark.parametrize("scale", [-0.125, 1.0])
def test_negative_and_unit_scale(avq, scale):
    inp = synth.generate("vit-b", B=1, H=2, N=1500, M0=40, C=8, P=6, T=64, seed=31)
    inp.scale = scale
    check_all(avq, inp)


def test_child_logits_far_above_the_shift(avq):
    # children spread six times wider around their parents than the workload
    # generator makes them: child logits of selected parents exceed the
    # parents' maximum logit by more than 32 (log2 units), past which the
    # kernel raises its softmax shift and rescales X and Z; the importance
    # values stay well inside fp32's range
    inp = synth.generate("vit-b", B=1, H=2, N=1500, M0=40, C=8, P=6, T=64, seed=31)
    ch = inp.f64("children")
    par = ch.mean(axis=2, keepdims=True)
    inp.children = synth.to_storage(par + 6.0 * (ch - par), inp.dtype)
    inp.scale = 0.5
    Q64, ch64 = inp.f64("Q"), inp.f64("children")
    par64, _ = oracle.build_tree(ch64, inp.dtype)
    l2e = inp.scale / np.log(2.0)
    sp = np.einsum("bhnd,hmd->bhnm", Q64, par64) * l2e
    sc = np.einsum("bhnd,hmcd->bhnmc", Q64, ch64) * l2e
    assert (sc.max(axis=(3, 4)) - sp.max(axis=3)).max() > 40.0   # the branch is taken
    check_all(avq, inp)


@pytest.mark.parametrize("dtype,d,M0,C,N", [("bf16", 64, 256, 8, 6000), ("bf16", 128, 64, 16, 3000),
                                            ("f32", 64, 40, 4, 2600)])
def test_skewed_keys_split_groups(avq, dtype, d, M0, C, N):
    # 70 % of the keys sit next to one child of parent 0, so one refinement
    # group (one work-group of the refinement kernel) holds most of the list
    inp = synth.generate("vit-b", B=1, H=2, N=N, d=d, M0=M0, C=C, P=5, T=64, dtype=dtype, seed=93 + N)
    rng = np.random.default_rng(N)
    K64, ch64 = inp.f64("K"), inp.f64("children")
    hot = rng.random((1, inp.H, N)) < 0.7
    near = ch64[:, 0, C // 2][None, :, None, :] + 0.01 * rng.standard_normal(K64.shape)
    inp.K = synth.to_storage(np.where(hot[..., None], near, K64), dtype)
    r = check_all(avq, inp)
    group = 2 if (C == 16 and d == 128) else 4
    heavy = r["count"][..., :group].sum(axis=-1)            # keys of the first group
    assert heavy.min() > 0.6 * N


# ------------------------------------------------------------------ invariants


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_key_per_leaf_equals_exact_attention(avq, dtype):
    inp = synth.generate_one_key_per_leaf(21, B=1, H=2, d=64, M0=16, C=8, T=32, dtype=dtype)
    _say(f"one key per leaf dtype={dtype} N={inp.N}")
    r = check_all(avq, inp, P=16, T=32)
    Q, K, V = (to_dev(x, dtype) for x in (inp.Q, inp.K, inp.V))
    Ye = tensor_to_f64(avq.exact_attention_fwd(Q, K, V, inp.scale), dtype)
    from _refs import softmax_attention
    ref = np.stack([softmax_attention(inp.f64("Q")[0, h], inp.f64("K")[0, h], inp.f64("V")[0, h],
                                      inp.scale) for h in range(2)])[None]
    assert np.abs(Ye - ref).max() <= Y_TOL[dtype]
    assert np.abs(r["g"]["Y"] - ref).max() <= Y_TOL[dtype]


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_exact_attention_kernel(avq, dtype, d):
    _say(f"exact attention dtype={dtype} d={d}")
    rng = np.random.default_rng(3)
    B, H, N = 1, 2, 333
    x = rng.standard_normal((3, B, H, N, d))
    st = [synth.to_storage(x[i], dtype) for i in range(3)]
    Q, K, V = (to_dev(s, dtype) for s in st)
    Y = tensor_to_f64(avq.exact_attention_fwd(Q, K, V, 0.125), dtype)
    f = [synth.storage_to_f64(s, dtype) for s in st]
    from _refs import softmax_attention
    ref = np.stack([softmax_attention(f[0][0, h], f[1][0, h], f[2][0, h], 0.125) for h in range(H)])[None]
    assert np.abs(Y - ref).max() <= Y_TOL[dtype] / 4


def test_constant_values_give_constant_output(avq):
    inp = synth.generate("long-64k", B=1, H=2, N=4096)
    inp.V[:] = synth.f64_to_bf16_bits(np.full(1, 0.75))[0]
    _say("constant values")
    for P in (0, 16, 256):
        ch = to_dev(inp.children, "bf16")
        K, V, Q = (to_dev(x, "bf16") for x in (inp.K, inp.V, inp.Q))
        parents, sq = avq.build_tree(ch)
        _, _, _, pack = avq.assign_aggregate(K, V, parents, ch, sq)
        Y, _, _ = avq.attention_fwd(Q, parents, ch, pack, P, 128, inp.scale)
        torch.cuda.synchronize()
        assert np.abs(tensor_to_f64(Y, "bf16") - 0.75).max() <= 4e-3


def test_forward_equals_the_stages(avq):
    # the one-call helper runs the same three entry points: identical bits
    inp = synth.generate("vit-b", B=1, H=2, N=900, M0=24, C=8, P=3, T=64, seed=12)
    _say(f"forward() vs stages: {inp.name} N={inp.N} M0={inp.M0}")
    ch = to_dev(inp.children, inp.dtype)
    K, V, Q = (to_dev(x, inp.dtype) for x in (inp.K, inp.V, inp.Q))
    Y1 = avq.forward(Q, K, V, ch, inp.P, inp.T, inp.scale)
    parents, sq = avq.build_tree(ch)
    _, _, _, pack = avq.assign_aggregate(K, V, parents, ch, sq)
    Y2, _, _ = avq.attention_fwd(Q, parents, ch, pack, inp.P, inp.T, inp.scale)
    Y3 = avq.forward(Q, K, V, ch, inp.P, inp.T, inp.scale, tree=(parents, sq))
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(Y1, Y3)


def test_repeated_runs_are_bitwise_identical(avq):
    # no kernel accumulates through atomics or in a scheduling-dependent
    # order, so every run gives the same bits (different input sets
    # interleaved, so nothing is served from a previous run's outputs)
    inp = synth.generate("vit-b", B=1, H=4, N=3000, M0=64, C=8, P=8, T=128, seed=44)
    _say(f"repeated runs: {inp.name} H={inp.H} N={inp.N} M0={inp.M0}")
    ch = to_dev(inp.children, inp.dtype)
    K, V, Q = (to_dev(x, inp.dtype) for x in (inp.K, inp.V, inp.Q))
    Kb, Vb, Qb = (torch.flip(x, dims=[2]).contiguous() for x in (K, V, Q))
    parents, sq = avq.build_tree(ch)
    ref = None
    for it in range(12):
        vsum, count, leaf, pack = avq.assign_aggregate(K, V, parents, ch, sq, want_leaf=True)
        Y, sel, imp = avq.attention_fwd(Q, parents, ch, pack, inp.P, inp.T, inp.scale,
                                        want_sel=True, want_importance=True)
        # (the operand pack's alignment gaps are never written, so it is
        # compared through Y, which reads every byte it needs)
        got = dict(vsum=vsum, count=count, leaf=leaf, Y=Y, sel=sel, imp=imp)
        got = {k: t.clone() for k, t in got.items()}
        if ref is None:
            ref = got
        else:
            for k in ref:
                assert torch.equal(ref[k], got[k]), (it, k)
        avq.forward(Qb, Kb, Vb, ch, inp.P, inp.T, inp.scale, tree=(parents, sq))
    torch.cuda.synchronize()


def test_invalid_arguments_raise(avq):
    _say("invalid arguments")
    inp = synth.generate("vit-b", B=1, H=1, N=256, M0=8)
    ch = to_dev(inp.children, "bf16")
    K, V, Q = (to_dev(x, "bf16") for x in (inp.K, inp.V, inp.Q))
    parents, sq = avq.build_tree(ch)
    _, _, _, pack = avq.assign_aggregate(K, V, parents, ch, sq)
    with pytest.raises(avq.AvqError, match="INVALID_ARG"):
        avq.attention_fwd(Q, parents, ch, pack, 9, 128, inp.scale)   # P > M0
    with pytest.raises(avq.AvqError, match="UNSUPPORTED"):
        avq.attention_fwd(Q, parents, ch, pack, 2, 48, inp.scale)   # tile 48
    with pytest.raises(avq.AvqError, match="UNSUPPORTED"):
        avq.attention_fwd(Q, parents, ch, pack, 2, 16, inp.scale)   # tile 16
    with pytest.raises(avq.AvqError, match="INVALID_ARG"):
        avq.attention_fwd(Q, parents, ch, pack, 2, 128, float("nan"))
    with pytest.raises(avq.AvqError, match="UNSUPPORTED"):
        bad = torch.zeros((1, 8, 4, 96), dtype=torch.bfloat16, device=DEV)
        avq.build_tree(bad)   # d = 96
    # output buffers of the wrong shape or type are refused before any launch
    with pytest.raises(avq.AvqError, match="Q's shape"):
        avq.attention_fwd(Q, parents, ch, pack, 2, 128, inp.scale, out=Q[:, :, :128].contiguous())
    with pytest.raises(avq.AvqError, match="dtype"):
        avq.attention_fwd(Q, parents, ch, pack, 2, 128, inp.scale, out=Q.float())
    vsum, count, _, pk = avq.assign_aggregate(K, V, parents, ch, sq)
    with pytest.raises(avq.AvqError, match="do not match"):
        avq.assign_aggregate(K, V, parents, ch, sq, out=(vsum[:, :, :-1].contiguous(), count, pk))
    with pytest.raises(avq.AvqError, match="do not match"):
        avq.assign_aggregate(K, V, parents, ch, sq, out=(vsum, count, pk[:-1]))
    torch.cuda.synchronize()
