"""Codebook diagnostics and capture on the GPU against the CPU oracle.

The oracle receives the GPU's own leaf ids and selections, so these tests
check the diagnostics' arithmetic; the leaves and selections themselves are
checked by the parity tests."""

import sys

import numpy as np
import pytest

import oracle
import synth
from _protocol import tensor_to_f64

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


def _dev(arr, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(DEV)


def _run(avq, inp, P=None):
    P = inp.P if P is None else P
    ch = _dev(inp.children, inp.dtype)
    K, V, Q = (_dev(x, inp.dtype) for x in (inp.K, inp.V, inp.Q))
    parents, sq, fr = avq.build_tree(ch)
    vsum, count, leaf = avq.assign_aggregate(K, V, parents, ch, sq, fr, want_leaf=True)
    Y, sel, _ = avq.attention_fwd(Q, parents, ch, vsum, count, P, inp.T, inp.scale, want_sel=True)
    return dict(ch=ch, K=K, Q=Q, parents=parents, count=count, leaf=leaf, sel=sel)


CASES = [("vit-b", dict(B=1, H=2, N=3000)), ("seg-zipf", dict(B=2, H=2, N=2500)),
         ("wide-d128", dict(B=1, H=2, N=1500)), ("tiny-f32", dict()), ("flat-64k", dict(B=1, H=2, N=2000)),
         ("long-64k", dict())]


@pytest.mark.parametrize("name,over", CASES)
def test_commitment_and_active_ratio(avq, name, over):
    inp = synth.generate(name, **over)
    _say(f"codebook diagnostics {name} B={inp.B} H={inp.H} N={inp.N} M0={inp.M0} C={inp.C}")
    r = _run(avq, inp)
    cm, ac = avq.codebook_diagnostics(r["K"], r["parents"], r["ch"], r["leaf"], r["count"])
    cm2, ac2 = avq.codebook_diagnostics(r["K"], r["parents"], r["ch"], r["leaf"], r["count"])
    torch.cuda.synchronize()
    assert torch.equal(cm, cm2) and torch.equal(ac, ac2)          # fixed summation order
    leaf = r["leaf"].cpu().numpy()
    par64 = tensor_to_f64(r["parents"], inp.dtype)
    ref = oracle.commitment(inp.f64("K"), par64, inp.f64("children"), leaf)
    # fp32 sums of exact fp32 squared differences over N keys: relative 1e-5
    np.testing.assert_allclose(cm.cpu().numpy(), ref, rtol=1e-5)
    act = oracle.active_ratio(r["count"].cpu().numpy(), inp.N)
    np.testing.assert_array_equal(ac.cpu().numpy(), act.astype(np.float32))
    _say(f"  commitment {ref.mean():.4f} active ratio {act.mean():.4f}")


@pytest.mark.parametrize("name,over,P", [("vit-b", dict(B=1, H=2, N=1500), 8), ("vit-b", dict(B=1, H=1, N=700, T=32), 3),
                                         ("wide-d128", dict(B=1, H=2, N=900), 32),
                                         ("tiny-f32", dict(N=800), 4), ("vit-b", dict(B=1, H=1, N=500), 0),
                                         ("vit-b", dict(B=1, H=1, N=600, M0=16), 16)])
def test_capture(avq, name, over, P):
    inp = synth.generate(name, **over)
    _say(f"capture {name} N={inp.N} M0={inp.M0} P={P} T={inp.T}")
    r = _run(avq, inp, P)
    cap = avq.capture(r["Q"], r["K"], r["ch"], r["leaf"], r["sel"], inp.T, inp.scale)
    torch.cuda.synchronize()
    leaf = r["leaf"].cpu().numpy()
    pst = np.where(leaf < inp.M0, leaf, (leaf - inp.M0) // max(inp.C, 1))
    ref = oracle.capture(inp.f64("Q"), inp.f64("K"), pst, r["sel"].cpu().numpy(), inp.T, inp.scale, inp.M0)
    err = np.abs(cap.cpu().numpy() - ref).max()
    _say(f"  mean capture {ref.mean():.4f} max|d| {err:.2e}")
    assert err <= 1e-4
    if P == inp.M0:
        assert np.abs(cap.cpu().numpy() - 1).max() <= 1e-5
    if P == 0:
        assert (cap.cpu().numpy() == 0).all()
