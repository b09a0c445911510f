"""Token reordering along the Gilbert curve on the GPU: the gather/scatter
kernel against numpy indexing (bit-exact), and an AVQ forward run on tokens
in curve order, moved back afterwards, against the oracle."""

import sys

import numpy as np
import pytest

import oracle
import synth
from _protocol import Y_TOL, tensor_to_f64

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


@pytest.mark.parametrize("dtype,d,W,H,cls", [(torch.bfloat16, 64, 28, 28, True), (torch.float32, 128, 30, 17, False),
                                             (torch.bfloat16, 128, 64, 64, False), (torch.float32, 64, 1, 5, True)])
def test_permute_tokens_gather_and_scatter(avq, dtype, d, W, H, cls):
    _say(f"permute dtype={dtype} d={d} grid={W}x{H} class_token={cls}")
    g = avq.gilbert_order(W, H).numpy().astype(np.int64)
    order = np.concatenate([[0], 1 + g]) if cls else g          # the class token stays first
    N = order.size
    x = torch.randn((2, 3, N, d), generator=torch.Generator().manual_seed(N)).to(dtype).to(DEV)
    o = torch.from_numpy(order.astype(np.int32)).to(DEV)
    y = avq.permute_tokens(x, o)
    z = avq.permute_tokens(y, o, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), x.cpu()[:, :, order])
    assert torch.equal(z, x)


def test_forward_in_gilbert_order(avq):
    # vit-b's 64 x 64 patch grid: Q, K, V moved into curve order, the forward
    # run there, Y moved back; against the oracle on the reordered tokens
    inp = synth.generate("vit-b", B=1, H=2)
    _say(f"forward in Gilbert order: {inp.name} N={inp.N}")
    order = avq.gilbert_order(64, 64).numpy().astype(np.int64)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    Q, K, V = (to(x) for x in (inp.Q, inp.K, inp.V))
    o = torch.from_numpy(order.astype(np.int32)).to(DEV)
    Qg, Kg, Vg = (avq.permute_tokens(x, o) for x in (Q, K, V))
    ch = to(inp.children)
    Yg = avq.forward(Qg, Kg, Vg, ch, inp.P, inp.T, inp.scale)
    Y = avq.permute_tokens(Yg, o, inverse=True)
    torch.cuda.synchronize()
    ro = synth.Inputs(**{**inp.__dict__})
    ro.Q, ro.K, ro.V = (x[:, :, order] for x in (inp.Q, inp.K, inp.V))
    ref = oracle.forward(ro)["Y"]
    back = np.empty_like(ref)
    back[:, :, order] = ref
    err = np.abs(tensor_to_f64(Y, "bf16") - back).max()
    _say(f"  max|dY| = {err:.3e}")
    assert err <= Y_TOL["bf16"]
