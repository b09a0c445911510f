"""The allocation-free stage-1 entry point (avq_assign_aggregate_noalloc,
scratch in a static device array) against avq_assign_aggregate with a
caller workspace: identical bits, on two calls in a row, the second with a
smaller input (so stale scratch contents from the first call are present),
and a shape past the scratch limit is refused before any launch."""

import sys

import numpy as np
import pytest

import synth

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


def _compare(avq, inp, force):
    _say(f"noalloc vs workspace: {inp.name} dtype={inp.dtype} B={inp.B} H={inp.H} N={inp.N} "
         f"d={inp.d} M0={inp.M0} C={inp.C} force_child={force}")
    ch = _dev(inp.children, inp.dtype)
    K, V = _dev(inp.K, inp.dtype), _dev(inp.V, inp.dtype)
    parents, sq, fr = avq.build_tree(ch)
    ref_v, ref_c, ref_l = avq.assign_aggregate(K, V, parents, ch, sq, fr, force_child=force, want_leaf=True)
    S = inp.M0 * (1 + inp.C)
    vsum = torch.full((inp.B, inp.H, S, inp.d), float("nan"), dtype=torch.float32, device=DEV)
    count = torch.full((inp.B, inp.H, S), -7, dtype=torch.int32, device=DEV)
    leaf = torch.full((inp.B, inp.H, inp.N), -7, dtype=torch.int32, device=DEV)
    avq.assign_aggregate_noalloc(K, V, parents, ch, sq, fr, (vsum, count), force_child=force, leaf=leaf)
    torch.cuda.synchronize()
    assert torch.equal(vsum, ref_v)
    assert torch.equal(count, ref_c)
    assert torch.equal(leaf, ref_l)


def test_noalloc_matches_workspace_entry_point_twice(avq):
    # first call large (N = 65536 over 8 heads: 2.3 MB of scratch), second
    # smaller and of another shape, reading scratch the first call left
    _compare(avq, synth.generate("long-64k"), False)
    _compare(avq, synth.generate("wide-d128", B=1, H=3, N=5000, M0=100), True)


def test_noalloc_skewed_keys_split_groups(avq):
    """Zipf-skewed keys (seg-zipf's generator, 8192 keys per head): a group
    holds more keys than the refinement's split target, so its slices store
    partial sums in the scratch and the last one adds them."""
    _compare(avq, synth.generate("seg-zipf", B=1, H=4, N=8192), False)


def test_noalloc_refuses_shapes_past_the_scratch(avq):
    _say("noalloc scratch limit")
    B, H, N, d, M0, C = 1, 64, 65536, 64, 16, 4   # 16 MiB of keys + segments > 16 MiB
    assert avq.assign_aggregate_workspace_size(B, H, N, M0, C, d) > avq.NOALLOC_SCRATCH_BYTES
    K = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device=DEV)
    ch = torch.zeros((H, M0, C, d), dtype=torch.bfloat16, device=DEV)
    parents, sq, fr = avq.build_tree(ch)
    S = M0 * (1 + C)
    out = (torch.empty((B, H, S, d), dtype=torch.float32, device=DEV),
           torch.empty((B, H, S), dtype=torch.int32, device=DEV))
    with pytest.raises(avq.AvqError, match="UNSUPPORTED"):
        avq.assign_aggregate_noalloc(K, K, parents, ch, sq, fr, out)
    torch.cuda.synchronize()
