"""Host-side checks of the C-ABI library that need no GPU: it loads, exports
every entry point include/avq.h declares, sizes its workspace, and rejects
invalid arguments before anything is enqueued (those paths touch no device
memory and make no HIP call)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "avq.h")


@pytest.fixture(scope="module")
def lib():
    import adaptive_vector_quantized_avq_amd as avq
    if not os.path.exists(avq.library_path()):
        pytest.skip("libavq.so not built (run __graft_entry__.build())")
    return avq.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(avq_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("avq_build_tree", "avq_assign_aggregate", "avq_attention_fwd"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert lib.avq_abi_version() == 3
    assert lib.avq_status_string(0) == b"AVQ_OK"
    assert lib.avq_status_string(-1) == b"AVQ_ERR_INVALID_ARG"
    assert lib.avq_status_string(-2) == b"AVQ_ERR_UNSUPPORTED"
    assert lib.avq_status_string(-3) == b"AVQ_ERR_HIP"


def test_attention_workspace_size(lib):
    f = lib.avq_attention_workspace_size
    # per (b,h): parent sums [d][256] + counts [256] + child sums [257][d][8] +
    # counts [257][8] (one all-zero entry), then, for bf16, the counts as
    # three bf16 parts: parents [4][256], children [257][3][8]; each section
    # 256-byte aligned
    al = lambda x: (x + 255) // 256 * 256
    per = al(64 * 256 * 2) + al(256 * 4) + al(257 * 64 * 8 * 2) + al(257 * 8 * 4)
    assert f(1, 8, 256, 8, 64, 1) == 8 * (per + al(4 * 256 * 2) + al(257 * 3 * 8 * 2))
    assert f(1, 8, 256, 8, 64, 0) == 8 * (al(64 * 256 * 4) + al(256 * 4) + al(257 * 64 * 8 * 4) + al(257 * 8 * 4))
    assert f(1, 1, 300, 8, 64, 1) == 0
    assert f(0, 1, 16, 8, 64, 1) == 0


def _assign_ws(B, H, N, M0, C, d):
    """[B*H*N] int32 key list + [B*H][groups][ceil(N/1024) chunks] int2
    segments + each chunk's largest group count [B*H][chunks][2] i32 + the split
    groups' partial sums [B*H][ceil(N/target)][rows * (d + 1)] fp32 and their
    flags [B*H][ceil(N/target)] u32, each 256-aligned;
    groups of 4 parents (of 2 for C = 16 at d = 128), target = twice the
    mean group length and at least 1024 keys, rows = the group's slots
    rounded up to 16."""
    al = lambda x: (x + 255) // 256 * 256
    grp = 2 if (C == 16 and d == 128) else 4
    ngroups = -(-M0 // grp)
    target = max(1024, 2 * -(-N // ngroups))
    npart = -(-N // target)
    rows = -(-(grp * (C + 1)) // 16) * 16
    bh = B * H
    return (al(bh * N * 4) + al(bh * ngroups * -(-N // 1024) * 8) + al(bh * -(-N // 1024) * 8)
            + al(bh * npart * rows * (d + 1) * 4) + al(bh * npart * 4))


def test_workspace_size(lib):
    f = lib.avq_assign_aggregate_workspace_size
    assert f(1, 8, 65536, 256, 8, 64) == _assign_ws(1, 8, 65536, 256, 8, 64)
    assert f(2, 10, 32768, 256, 16, 128) == _assign_ws(2, 10, 32768, 256, 16, 128)
    assert f(2, 16, 16384, 128, 8, 64) == _assign_ws(2, 16, 16384, 128, 8, 64)
    # long-64k: lists 2 MiB, segments 256 KiB, chunk maxima 4 KiB, 32 partial
    # slots per head (target 2048 keys)
    assert _assign_ws(1, 8, 65536, 256, 8, 64) == 8 * 65536 * 4 + 262144 + 4096 + 8 * 32 * 48 * 65 * 4 + 1024
    assert f(1, 1, 1, 1, 4, 64) > 0
    assert f(1, 1, 1, 300, 4, 64) == 0      # M0 > 256 unsupported
    assert f(1, 1, 1, 8, 3, 64) == 0        # C = 3 unsupported
    assert f(1, 1, 0, 8, 4, 64) == 0        # N = 0 invalid


def _fake(n=1):
    # never dereferenced: every call below fails validation first
    return ctypes.c_void_p(0x1000 * n)


def test_invalid_arguments_are_rejected_before_launch(lib):
    import adaptive_vector_quantized_avq_amd  # noqa: F401  (sets argtypes)
    p = _fake()
    af = lib.avq_attention_fwd
    args = dict(Q=p, par=p, ch=p, vs=p, cn=p, B=1, H=1, N=128, d=64, M0=16, C=4, P=4, tile=64,
                scale=0.125, dt=1, ws=p, wsb=1 << 20)

    def call(**kw):
        a = dict(args, **kw)
        return af(a["Q"], a["par"], a["ch"], a["vs"], a["cn"], a["B"], a["H"], a["N"], a["d"],
                  a["M0"], a["C"], a["P"], a["tile"], a["scale"], a["dt"], p, None, None,
                  a["ws"], a["wsb"], None)

    assert call(Q=None) == -1
    assert call(vs=None) == -1
    assert call(cn=None) == -1
    assert call(ws=None) == -1
    assert call(wsb=64) == -1
    assert b"workspace" in lib.avq_last_error()
    assert call(ws=ctypes.c_void_p(0x1010)) == -1
    assert call(tile=16) == -2
    assert call(P=17) == -1
    assert call(P=-1) == -1
    assert call(N=0) == -1
    assert call(B=0) == -1
    assert call(tile=0) == -1
    assert call(scale=float("inf")) == -1
    assert call(dt=7) == -1
    assert call(d=96) == -2
    assert call(C=3) == -2
    assert call(C=0) == -1             # flat codebook: P must be 0
    assert call(C=-1) == -1
    assert call(M0=300, P=4) == -2
    assert call(tile=48) == -2
    assert b"tile" in lib.avq_last_error()
    assert call(N=(1 << 20) + 1) == -2

    aa = lib.avq_assign_aggregate
    # a valid call template; each case below breaks exactly one argument
    base = [p, p, p, p, p, p, 1, 1, 128, 64, 16, 4, 1, 0, p, p, None, p, 1 << 20, None]
    bad_flags = list(base)
    bad_flags[13] = 4
    assert aa(*bad_flags) == -1
    unfused_tree = list(base)          # the unfused path is for flat codebooks only
    unfused_tree[13] = 2
    assert aa(*unfused_tree) == -2
    flat_forced = list(base)           # C = 0 has no children to force
    flat_forced[11], flat_forced[13] = 0, 1
    assert aa(*flat_forced) == -1
    no_frame = list(base)
    no_frame[5] = None
    assert aa(*no_frame) == -1
    no_ws = list(base)
    no_ws[17] = None
    assert aa(*no_ws) == -1
    small_ws = list(base)
    small_ws[18] = 16
    assert aa(*small_ws) == -1
    misaligned = list(base)
    misaligned[17] = ctypes.c_void_p(0x1004)
    assert aa(*misaligned) == -1
    assert lib.avq_build_tree(None, 1, 4, 4, 64, 1, p, p, p, None) == -1
    assert lib.avq_build_tree(p, 1, 4, 4, 64, 1, p, p, None, None) == -1
    assert lib.avq_build_tree(p, 1, 4, 4, 64, 5, p, p, p, None) == -1
    assert lib.avq_exact_attention_fwd(p, p, p, 1, 1, 16, 80, 1.0, 1, p, None) == -2


@pytest.mark.parametrize("W,H", [(1, 1), (1, 9), (7, 1), (4, 4), (5, 3), (3, 5), (28, 28), (64, 64),
                                 (13, 40), (256, 256), (33, 18), (100, 7)])
def test_gilbert_order_matches_the_oracle(lib, W, H):
    # host code of the library (no GPU call) against the oracle's own
    # implementation of the curve
    import numpy as np
    import oracle
    import adaptive_vector_quantized_avq_amd as avq
    np.testing.assert_array_equal(avq.gilbert_order(W, H).numpy(), oracle.gilbert_order(W, H))


def test_gilbert_order_rejects_bad_grids(lib):
    import adaptive_vector_quantized_avq_amd as avq
    buf = ctypes.create_string_buffer(64)
    assert lib.avq_gilbert_order(0, 4, buf) == -1
    assert lib.avq_gilbert_order(2048, 1024, buf) == -2
    assert lib.avq_gilbert_order(4, 4, None) == -1
    assert avq.gilbert_order(2, 3).numel() == 6


def test_three_level_workspace_sizes(lib):
    al = lambda x: (x + 255) // 256 * 256
    # per (b,h): the two-level pack of 64 roots with 8 children, then the
    # children's leaf sums [513][d][8] and counts [513][8]
    per = (al(64 * 64 * 2) + al(64 * 4) + al(65 * 64 * 8 * 2) + al(65 * 8 * 4)
           + al(513 * 64 * 8 * 2) + al(513 * 8 * 4))
    assert lib.avq_attention3_workspace_size(1, 8, 64, 8, 64, 1) == 8 * per
    assert lib.avq_attention3_workspace_size(1, 8, 64, 0, 64, 1) == 0
    # the second descent's workspace (512 children as parents, in groups of
    # 4) + leaf ids
    want = _assign_ws(1, 8, 65536, 512, 8, 64) + al(8 * 65536 * 4)
    assert lib.avq_assign_aggregate3_workspace_size(1, 8, 65536, 64, 8, 64) == want
    assert lib.avq_assign_aggregate3_workspace_size(1, 8, 65536, 64, 0, 64) == 0


def test_three_level_rejects_bad_arguments(lib):
    p = ctypes.c_void_p(16)
    lib.avq_build_tree3.argtypes = [ctypes.c_void_p] + [ctypes.c_int] * 5 + [ctypes.c_void_p] * 5
    assert lib.avq_build_tree3(p, 1, 4, 0, 64, 1, p, p, p, p, None) == -1        # needs children
    assert lib.avq_build_tree3(p, 1, 4, 3, 64, 1, p, p, p, p, None) == -2        # C = 3
    assert lib.avq_build_tree3(None, 1, 4, 4, 64, 1, p, p, p, p, None) == -1
    f = lib.avq_attention3_fwd
    f.argtypes = ([ctypes.c_void_p] * 6 + [ctypes.c_int] * 8 + [ctypes.c_float, ctypes.c_int]
                  + [ctypes.c_void_p] * 4 + [ctypes.c_size_t, ctypes.c_void_p])
    big = 1 << 40
    # P*C = 272 level-1 candidates: more than a tile's selection handles
    assert f(p, p, p, p, p, p, 1, 1, 256, 64, 64, 16, 17, 128, 1.0, 1, p, None, None, p, big, None) == -2
    assert f(p, p, p, p, p, p, 1, 1, 256, 64, 64, 8, 65, 128, 1.0, 1, p, None, None, p, big, None) == -1
    g = lib.avq_assign_aggregate3
    g.argtypes = ([ctypes.c_void_p] * 7 + [ctypes.c_int] * 7 + [ctypes.c_uint]
                  + [ctypes.c_void_p] * 4 + [ctypes.c_size_t, ctypes.c_void_p])
    assert g(p, p, p, p, p, p, p, 1, 1, 256, 64, 8, 4, 1, 2, p, p, None, p, big, None) == -1   # unfused flag
