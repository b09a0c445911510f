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
    assert lib.avq_abi_version() == 1
    assert lib.avq_status_string(0) == b"AVQ_OK"
    assert lib.avq_status_string(-1) == b"AVQ_ERR_INVALID_ARG"
    assert lib.avq_status_string(-2) == b"AVQ_ERR_UNSUPPORTED"
    assert lib.avq_status_string(-3) == b"AVQ_ERR_HIP"


def test_operand_pack_size(lib):
    f = lib.avq_operand_pack_size
    # per (b,h): parent sums [d][256] + counts [256] + child sums [257][d][8] +
    # counts [257][8] (one all-zero entry), each section 256-byte aligned
    al = lambda x: (x + 255) // 256 * 256
    per = al(64 * 256 * 2) + al(256 * 4) + al(257 * 64 * 8 * 2) + al(257 * 8 * 4)
    assert f(1, 8, 256, 8, 64, 1) == 8 * per
    assert f(1, 1, 300, 8, 64, 1) == 0
    assert f(0, 1, 16, 8, 64, 1) == 0


def test_workspace_size(lib):
    f = lib.avq_assign_aggregate_workspace_size
    # [B*H*N] int32 key list + [B*H][ceil(M0/group) groups][ceil(N/1024) chunks]
    # int2 segments, each 256-aligned; groups of 4 parents, of 2 for C = 16 at
    # d = 128
    assert f(1, 8, 65536, 256, 8, 64) == 8 * 65536 * 4 + ((8 * 64 * 64 * 8 + 255) // 256) * 256
    assert f(2, 10, 32768, 256, 16, 128) == 20 * 32768 * 4 + ((20 * 128 * 32 * 8 + 255) // 256) * 256
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
    args = dict(Q=p, par=p, ch=p, pk=p, B=1, H=1, N=128, d=64, M0=16, C=4, P=4, tile=64,
                scale=0.125, dt=1)

    def call(**kw):
        a = dict(args, **kw)
        return af(a["Q"], a["par"], a["ch"], a["pk"], a["B"], a["H"], a["N"], a["d"],
                  a["M0"], a["C"], a["P"], a["tile"], a["scale"], a["dt"], p, None, None, None)

    assert call(Q=None) == -1
    assert call(pk=None) == -1
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
    assert call(M0=300, P=4) == -2
    assert call(tile=48) == -2
    assert b"tile" in lib.avq_last_error()
    # fp32 codebooks of 256 parents with 256-query tiles and a large P exceed
    # the attention kernel's 160 KB of LDS
    assert call(dt=0, M0=256, tile=256, P=200) == -2
    assert call(dt=0, d=128, M0=256, tile=256, P=240) == -2
    assert b"LDS" in lib.avq_last_error()
    assert call(N=(1 << 20) + 1) == -2

    aa = lib.avq_assign_aggregate
    # a valid call template; each case below breaks exactly one argument
    base = [p, p, p, p, p, 1, 1, 128, 64, 16, 4, 1, 0, p, p, None, p, p, 1 << 20, None]
    bad_flags = list(base)
    bad_flags[12] = 2
    assert aa(*bad_flags) == -1
    no_pack = list(base)
    no_pack[16] = None
    assert aa(*no_pack) == -1
    small_ws = list(base)
    small_ws[18] = 16
    assert aa(*small_ws) == -1
    misaligned = list(base)
    misaligned[17] = ctypes.c_void_p(0x1004)
    assert aa(*misaligned) == -1
    assert lib.avq_build_tree(None, 1, 4, 4, 64, 1, p, p, None) == -1
    assert lib.avq_build_tree(p, 1, 4, 4, 64, 5, p, p, None) == -1
    assert lib.avq_exact_attention_fwd(p, p, p, 1, 1, 16, 80, 1.0, 1, p, None) == -2
