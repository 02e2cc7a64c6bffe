"""Host checks of the C-ABI library: it loads and exports every declared entry point."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tvp.h")
LIB = os.path.join(ROOT, "tree_verification_pass_amd", "libtvp.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^(?:const\s+)?[A-Za-z_][\w]*\s*\**\s+\**([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_pass():
    names = declared_functions()
    for must in ("w12_encode_count", "w12_encode", "w12_decode", "w12_gemm", "tree_attention", "accept_path",
                 "tvp_plan_create", "verify_step", "verify_step_batched", "tvp_plan_destroy"):
        assert must in names


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_status_strings_and_binding_names():
    import tree_verification_pass_amd as tvp
    assert tvp.tvp_status_string(0) == "ok"
    assert "tree" in tvp.tvp_status_string(3)
    assert set(tvp.EXPORTED) <= set(declared_functions())


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_pack_size_layout_host_only():
    import tree_verification_pass_amd as tvp
    p = tvp.w12_pack_size(1000, 1000, 37)
    assert p.n_tiles == 32 and p.n_kb == 16
    assert p.off_rec == 0 and p.off_escoff >= 32 * 16 * 3072 and p.bytes % 256 == 0
    q = tvp.w12_pack_size(2 * 1000, 512, 0, tvp.TVP_CHAN_GATEUP, 1000)
    assert q.n_tiles == 63
    r = tvp.w12_pack_size((6 + 4) * 64, 1000, 0, tvp.TVP_CHAN_QKV, 6, 2, 64)
    assert r.n_tiles == 8 * 2 + 4
    with pytest.raises(tvp.TvpError):
        tvp.w12_pack_size(100, 70000, 0)
    with pytest.raises(tvp.TvpError):
        tvp.w12_pack_size(2 * 1000, 512, 0, tvp.TVP_CHAN_GATEUP, 999)


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_packed_activation_size_host_only():
    import tree_verification_pass_amd as tvp
    # 32 row slots x k padded to a multiple of 64
    for k, want in ((0, 0), (1, 2048), (64, 2048), (65, 4096), (5120, 80 * 2048), (17408, 272 * 2048)):
        assert tvp.w12_packed_x_elems(k) == want
