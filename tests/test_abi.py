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


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_w12_validate_host_only():
    """The library's host-side format check of a canonical tensor's side data
    accepts what the oracle's encoder writes and rejects each kind of damage:
    a window base outside 1..239, escape pointers that do not run from 0 to
    n_esc without decreasing, escape columns out of order or past k_in."""
    import numpy as np

    import tree_verification_pass_amd as tvp
    from oracle import w12 as ow12
    from synth import gen_linear_bf16, make_generator
    from synth.configs import TINY_RECIPE
    from synth.weights import bf16_bits_numpy

    k = 300
    t = ow12.encode(bf16_bits_numpy(gen_linear_bf16(make_generator(11), 40, k, TINY_RECIPE)))
    assert t.n_esc > 40  # several escapes per channel on this recipe
    ok = lambda b, p, i, kk=k: tvp.w12_validate(b, p, i, kk)  # noqa: E731
    assert ok(t.base, t.esc_ptr, t.esc_idx) == tvp.TVP_OK
    # the all-patterns channel: base 1, 61440 escapes, columns up to 65535
    allpat = np.random.default_rng(7).permutation(65536).astype(np.uint16)[None, :]
    ta = ow12.encode(allpat)
    assert ok(ta.base, ta.esc_ptr, ta.esc_idx, 65536) == tvp.TVP_OK
    bad = []
    for b in (0, 240, 255):
        base = t.base.copy()
        base[7] = b
        bad.append((base, t.esc_ptr, t.esc_idx, k))
    p = t.esc_ptr.copy()
    p[0] = 1
    bad.append((t.base, p, t.esc_idx, k))
    p = t.esc_ptr.copy()
    p[-1] -= 1
    bad.append((t.base, p, t.esc_idx, k))
    p = t.esc_ptr.copy()
    j = int(np.flatnonzero(np.diff(p.astype(np.int64)) >= 2)[0])  # a channel with >= 2 escapes
    p[j + 1], p[j + 2] = p[j + 2] + 1, p[j + 1]  # decreasing pair inside the CSR
    bad.append((t.base, p, t.esc_idx, k))
    i = t.esc_idx.copy()
    a = int(t.esc_ptr[j])
    i[a], i[a + 1] = i[a + 1], i[a]  # two columns of one channel swapped
    bad.append((t.base, t.esc_ptr, i, k))
    i = t.esc_idx.copy()
    i[a + 1] = i[a]  # a repeated column
    bad.append((t.base, t.esc_ptr, i, k))
    i = t.esc_idx.copy()
    last = int(t.esc_ptr[j + 1]) - 1
    i[last] = k  # past the last column
    bad.append((t.base, t.esc_ptr, i, k))
    bad.append((t.base, t.esc_ptr, t.esc_idx, 70000))  # k_in beyond uint16 columns
    for case in bad:
        assert ok(*case) == tvp.TVP_ERR_FORMAT
