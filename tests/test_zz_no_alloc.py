"""The GEMM entry point that allocates nothing (w12_gemm_ex_noalloc, scratch
in a library-owned per-GPU device array) against the GEMM with a caller
workspace (w12_gemm_ex), through the C ABI: bit-identical outputs on calls
in a row whose inputs shrink (a 27B-like LM-head slice with its argmax and
logits, a SwiGLU GEMM whose remaining channel groups run as K slices, a
one-row plain GEMM), each also against the oracle's fp64 product; shapes whose
scratch would not fit the array are refused before any launch."""

import numpy as np
import pytest
import torch

from oracle.bf16 import from_bits
from synth import gen_linear_bf16, make_generator
from synth.configs import LARGE_RECIPE, TINY_RECIPE
from synth.weights import bf16_bits_numpy
from tests.parity import row_max_abs_rel

pytestmark = pytest.mark.gpu


def _x(m, k, seed, dev):
    return torch.randn(m, k, generator=make_generator(seed)).to(torch.bfloat16).to(dev)


def test_noalloc_gemm_equals_workspace_gemm(cuda):
    import tree_verification_pass_amd as tvp

    # call 1: 8192 x 5120 with the argmax epilogue and the logits dump, 32 rows
    # row-major (the activations are packed into the scratch first)
    V, H = 8192, 5120
    print("[noalloc] argmax 8192x5120, m=32", flush=True)
    w = gen_linear_bf16(make_generator(501, cuda), V, H, LARGE_RECIPE, device=cuda)
    wb = bf16_bits_numpy(w)
    pw = tvp.w12_pack(tvp.w12_encode(w))
    x = _x(32, H, 502, cuda)
    outs = []
    for fn in (tvp.w12_gemm_ex_noalloc, None):
        am = torch.full((32,), -1, dtype=torch.int32, device=cuda)
        lg = torch.full((32, V), float("nan"), dtype=torch.float32, device=cuda)
        epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_ARGMAX, argmax=am.data_ptr(), logits=lg.data_ptr(), ldl=V)
        if fn is None:
            tvp.w12_gemm_ex(x, pw, epi)
        else:
            fn(x, 32, pw, epi)
        torch.cuda.synchronize()
        outs.append((am.cpu().numpy(), lg.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1].view(np.int32), outs[1][1].view(np.int32))
    ref = from_bits(bf16_bits_numpy(x)) @ from_bits(wb).T
    assert row_max_abs_rel(outs[0][1].astype(np.float64), ref).max() <= 2e-3
    assert np.array_equal(outs[0][0], np.argmax(outs[0][1], axis=1))

    # call 2 (smaller): SwiGLU with 263 tiles, 9 rows -- the groups past the
    # last full round run as K slices whose sums sit in the scratch
    Hs, F = 1000, 4200
    print("[noalloc] swiglu 8400x1000, m=9", flush=True)
    wg = gen_linear_bf16(make_generator(503, cuda), 2 * F, Hs, TINY_RECIPE, device=cuda)
    pg = tvp.w12_pack(tvp.w12_encode(wg), tvp.TVP_CHAN_GATEUP, F)
    xs = _x(9, Hs, 504, cuda)
    us = []
    for use_noalloc in (True, False):
        u = torch.full((9, F), float("nan"), dtype=torch.bfloat16, device=cuda)
        epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_SWIGLU, y=u.data_ptr(), ldy=F)
        if use_noalloc:
            tvp.w12_gemm_ex_noalloc(xs, 9, pg, epi)
        else:
            tvp.w12_gemm_ex(xs, pg, epi)
        torch.cuda.synchronize()
        us.append(u.cpu().view(torch.int16).numpy())
    assert np.array_equal(us[0], us[1])

    # call 3 (smaller still): one row, plain fp32 output
    print("[noalloc] f32 96x200, m=1", flush=True)
    w3 = gen_linear_bf16(make_generator(505, cuda), 96, 200, TINY_RECIPE, device=cuda)
    p3 = tvp.w12_pack(tvp.w12_encode(w3))
    x3 = _x(1, 200, 506, cuda)
    y_a = torch.full((1, 96), float("nan"), dtype=torch.float32, device=cuda)
    tvp.w12_gemm_ex_noalloc(x3, 1, p3, tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_F32, y=y_a.data_ptr(), ldy=96))
    y_b = tvp.w12_gemm(x3, p3, out_fp32=True)
    torch.cuda.synchronize()
    assert torch.equal(y_a, y_b)
    ref3 = from_bits(bf16_bits_numpy(x3)) @ from_bits(bf16_bits_numpy(w3)).T
    assert row_max_abs_rel(y_a.cpu().numpy().astype(np.float64), ref3).max() <= 2e-3


def test_noalloc_refuses_scratch_beyond_its_array(cuda):
    import tree_verification_pass_amd as tvp

    # 192 rows over 34816 x 5120 takes the wide path, whose split sums need far
    # more than the array holds: refused before any launch
    w = gen_linear_bf16(make_generator(507, cuda), 2 * 17408, 5120, LARGE_RECIPE, device=cuda)
    pw = tvp.w12_pack(tvp.w12_encode(w))
    assert tvp.w12_gemm_workspace(192, pw) > 8 << 20
    x = _x(192, 5120, 508, cuda)
    y = torch.zeros(192, 2 * 17408, dtype=torch.bfloat16, device=cuda)
    with pytest.raises(tvp.TvpError) as e:
        tvp.w12_gemm_ex_noalloc(x, 192, pw, tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_BF16, y=y.data_ptr(), ldy=2 * 17408))
    assert e.value.status == tvp.TVP_ERR_WORKSPACE
