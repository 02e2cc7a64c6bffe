"""The INT8 LM head with its Cauchy-Schwarz certified candidate filter on the
GPU against the oracle (through the C ABI).

* Encoding, against ``oracle.lmhead_i8.encode``: the int8 values, scales,
  escape columns and values bit for bit; the residual norm not below the
  oracle's exact one (within 2^-20 above), the GPU's working radius above it.
* Approximate logits within the fp32 accumulation bound of the oracle's.
* The certified argmax at 1, 13 and 32 rows equals the oracle's (the exact
  argmax) on a ragged head with duplicated rows (exact ties go to the
  smallest id), and at the full 151936 x 5120 LM head equals the exact fp64
  argmax and the W12 head's argmax on every row whose top-2 margin exceeds
  twice the fp32 accumulation bound; the certified sets stay small.
"""

import numpy as np
import pytest
import torch

from oracle import lmhead_i8 as oh
from oracle.bf16 import from_bits, round_bf16, to_bits
from synth import gen_linear_bf16, make_generator
from synth.configs import LARGE_RECIPE
from synth.weights import bf16_bits_numpy, sub_seed
from tests.test_gpu_strict_27b import pack_rows_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tvp():
    import tree_verification_pass_amd as m
    return m


def _u16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _dev(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


@pytest.fixture(scope="module")
def ragged(tvp, cuda):
    V, k = 3001, 1000
    w = bf16_bits_numpy(gen_linear_bf16(make_generator(sub_seed(91, 1)), V, k, LARGE_RECIPE))
    rng = np.random.default_rng(91)
    dup = rng.choice(V, 40, replace=False)
    w[dup[1:]] = w[dup[0]]  # exact ties between rows
    wd = _dev(w, cuda)
    head = tvp.lmhead_i8_encode(wd)
    exact = tvp.w12_encode(wd)
    return w, head, exact, oh.encode(w)


def test_i8_encode_matches_oracle(tvp, cuda, ragged):
    w, head, _, ref = ragged
    print("[i8 head] encode 3001 x 1000", flush=True)
    assert np.array_equal(head.q.cpu().numpy(), ref.q)
    assert np.array_equal(head.scale.cpu().numpy().view(np.uint32), ref.scale.view(np.uint32))
    assert np.array_equal(head.esc_col.cpu().numpy().view(np.uint16).astype(np.int64), ref.esc_col)
    assert np.array_equal(from_bits(head.esc_val.cpu().numpy().view(np.uint16)), ref.esc_val)
    r = head.r.cpu().numpy().astype(np.float64)
    r_ref = ref.r.astype(np.float64)
    assert np.all(r >= r_ref * (1 - 2.0 ** -23)) and np.all(r <= r_ref * (1 + 2.0 ** -20))
    assert np.all(head.r_eff.cpu().numpy() >= head.r.cpu().numpy())


@pytest.mark.parametrize("m", [1, 13, 32])
def test_i8_argmax_matches_oracle_ragged(tvp, cuda, ragged, m):
    w, head, exact, ref = ragged
    print(f"[i8 head] argmax 3001 x 1000, m={m}", flush=True)
    f = round_bf16(np.random.default_rng(100 + m).standard_normal((m, 1000)))
    if m > 1:
        f[1] = 0.0  # every logit equal: the smallest id
    xp = _dev(pack_rows_host(to_bits(f)), cuda)
    am, nc, apx = tvp.lmhead_i8_argmax(xp, m, head, exact, want_approx=True)
    am2, _, _ = tvp.lmhead_i8_argmax(xp, m, head, exact)
    torch.cuda.synchronize()
    assert torch.equal(am, am2)
    a_ref = oh.approx_logits(f, ref)
    bound = 4.0 * 1000 * 2.0 ** -24 * (np.abs(f) @ np.abs(ref.dequant()).T) * ref.scale.astype(np.float64)[None, :]
    assert np.all(np.abs(apx.cpu().numpy().astype(np.float64) - a_ref) <= bound + 1e-30)
    want = oh.argmax(f, ref, w)
    got = am.cpu().numpy()
    exact_lg = f @ from_bits(w).T
    part = np.sort(exact_lg, axis=1)
    acc = 4.0 * 1000 * 2.0 ** -24 * (np.abs(f) @ np.abs(from_bits(w)).T).max(axis=1)
    decidable = (part[:, -1] - part[:, -2] > 2 * acc) | (part[:, -1] == part[:, 0])
    print(f"  candidates per row: max {int(nc.max())}, mean {float(nc.float().mean()):.1f}; "
          f"decidable {decidable.mean():.3f}", flush=True)
    assert np.array_equal(got[decidable], want[decidable])
    if m > 1:
        assert got[1] == 0  # all equal: id 0


def test_i8_argmax_full_head(tvp, cuda):
    V, H = 151936, 5120
    print(f"[i8 head] full LM head {V} x {H}, m=32", flush=True)
    wd = gen_linear_bf16(make_generator(sub_seed(92, 1), cuda), V, H, LARGE_RECIPE, device=cuda)
    head = tvp.lmhead_i8_encode(wd)
    exact = tvp.w12_encode(wd)
    pw = tvp.w12_pack(exact)
    w = bf16_bits_numpy(wd)
    del wd
    x = bf16_bits_numpy(torch.randn(32, H, generator=make_generator(sub_seed(92, 2))).to(torch.bfloat16))
    xp = _dev(pack_rows_host(x), cuda)
    am, nc, _ = tvp.lmhead_i8_argmax(xp, 32, head, exact)
    am_w12 = torch.zeros(32, dtype=torch.int32, device=cuda)
    tvp.w12_gemm_px(xp, 32, pw, tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_ARGMAX, argmax=am_w12.data_ptr()))
    torch.cuda.synchronize()
    xv = from_bits(x)
    top2 = np.full((32, 2), -np.inf)
    top1_id = np.zeros(32, np.int64)
    acc = np.zeros(32)
    for c0 in range(0, V, 8192):
        wc = from_bits(w[c0: c0 + 8192])
        lg = xv @ wc.T
        acc = np.maximum(acc, (4.0 * H * 2.0 ** -24 * (np.abs(xv) @ np.abs(wc).T)).max(axis=1))
        both = np.concatenate([top2, np.sort(lg, axis=1)[:, -2:]], axis=1)
        i = np.argmax(lg, axis=1)
        better = lg[np.arange(32), i] > top2[:, 1]
        top1_id = np.where(better, c0 + i, top1_id)
        top2 = np.sort(both, axis=1)[:, -2:]
    decidable = top2[:, 1] - top2[:, 0] > 2 * acc
    got, w12 = am.cpu().numpy(), am_w12.cpu().numpy()
    print(f"  candidates per row: max {int(nc.max())}, mean {float(nc.float().mean()):.2f}; "
          f"decidable {decidable.mean():.3f}", flush=True)
    assert np.array_equal(got[decidable], top1_id[decidable])
    assert np.array_equal(got[decidable], w12[decidable])
    assert int(nc.min()) >= 1 and int(nc.max()) <= 64
