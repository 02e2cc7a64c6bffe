"""GPU parity of the individual kernels against the CPU oracle (through the C ABI).

W12 encoder bytes and decode: bit-exact.  GEMM: within the logits tolerance
(max-abs-rel 2e-3) and within an fp32 accumulation bound, and bitwise
reproducible.  Tree attention: within bf16 rounding bounds.  Acceptance: exact.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import w12 as ow12
from oracle import model as om
from oracle.accept import accept as oaccept
from oracle.bf16 import from_bits, round_bf16
from synth import LinearRecipe, best_first_topology, gen_linear_bf16, make_generator
from synth.configs import LARGE_RECIPE, TINY_RECIPE
from synth.weights import bf16_bits_numpy
from tests.parity import row_max_abs_rel

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "w12_handworked.json")


@pytest.fixture(scope="module")
def tvp():
    import tree_verification_pass_amd as m
    return m


def _u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def _gpu_w12_equals_oracle(t, o: ow12.W12Tensor):
    assert t.n_esc == o.n_esc
    assert np.array_equal(t.hi.cpu().numpy(), o.hi)
    assert np.array_equal(t.lo.cpu().numpy(), o.lo)
    assert np.array_equal(t.base.cpu().numpy(), o.base)
    assert np.array_equal(t.esc_ptr.cpu().numpy().view(np.uint32), o.esc_ptr)
    if o.n_esc:
        assert np.array_equal(_u16(t.esc_idx)[: o.n_esc], o.esc_idx)
        assert np.array_equal(_u16(t.esc_val)[: o.n_esc], o.esc_val)


def _cases():
    g = json.load(open(GOLDEN))
    hand = np.array([[int(x, 16) for x in r] for r in g["weights"]], dtype=np.uint16)
    allpat = np.random.default_rng(7).permutation(65536).astype(np.uint16)
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((37, 1000)) * 10.0 ** rng.uniform(-6, 2, (37, 1))).astype(np.float32)
    x[rng.random(x.shape) < 0.03] = 0
    ragged = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    ragged[rng.random(ragged.shape) < 0.005] = 0x7FC1
    cfg_w = bf16_bits_numpy(gen_linear_bf16(make_generator(3), 96, 5120, LARGE_RECIPE))
    tiny_w = bf16_bits_numpy(gen_linear_bf16(make_generator(4), 64, 512, TINY_RECIPE))
    return {"handworked": hand, "all_patterns_row": allpat[None, :], "all_patterns_256": allpat.reshape(256, 256),
            "ragged": ragged, "large_recipe": cfg_w, "tiny_recipe": tiny_w}


@pytest.mark.parametrize("name", list(_cases().keys()))
def test_encoder_bytes_and_decode_bit_exact(tvp, cuda, name):
    w = _cases()[name]
    print(f"[w12 codec] {name} shape={w.shape}", flush=True)
    wt = torch.from_numpy(w.view(np.int16).copy()).view(torch.bfloat16).to(cuda)
    t = tvp.w12_encode(wt)
    _gpu_w12_equals_oracle(t, ow12.encode(w))
    assert np.array_equal(_u16(tvp.w12_decode(t)), w)


def _packed(tvp, w_bits: np.ndarray, cuda, chan_map=0, a=0, b=0, c=0):
    wt = torch.from_numpy(w_bits.view(np.int16).copy()).view(torch.bfloat16).to(cuda)
    return tvp.w12_pack(tvp.w12_encode(wt), chan_map, a, b, c)


def _x(m, k, seed, cuda):
    g = make_generator(seed)
    return torch.randn(m, k, generator=g).to(torch.bfloat16).to(cuda)


def _check_gemm(y_fp32: np.ndarray, x_bits: np.ndarray, w_bits: np.ndarray):
    xv, wv = from_bits(x_bits), from_bits(w_bits)
    ref = xv @ wv.T
    bound = np.abs(xv) @ np.abs(wv).T
    k = xv.shape[1]
    err = np.abs(y_fp32 - ref)
    assert np.all(err <= 4.0 * k * 2.0 ** -24 * bound + 1e-30), float((err / (bound + 1e-30)).max())
    assert row_max_abs_rel(y_fp32, ref).max() <= 2e-3
    return ref


@pytest.mark.parametrize("m", [1, 5, 16, 17, 32, 33, 100, 129, 160, 192])
def test_gemm_ragged_shapes(tvp, cuda, m):
    w_bits = bf16_bits_numpy(gen_linear_bf16(make_generator(8), 1000, 1000, TINY_RECIPE))
    print(f"[gemm] m={m} n=1000 k=1000", flush=True)
    pw = _packed(tvp, w_bits, cuda)
    x = _x(m, 1000, 100 + m, cuda)
    y32 = tvp.w12_gemm(x, pw, out_fp32=True)
    y16 = tvp.w12_gemm(x, pw, out_fp32=False)
    torch.cuda.synchronize()
    ref = _check_gemm(y32.cpu().numpy().astype(np.float64), _u16(x), w_bits)
    # bf16 output is the fp32 result rounded once
    assert np.array_equal(_u16(y16), np.asarray(
        torch.from_numpy(y32.cpu().numpy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)))
    # ... so it is within half a bf16 ulp of the fp32 result
    g16 = from_bits(_u16(y16))
    assert np.all(np.abs(g16 - y32.cpu().numpy()) <= 2.0 ** -8 * np.abs(y32.cpu().numpy()))
    # bitwise reproducible
    y32b = tvp.w12_gemm(x, pw, out_fp32=True)
    assert torch.equal(y32, y32b)


@pytest.mark.parametrize("n_out,k_in", [(17408, 5120), (5120, 17408), (6144, 5120)])
@pytest.mark.parametrize("m", [1, 16, 32])
def test_gemm_27b_shapes_sampled(tvp, cuda, n_out, k_in, m):
    """Full 27B-like GEMM shapes (weights [K x N] read as K_in x N_out): every
    output row is checked on a sample of 256 channels against the oracle."""
    print(f"[gemm 27b] n_out={n_out} k_in={k_in} m={m}", flush=True)
    g = make_generator(1000 + n_out + k_in, "cuda")
    w = gen_linear_bf16(g, n_out, k_in, LARGE_RECIPE)
    t = tvp.w12_encode(w)
    pw = tvp.w12_pack(t)
    x = _x(m, k_in, 7 + m, cuda)
    y = tvp.w12_gemm(x, pw, out_fp32=True)
    torch.cuda.synchronize()
    cols = np.sort(np.random.default_rng(n_out + m).choice(n_out, 256, replace=False))
    w_s = bf16_bits_numpy(w[torch.as_tensor(cols, device=cuda)])
    _check_gemm(y.cpu().numpy()[:, cols].astype(np.float64), _u16(x), w_s)
    # the encoder is checked byte for byte on the same sampled channels
    o = ow12.encode(w_s)
    assert np.array_equal(t.base.cpu().numpy()[cols], o.base)
    assert np.array_equal(t.hi.cpu().numpy()[cols], o.hi)
    y2 = tvp.w12_gemm(x, pw, out_fp32=True)
    assert torch.equal(y, y2)


def test_gemm_fused_epilogues(tvp, cuda):
    H, F, hq, hkv, d = 1000, 1000, 6, 2, 64
    m = 13
    print("[gemm epilogues] resid/swiglu/qkv/argmax", flush=True)
    rng = np.random.default_rng(0)
    # residual
    w_o = bf16_bits_numpy(gen_linear_bf16(make_generator(21), H, hq * d, TINY_RECIPE))
    x = _x(m, hq * d, 1, cuda)
    res = _x(m, H, 2, cuda)
    y = res.clone()
    epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_RESID, y=y.data_ptr(), ldy=H, resid=y.data_ptr(), ldr=H)
    tvp.w12_gemm_ex(x, _packed(tvp, w_o, cuda), epi)
    torch.cuda.synchronize()
    acc = from_bits(_u16(x)) @ from_bits(w_o).T
    ref = round_bf16(from_bits(_u16(res)) + acc)
    got = from_bits(_u16(y))
    # one bf16 ulp, plus the fp32 accumulation bound where res + acc cancels
    fp32_err = 4.0 * (hq * d) * 2.0 ** -24 * (np.abs(from_bits(_u16(x))) @ np.abs(from_bits(w_o)).T)
    assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 2.0 * fp32_err)
    assert np.mean(got == ref) > 0.98
    # swiglu with the gate/up channel map
    w_gu = bf16_bits_numpy(gen_linear_bf16(make_generator(22), 2 * F, H, TINY_RECIPE))
    xb = _x(m, H, 3, cuda)
    u = torch.zeros(m, F, dtype=torch.bfloat16, device=cuda)
    epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_SWIGLU, y=u.data_ptr(), ldy=F)
    tvp.w12_gemm_ex(xb, _packed(tvp, w_gu, cuda, tvp.TVP_CHAN_GATEUP, F), epi)
    torch.cuda.synchronize()
    gu = from_bits(_u16(xb)) @ from_bits(w_gu).T
    ref = round_bf16(om.silu(gu[:, :F]) * gu[:, F:])
    got = from_bits(_u16(u))
    assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-6 * np.abs(ref).max())
    # qkv: rope at positions, k and v written to cache slots
    w_qkv = bf16_bits_numpy(gen_linear_bf16(make_generator(23), (hq + 2 * hkv) * d, H, TINY_RECIPE))
    xa = _x(m, H, 4, cuda)
    s_max = 64
    kc = torch.zeros(hkv, s_max, d, dtype=torch.bfloat16, device=cuda)
    vc = torch.zeros_like(kc)
    q = torch.zeros(m, hq * d, dtype=torch.bfloat16, device=cuda)
    pos = rng.integers(0, 9000, m).astype(np.int32)
    slot = rng.permutation(s_max)[:m].astype(np.int32)
    pos_t, slot_t = torch.as_tensor(pos, device=cuda), torch.as_tensor(slot, device=cuda)
    epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_QKV, y=q.data_ptr(), ldy=hq * d, pos=pos_t.data_ptr(),
                              slot=slot_t.data_ptr(), k_cache=kc.data_ptr(), v_cache=vc.data_ptr(),
                              s_stride=s_max, rope_theta=1e6)
    tvp.w12_gemm_ex(xa, _packed(tvp, w_qkv, cuda, tvp.TVP_CHAN_QKV, hq, hkv, d), epi)
    torch.cuda.synchronize()
    qkv = from_bits(_u16(xa)) @ from_bits(w_qkv).T
    q_ref = round_bf16(om.rope(qkv[:, : hq * d].reshape(m, hq, d), pos, 1e6)).reshape(m, hq * d)
    k_ref = round_bf16(om.rope(qkv[:, hq * d: (hq + hkv) * d].reshape(m, hkv, d), pos, 1e6))
    v_ref = round_bf16(qkv[:, (hq + hkv) * d:].reshape(m, hkv, d))
    for got, ref in ((from_bits(_u16(q)), q_ref),
                     (from_bits(_u16(kc)).transpose(1, 0, 2)[slot], k_ref),
                     (from_bits(_u16(vc)).transpose(1, 0, 2)[slot], v_ref)):
        assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-4 * np.abs(ref).max())
        assert np.mean(got == ref) > 0.97
    # argmax over a vocabulary, ties to the smallest id, plus the logits dump
    V = 3000
    w_lm = bf16_bits_numpy(gen_linear_bf16(make_generator(24), V, H, TINY_RECIPE))
    w_lm[:, :] = w_lm[:, :]
    am = torch.zeros(m, dtype=torch.int32, device=cuda)
    lg = torch.zeros(m, V, dtype=torch.float32, device=cuda)
    epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_ARGMAX, argmax=am.data_ptr(), logits=lg.data_ptr(), ldl=V)
    tvp.w12_gemm_ex(xa, _packed(tvp, w_lm, cuda), epi)
    torch.cuda.synchronize()
    lg_np = lg.cpu().numpy().astype(np.float64)
    ref = from_bits(_u16(xa)) @ from_bits(w_lm).T
    assert row_max_abs_rel(lg_np, ref).max() <= 2e-3
    assert np.array_equal(am.cpu().numpy(), np.argmax(lg.cpu().numpy(), axis=1))


@pytest.mark.parametrize("m", [9, 32])
def test_gemm_remaining_groups_split_over_k(tvp, cuda, m):
    """More channel groups than CUs, not a multiple of them: the groups past
    the last full round are computed as K slices, and the slice of a group
    that arrives last sums them and applies the epilogue.  Each whole-K
    epilogue through that path against the oracle."""
    H, F, hq, hkv, d = 1000, 4200, 120, 8, 64  # 263, 263 and 272 tiles of 32 channels
    print(f"[gemm remaining groups] m={m} swiglu/resid/qkv", flush=True)
    rng = np.random.default_rng(m)
    w_gu = bf16_bits_numpy(gen_linear_bf16(make_generator(41), 2 * F, H, TINY_RECIPE))
    xb = _x(m, H, 42, cuda)
    u = torch.zeros(m, F, dtype=torch.bfloat16, device=cuda)
    epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_SWIGLU, y=u.data_ptr(), ldy=F)
    pgu = _packed(tvp, w_gu, cuda, tvp.TVP_CHAN_GATEUP, F)
    tvp.w12_gemm_ex(xb, pgu, epi)
    torch.cuda.synchronize()
    gu = from_bits(_u16(xb)) @ from_bits(w_gu).T
    ref = round_bf16(om.silu(gu[:, :F]) * gu[:, F:])
    got = from_bits(_u16(u))
    assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-6 * np.abs(ref).max())
    u2 = torch.zeros_like(u)
    tvp.w12_gemm_ex(xb, pgu, tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_SWIGLU, y=u2.data_ptr(), ldy=F))
    torch.cuda.synchronize()
    assert torch.equal(u, u2)  # reproducible bit for bit
    # residual add on 8400 plain channels
    w_o = bf16_bits_numpy(gen_linear_bf16(make_generator(43), 2 * F, H, TINY_RECIPE))
    x = _x(m, H, 44, cuda)
    res = _x(m, 2 * F, 45, cuda)
    y = res.clone()
    epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_RESID, y=y.data_ptr(), ldy=2 * F, resid=y.data_ptr(), ldr=2 * F)
    tvp.w12_gemm_ex(x, _packed(tvp, w_o, cuda), epi)
    torch.cuda.synchronize()
    acc = from_bits(_u16(x)) @ from_bits(w_o).T
    ref = round_bf16(from_bits(_u16(res)) + acc)
    got = from_bits(_u16(y))
    fp32_err = 4.0 * H * 2.0 ** -24 * (np.abs(from_bits(_u16(x))) @ np.abs(from_bits(w_o)).T)
    assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 2.0 * fp32_err)
    assert np.mean(got == ref) > 0.98
    # qkv: rope at positions, k and v written to cache slots
    w_qkv = bf16_bits_numpy(gen_linear_bf16(make_generator(46), (hq + 2 * hkv) * d, H, TINY_RECIPE))
    xa = _x(m, H, 47, cuda)
    s_max = 64
    kc = torch.zeros(hkv, s_max, d, dtype=torch.bfloat16, device=cuda)
    vc = torch.zeros_like(kc)
    q = torch.zeros(m, hq * d, dtype=torch.bfloat16, device=cuda)
    pos = rng.integers(0, 9000, m).astype(np.int32)
    slot = rng.permutation(s_max)[:m].astype(np.int32)
    pos_t, slot_t = torch.as_tensor(pos, device=cuda), torch.as_tensor(slot, device=cuda)
    epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_QKV, y=q.data_ptr(), ldy=hq * d, pos=pos_t.data_ptr(),
                              slot=slot_t.data_ptr(), k_cache=kc.data_ptr(), v_cache=vc.data_ptr(),
                              s_stride=s_max, rope_theta=1e6)
    tvp.w12_gemm_ex(xa, _packed(tvp, w_qkv, cuda, tvp.TVP_CHAN_QKV, hq, hkv, d), epi)
    torch.cuda.synchronize()
    qkv = from_bits(_u16(xa)) @ from_bits(w_qkv).T
    q_ref = round_bf16(om.rope(qkv[:, : hq * d].reshape(m, hq, d), pos, 1e6)).reshape(m, hq * d)
    k_ref = round_bf16(om.rope(qkv[:, hq * d: (hq + hkv) * d].reshape(m, hkv, d), pos, 1e6))
    v_ref = round_bf16(qkv[:, (hq + hkv) * d:].reshape(m, hkv, d))
    for got, ref in ((from_bits(_u16(q)), q_ref),
                     (from_bits(_u16(kc)).transpose(1, 0, 2)[slot], k_ref),
                     (from_bits(_u16(vc)).transpose(1, 0, 2)[slot], v_ref)):
        assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-4 * np.abs(ref).max())
        assert np.mean(got == ref) > 0.97


@pytest.mark.parametrize("m", [1, 16, 32])
def test_gemm_caller_counters_match_and_stay_zero(tvp, cuda, m):
    """Arrival counters held by the caller (as the verification pass holds
    them): every call leaves them at zero, and the result is the same bits as
    a call whose counters the library clears in its workspace.  Two weights
    with remaining groups (263 and 272 tiles) alternate over four calls."""
    H, F = 1000, 4200
    print(f"[gemm caller counters] m={m}", flush=True)
    w_gu = bf16_bits_numpy(gen_linear_bf16(make_generator(51), 2 * F, H, TINY_RECIPE))
    w_pl = bf16_bits_numpy(gen_linear_bf16(make_generator(52), 8704, H, TINY_RECIPE))
    xb = _x(m, H, 53, cuda)
    pgu = _packed(tvp, w_gu, cuda, tvp.TVP_CHAN_GATEUP, F)
    ppl = _packed(tvp, w_pl, cuda)
    cnt = torch.zeros(tvp.TVP_GEMM_COUNTERS, dtype=torch.int32, device=cuda)

    def run(counters):
        u = torch.zeros(m, F, dtype=torch.bfloat16, device=cuda)
        y = torch.zeros(m, 8704, dtype=torch.bfloat16, device=cuda)
        tvp.w12_gemm_ex(xb, pgu, tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_SWIGLU, y=u.data_ptr(), ldy=F,
                                                     counters=counters))
        tvp.w12_gemm_ex(xb, ppl, tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_BF16, y=y.data_ptr(), ldy=8704,
                                                     counters=counters))
        torch.cuda.synchronize()
        return u, y

    u0, y0 = run(None)
    for _ in range(2):
        u1, y1 = run(cnt.data_ptr())
        assert torch.equal(u0, u1) and torch.equal(y0, y1)
        assert int(cnt.abs().sum()) == 0
    xv, wv = from_bits(_u16(xb)), from_bits(w_pl)
    ref = xv @ wv.T
    fp32_err = 4.0 * H * 2.0 ** -24 * (np.abs(xv) @ np.abs(wv).T)
    got = from_bits(_u16(y0))
    assert np.all(np.abs(got - round_bf16(ref)) <= 2.0 ** -7 * np.abs(ref) + 2.0 * fp32_err)


@pytest.mark.parametrize("m", [4, 70])  # skinny kernel's epilogue; wide kernel's fix-up (8 threads per row)
def test_argmax_ties_go_to_smallest_id(tvp, cuda, m):
    # identical channels produce exactly equal logits: the smallest id must win
    H, V = 256, 2048
    base = bf16_bits_numpy(gen_linear_bf16(make_generator(31), 1, H, TINY_RECIPE))
    w = np.repeat(base, V, axis=0)
    rng = np.random.default_rng(2)
    w[rng.permutation(V)[:1500]] = bf16_bits_numpy(gen_linear_bf16(make_generator(32), 1500, H, TINY_RECIPE))
    x = _x(m, H, 9, cuda)
    am = torch.zeros(m, dtype=torch.int32, device=cuda)
    lg = torch.zeros(m, V, dtype=torch.float32, device=cuda)
    epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_ARGMAX, argmax=am.data_ptr(), logits=lg.data_ptr(), ldl=V)
    tvp.w12_gemm_ex(x, _packed(tvp, w, cuda), epi)
    torch.cuda.synchronize()
    lgn = lg.cpu().numpy()
    assert np.array_equal(am.cpu().numpy(), np.argmax(lgn, axis=1))  # numpy: first maximum


def _attn_case(cuda, n, hq, hkv, d, L, seed, parents=None):
    rng = np.random.default_rng(seed)
    if parents is None:
        parents, _, _ = best_first_topology(rng, n)
    s_max = L + n + 5
    g = make_generator(seed)
    q = torch.randn(n, hq, d, generator=g).to(torch.bfloat16)
    kc = torch.randn(hkv, s_max, d, generator=g).to(torch.bfloat16)
    vc = torch.randn(hkv, s_max, d, generator=g).to(torch.bfloat16)
    return parents, q, kc, vc


def _attn_ref(parents, q, kc, vc, L):
    n = len(parents)
    qv = from_bits(_u16(q))
    kv = from_bits(_u16(kc))[:, : L + n]
    vv = from_bits(_u16(vc))[:, : L + n]
    vis = np.concatenate([np.ones((n, L), bool), om.ancestor_mask(parents)], axis=1)
    return round_bf16(om.attention(qv, kv, vv, vis)), np.abs(vv).max()


@pytest.mark.parametrize("n,hq,hkv,d,L", [(32, 40, 8, 128, 4096), (32, 32, 8, 128, 2048), (8, 8, 8, 64, 256),
                                          (13, 6, 2, 64, 300), (1, 4, 4, 128, 0), (64, 4, 1, 64, 700),
                                          (5, 10, 2, 128, 513),
                                          # two 32-row blocks per workgroup: three blocks (one pair
                                          # half empty), one pair with a single split, four blocks
                                          (13, 5, 1, 128, 300), (32, 8, 4, 128, 100), (20, 12, 2, 128, 1500),
                                          # merges over more than one pass of 8 splits: one-node decoding
                                          # (15 splits of 288 keys) and 32 splits of 256 keys
                                          (1, 40, 8, 128, 4096), (2, 8, 2, 64, 8000)])
def test_tree_attention_matches_oracle(tvp, cuda, n, hq, hkv, d, L):
    print(f"[tree_attention] n={n} hq={hq} hkv={hkv} d={d} L={L}", flush=True)
    parents, q, kc, vc = _attn_case(cuda, n, hq, hkv, d, L, seed=n + L)
    out, st = tvp.tree_attention(q.to(cuda), kc.to(cuda), vc.to(cuda), L, torch.as_tensor(parents, device=cuda))
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref, vmax = _attn_ref(parents, q, kc, vc, L)
    got = from_bits(_u16(out))
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * vmax + 2.0 ** -7 * np.abs(ref)), float(np.abs(got - ref).max())
    out2, _ = tvp.tree_attention(q.to(cuda), kc.to(cuda), vc.to(cuda), L, torch.as_tensor(parents, device=cuda))
    assert torch.equal(out, out2)


def test_tree_attention_merge_repeatable(tvp, cuda):
    """The in-launch split merge (device-scope partial stores, an arrival
    counter per row block, the last split merging every split in split
    order) at the 27B-like shape, 32 nodes over 4096 keys, over many
    launches in a row: every launch gives the same bits."""
    n, hq, hkv, d, L, reps = 32, 40, 8, 128, 4096, 48
    print(f"[tree_attention] merge over {reps} launches n={n} hq={hq} hkv={hkv} L={L}", flush=True)
    parents, q, kc, vc = _attn_case(cuda, n, hq, hkv, d, L, seed=7)
    qd, kd, vd = q.to(cuda), kc.to(cuda), vc.to(cuda)
    pd = torch.as_tensor(parents, device=cuda)
    outs = [tvp.tree_attention(qd, kd, vd, L, pd) for _ in range(reps)]
    torch.cuda.synchronize()
    assert all(int(st.item()) == 0 for _, st in outs)
    same = [torch.equal(outs[0][0], o) for o, _ in outs[1:]]
    assert all(same), f"{same.count(False)} of {reps - 1} launches differ from the first"


def test_tree_attention_chain_equals_causal_and_star(tvp, cuda):
    n, hq, hkv, d, L = 16, 8, 2, 128, 100
    for parents in (np.arange(-1, n - 1, dtype=np.int32), np.array([-1] + [0] * (n - 1), dtype=np.int32)):
        _, q, kc, vc = _attn_case(cuda, n, hq, hkv, d, L, seed=3, parents=parents)
        out, st = tvp.tree_attention(q.to(cuda), kc.to(cuda), vc.to(cuda), L, torch.as_tensor(parents, device=cuda))
        ref, vmax = _attn_ref(parents, q, kc, vc, L)
        got = from_bits(_u16(out))
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * vmax + 2.0 ** -7 * np.abs(ref))


@pytest.mark.parametrize("n,hq,hkv,d,L,spare", [(32, 40, 8, 128, 4064, 0), (7, 8, 2, 64, 250, 0),
                                                (13, 6, 2, 128, 500, 9)])
def test_tree_attention_never_reads_past_the_keys(tvp, cuda, n, hq, hkv, d, L, spare):
    """Caches whose slots from ctx_len + n on hold NaN (spare > 0), and caches
    filled exactly to their capacity (ctx_len + n == s_stride) that sit in a
    larger NaN-filled allocation: no key at or past the last tree slot may
    contribute (the ragged last block of a split is read as zeros), so the
    output is finite and equals the oracle."""
    print(f"[tree_attention bounds] n={n} hq={hq} hkv={hkv} d={d} L={L} spare={spare}", flush=True)
    parents, q, kc0, vc0 = _attn_case(cuda, n, hq, hkv, d, L, seed=3 * n + L)
    s = L + n + spare
    pad = 4096 * d
    caches = []
    for src in (kc0, vc0):
        flat = torch.full((hkv * s * d + pad,), float("nan"), dtype=torch.bfloat16, device=cuda)
        view = flat[: hkv * s * d].view(hkv, s, d)
        view[:, : L + n] = src[:, : L + n].to(cuda)
        caches.append((flat, view))
    (kf, kc), (vf, vc) = caches
    out, st = tvp.tree_attention(q.to(cuda), kc, vc, L, torch.as_tensor(parents, device=cuda))
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got = from_bits(_u16(out))
    assert np.isfinite(got).all()
    ref, vmax = _attn_ref(parents, q, kc0, vc0, L)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * vmax + 2.0 ** -7 * np.abs(ref)), float(np.abs(got - ref).max())


def test_tree_attention_malformed_tree_status(tvp, cuda):
    _, q, kc, vc = _attn_case(cuda, 4, 4, 4, 64, 10, seed=1, parents=np.array([-1, 0, 1, 2]))
    bad = torch.as_tensor(np.array([-1, 0, 3, 1], dtype=np.int32), device=cuda)
    out, st = tvp.tree_attention(q.to(cuda), kc.to(cuda), vc.to(cuda), 10, bad)
    torch.cuda.synchronize()
    assert int(st.item()) == tvp.TVP_ERR_TREE
    assert torch.isfinite(out.float()).all()


def test_accept_path_exact(tvp, cuda):
    rng = np.random.default_rng(4)
    print("[accept_path] random trees", flush=True)
    for trial in range(200):
        n = int(rng.integers(1, 100))
        parents = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, n)], dtype=np.int32)
        tokens = rng.integers(0, 3, n).astype(np.int32)
        am = rng.integers(0, 3, n).astype(np.int32)
        path, na, bonus, st = tvp.accept_path(torch.as_tensor(am, device=cuda), torch.as_tensor(tokens, device=cuda),
                                              torch.as_tensor(parents, device=cuda))
        p_ref, a_ref, b_ref = oaccept(am, tokens, parents)
        a = int(na.item())
        assert int(st.item()) == 0
        assert a == a_ref and int(bonus.item()) == b_ref
        assert path.cpu().numpy()[: a + 1].tolist() == p_ref
    for bad in ([0, 0], [-1, 1], [-1, 0, 2]):
        b = np.array(bad, dtype=np.int32)
        path, na, bonus, st = tvp.accept_path(torch.as_tensor(b, device=cuda), torch.as_tensor(b, device=cuda),
                                              torch.as_tensor(b, device=cuda))
        assert int(st.item()) == tvp.TVP_ERR_TREE and int(na.item()) == 0


def _packed_layout_host(x_bits: np.ndarray, k_pad: int) -> np.ndarray:
    """The packed activation layout written out element by element: (row, k)
    at (k // 8) * 256 + row * 8 + k % 8, 32 row slots, zeros elsewhere."""
    m, k_in = x_bits.shape
    out = np.zeros(k_pad * 32, np.uint16)
    for r in range(m):
        for k in range(k_in):
            out[(k // 8) * 256 + r * 8 + k % 8] = x_bits[r, k]
    return out


@pytest.mark.parametrize("m,k_in", [(1, 1000), (13, 1000), (17, 64), (32, 200)])
def test_packed_activation_layout(tvp, cuda, m, k_in):
    """w12_pack_x against the layout written out on the host, then the GEMM on
    packed input equals the GEMM on row-major input bit for bit (and the
    oracle within the GEMM bound), including the packed SwiGLU output."""
    print(f"[packed x] m={m} k_in={k_in}", flush=True)
    k_pad = -(-k_in // 64) * 64
    assert tvp.w12_packed_x_elems(k_in) == k_pad * 32
    x = _x(m, k_in, 300 + m, cuda)
    xp = tvp.w12_pack_x(x)
    torch.cuda.synchronize()
    assert np.array_equal(_u16(xp), _packed_layout_host(_u16(x), k_pad))
    w_bits = bf16_bits_numpy(gen_linear_bf16(make_generator(9), 96, k_in, TINY_RECIPE))
    pw = _packed(tvp, w_bits, cuda)
    y_row = tvp.w12_gemm(x, pw, out_fp32=True)
    y_pk = torch.zeros_like(y_row)
    tvp.w12_gemm_px(xp, m, pw, tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_F32, y=y_pk.data_ptr(), ldy=96))
    torch.cuda.synchronize()
    assert torch.equal(y_row, y_pk)
    _check_gemm(y_pk.cpu().numpy().astype(np.float64), _u16(x), w_bits)
    # SwiGLU written packed, read back through the host layout
    F = 80
    w_gu = bf16_bits_numpy(gen_linear_bf16(make_generator(10), 2 * F, k_in, TINY_RECIPE))
    pgu = _packed(tvp, w_gu, cuda, tvp.TVP_CHAN_GATEUP, F)
    u_row = torch.zeros(m, F, dtype=torch.bfloat16, device=cuda)
    tvp.w12_gemm_ex(x, pgu, tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_SWIGLU, y=u_row.data_ptr(), ldy=F))
    u_pk = torch.full((tvp.w12_packed_x_elems(F),), 7.0, dtype=torch.bfloat16, device=cuda)
    tvp.w12_gemm_px(xp, m, pgu, tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_SWIGLU, y=u_pk.data_ptr(), y_packed=1))
    torch.cuda.synchronize()
    got = _u16(u_pk)
    want = _u16(u_row)
    for r in range(m):
        for k in range(F):
            assert got[(k // 8) * 256 + r * 8 + k % 8] == want[r, k], (r, k)
    gu = from_bits(_u16(x)) @ from_bits(w_gu).T
    ref = round_bf16(om.silu(gu[:, :F]) * gu[:, F:])
    assert np.all(np.abs(from_bits(want) - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-6 * np.abs(ref).max())


def test_host_validation_launches_nothing(tvp, cuda):
    pw = _packed(tvp, bf16_bits_numpy(gen_linear_bf16(make_generator(1), 64, 64, TINY_RECIPE)), cuda)
    with pytest.raises(tvp.TvpError) as e:
        tvp.w12_gemm(_x(200, 64, 1, cuda), pw)
    assert e.value.status == tvp.TVP_ERR_SHAPE
    with pytest.raises(tvp.TvpError) as e:
        tvp.w12_gemm_ex(_x(4, 64, 1, cuda), pw, tvp.TvpGemmEpilogue(mode=99))
    assert e.value.status == tvp.TVP_ERR_ARG
    with pytest.raises(tvp.TvpError) as e:  # SwiGLU needs the gate/up channel map
        y = torch.zeros(4, 64, dtype=torch.bfloat16, device=cuda)
        tvp.w12_gemm_ex(_x(4, 64, 1, cuda), pw, tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_SWIGLU, y=y.data_ptr(), ldy=64))
    assert e.value.status == tvp.TVP_ERR_ARG
    # packed layouts: at most 32 rows, packed output only for SwiGLU
    with pytest.raises(tvp.TvpError) as e:
        tvp.w12_pack_x(_x(33, 64, 1, cuda))
    assert e.value.status == tvp.TVP_ERR_SHAPE
    xp = tvp.w12_pack_x(_x(4, 64, 1, cuda))
    y = torch.zeros(33, 64, dtype=torch.float32, device=cuda)
    with pytest.raises(tvp.TvpError) as e:
        tvp.w12_gemm_px(xp, 33, pw, tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_F32, y=y.data_ptr(), ldy=64))
    assert e.value.status == tvp.TVP_ERR_ARG
    with pytest.raises(tvp.TvpError) as e:
        tvp.w12_gemm_px(xp, 4, pw, tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_F32, y=y.data_ptr(), ldy=64, y_packed=1))
    assert e.value.status == tvp.TVP_ERR_ARG
    # a malformed canonical tensor is refused by the packer before any launch
    w = torch.from_numpy(bf16_bits_numpy(gen_linear_bf16(make_generator(2), 64, 200, TINY_RECIPE)).view(np.int16)
                         .copy()).view(torch.bfloat16).to(cuda)
    t = tvp.w12_encode(w)
    assert t.n_esc >= 2
    for damage in ("base", "order", "column"):
        t2 = tvp.W12Tensor(t.n_out, t.k_in, t.n_esc, t.hi, t.lo, t.base.clone(), t.esc_ptr, t.esc_idx.clone(),
                           t.esc_val)
        if damage == "base":
            t2.base[5] = 240
        elif damage == "order":
            i = t2.esc_idx.cpu().numpy().view(np.uint16).copy()
            ptr = t.esc_ptr.cpu().numpy()
            r = int(np.flatnonzero(np.diff(ptr) >= 2)[0])
            i[ptr[r]], i[ptr[r] + 1] = i[ptr[r] + 1], i[ptr[r]]
            t2.esc_idx.copy_(torch.from_numpy(i.view(np.int16)))
        else:
            t2.esc_idx[0] = 200
        with pytest.raises(tvp.TvpError) as e:
            tvp.w12_pack(t2)
        assert e.value.status == tvp.TVP_ERR_FORMAT, damage


def test_read_probe_reads_every_word_once(tvp, cuda):
    """The streaming-read probe of the measurement folds every 32-bit word of
    its input exactly once: the XOR of its 4096 output words is the XOR of the
    input (checked on a buffer that is not a multiple of the grid's stride)."""
    print("[read probe] 3 MiB + 48 B", flush=True)
    n_words = (3 << 20) // 4 + 12
    words = np.random.default_rng(5).integers(0, 2 ** 32, n_words, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32).copy()).to(cuda)
    sink = torch.zeros(4096, dtype=torch.int32, device=cuda)
    tvp.tvp_read_probe(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(words))
