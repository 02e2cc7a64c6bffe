"""Strict parity of the launches the 27B-like pass times, each fed the oracle's
own inputs (seeded synthetic tensors; nothing computed on the GPU is fed back):

* the fused gate/up GEMM with SwiGLU (34816 x 5120: two tiles per workgroup,
  the channel groups past the last full round as K slices, each group
  finished inside the launch by its slice that arrives last) from packed
  activations to packed output, at 1, 16 and 32 rows -- the 16-row MFMA
  shape below 17 rows, the 32-row shape above;
* the LM head (151936 x 5120) with its argmax and the fp32 logits dump, at 1,
  16 and 32 rows;
* the O (5120 x 5120) and down (5120 x 17408) projections with the residual
  add and the next RMSNorm, K-sliced exactly as in the pass, at 1, 16 and 32
  rows;
* one 27B-like decoder layer stage by stage at 32 nodes over a 4096-token
  context, tree attention included.

Rules (the oracle is fp64 between the bf16 rounding points): bf16 outputs
within one bf16 ulp of the oracle's value (or 2^-20 of the row's scale where
values cancel, or twice the fp32 accumulation bound where a residual cancels
the product) and at least 98% bit-identical; fp32 logits within the fp32
accumulation bound of every element and 2e-3 max-abs-rel per row; the argmax
equal to the first maximum of the dumped logits and, on every row whose
top-2 margin exceeds twice the row's error, to the oracle's argmax.  Every
launch is bitwise reproducible.
"""

import numpy as np
import pytest
import torch

from oracle import model as om
from oracle import w12 as ow12
from oracle.bf16 import from_bits, round_bf16, to_bits
from synth import best_first_topology, gen_linear_bf16, make_generator
from synth.configs import CONFIGS, LARGE_RECIPE, gen_kv_context, gen_layer
from synth.weights import bf16_bits_numpy, sub_seed
from tests.parity import row_max_abs_rel
from tests.test_gpu_stages import _same_bf16

pytestmark = pytest.mark.gpu

CFG = CONFIGS["27b"]
ROWS = (1, 16, 32)


@pytest.fixture(scope="module")
def tvp():
    import tree_verification_pass_amd as m
    return m


def _dev(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def _u16(t: torch.Tensor) -> np.ndarray:
    return bf16_bits_numpy(t.detach())


def pack_rows_host(x_bits: np.ndarray) -> np.ndarray:
    """The packed activation layout written on the host: element (row, k) at
    (k / 8) * 256 + row * 8 + k % 8, 32 row slots, k padded to 64 with zeros."""
    m, k = x_bits.shape
    kp = -(-k // 64) * 64
    out = np.zeros((kp // 8, 32, 8), np.uint16)
    xx = np.zeros((m, kp), np.uint16)
    xx[:, :k] = x_bits
    out[:, :m, :] = xx.reshape(m, kp // 8, 8).transpose(1, 0, 2)
    return out.reshape(-1)


def unpack_rows_host(p_bits: np.ndarray, m: int, k: int) -> np.ndarray:
    kp = -(-k // 64) * 64
    return p_bits[: kp * 32].reshape(kp // 8, 32, 8)[:, :m, :].transpose(1, 0, 2).reshape(m, kp)[:, :k]


def _acts(seed: int, m: int, k: int, std: float = 1.0) -> np.ndarray:
    g = make_generator(seed)
    return bf16_bits_numpy((torch.randn(m, k, generator=g) * std).to(torch.bfloat16))


def _weight(seed: int, n_out: int, k_in: int, dev):
    w = gen_linear_bf16(make_generator(seed, dev), n_out, k_in, LARGE_RECIPE, device=dev)
    return w, _u16(w)


def _encoder_sample_matches_oracle(t, w_bits: np.ndarray, seed: int):
    """The GPU encoder's planes equal the oracle encoder's on sampled channels."""
    cols = np.sort(np.random.default_rng(seed).choice(w_bits.shape[0], 64, replace=False))
    o = ow12.encode(w_bits[cols])
    assert np.array_equal(t.base.cpu().numpy()[cols], o.base)
    assert np.array_equal(t.hi.cpu().numpy()[cols], o.hi)
    assert np.array_equal(t.lo.cpu().numpy()[cols], o.lo)


# ----------------------------------------------------------------- gate/up
@pytest.fixture(scope="module")
def gateup(tvp, cuda):
    F, H = CFG.ffn, CFG.hidden
    w, bits = _weight(sub_seed(77, 1), 2 * F, H, cuda)
    t = tvp.w12_encode(w)
    _encoder_sample_matches_oracle(t, bits, 1)
    pw = tvp.w12_pack(t, tvp.TVP_CHAN_GATEUP, F)
    del t, w
    x = _acts(sub_seed(77, 2), 32, H)
    gu = from_bits(x) @ from_bits(bits).T  # fp64, the definition
    u_ref = round_bf16(om.silu(gu[:, :F]) * gu[:, F:])
    return pw, x, u_ref


@pytest.mark.parametrize("m", ROWS)
def test_gateup_swiglu_27b_strict(tvp, cuda, gateup, m):
    F, H = CFG.ffn, CFG.hidden
    pw, x, u_ref = gateup
    print(f"[strict 27b] gate/up + SwiGLU {2 * F}x{H}, m={m}", flush=True)
    xp = _dev(pack_rows_host(x[:m]), cuda)
    outs = []
    for _ in range(2):
        yp = torch.full((tvp.w12_packed_x_elems(F),), float("nan"), dtype=torch.bfloat16, device=cuda)
        tvp.w12_gemm_px(xp, m, pw, tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_SWIGLU, y=yp.data_ptr(), y_packed=1))
        torch.cuda.synchronize()
        outs.append(yp)
    assert torch.equal(outs[0][: F * 32].view(torch.int16), outs[1][: F * 32].view(torch.int16))
    got = from_bits(unpack_rows_host(_u16(outs[0]), m, F))
    _same_bf16(got, u_ref[:m], f"swiglu m={m}")


def test_gateup_handover_repeatable_27b(tvp, cuda, gateup):
    """The remaining groups' in-launch hand-over (device-scope slice stores,
    an arrival counter, the last slice summing them) over many launches in a
    row on one caller-held counter array, as the pass runs it: every launch
    gives the same bits and leaves the counters at zero."""
    F = CFG.ffn
    pw, x, _ = gateup
    m, reps = 32, 48
    print(f"[strict 27b] gate/up hand-over, {reps} launches, m={m}", flush=True)
    xp = _dev(pack_rows_host(x[:m]), cuda)
    cnt = torch.zeros(tvp.TVP_GEMM_COUNTERS, dtype=torch.int32, device=cuda)
    outs = []
    for _ in range(reps):
        yp = torch.full((tvp.w12_packed_x_elems(F),), float("nan"), dtype=torch.bfloat16, device=cuda)
        tvp.w12_gemm_px(xp, m, pw, tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_SWIGLU, y=yp.data_ptr(), y_packed=1,
                                                      counters=cnt.data_ptr()))
        outs.append(yp)
    torch.cuda.synchronize()
    assert int(cnt.abs().sum()) == 0
    ref = outs[0][: F * 32].view(torch.int16)
    same = [torch.equal(ref, o[: F * 32].view(torch.int16)) for o in outs[1:]]
    assert all(same), f"{same.count(False)} of {reps - 1} launches differ from the first"


# ----------------------------------------------------------------- LM head
@pytest.fixture(scope="module")
def lmhead(tvp, cuda):
    V, H = CFG.vocab, CFG.hidden
    w, bits = _weight(sub_seed(78, 1), V, H, cuda)
    t = tvp.w12_encode(w)
    _encoder_sample_matches_oracle(t, bits, 2)
    pw = tvp.w12_pack(t)
    del t, w
    x = _acts(sub_seed(78, 2), 32, H)
    xv = from_bits(x)
    ref = np.empty((32, V))
    bound = np.empty((32, V))
    for c0 in range(0, V, 8192):  # fp64 in chunks (the whole head would be 6 GB)
        wc = from_bits(bits[c0: c0 + 8192])
        ref[:, c0: c0 + 8192] = xv @ wc.T
        bound[:, c0: c0 + 8192] = np.abs(xv) @ np.abs(wc).T
    return pw, x, ref, bound


@pytest.mark.parametrize("m", ROWS)
def test_lm_head_argmax_27b_strict(tvp, cuda, lmhead, m):
    V, H = CFG.vocab, CFG.hidden
    pw, x, ref, bound = lmhead
    print(f"[strict 27b] LM head {V}x{H} + argmax, m={m}", flush=True)
    xp = _dev(pack_rows_host(x[:m]), cuda)
    res = []
    for _ in range(2):
        am = torch.full((m,), -7, dtype=torch.int32, device=cuda)
        lg = torch.full((m, V), float("nan"), dtype=torch.float32, device=cuda)
        tvp.w12_gemm_px(xp, m, pw, tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_ARGMAX, argmax=am.data_ptr(),
                                                       logits=lg.data_ptr(), ldl=V))
        torch.cuda.synchronize()
        res.append((am.cpu().numpy(), lg.cpu().numpy()))
    (am, lg), (am2, lg2) = res
    assert np.array_equal(am, am2) and np.array_equal(lg.view(np.int32), lg2.view(np.int32))
    g = lg.astype(np.float64)
    r, b = ref[:m], bound[:m]
    err = np.abs(g - r)
    worst = float((err / (b + 1e-300)).max())
    assert np.all(err <= 4.0 * H * 2.0 ** -24 * b + 1e-30), worst
    rel = row_max_abs_rel(g, r)
    assert rel.max() <= 2e-3
    assert np.array_equal(am, np.argmax(lg, axis=1))  # first maximum of the dumped logits
    part = np.partition(r, -2, axis=1)
    decidable = (part[:, -1] - part[:, -2]) > 2.0 * err.max(axis=1)
    print(f"  max_abs_rel={rel.max():.2e} err/bound={worst:.3f} decidable={decidable.mean():.3f}", flush=True)
    assert np.array_equal(am[decidable], np.argmax(r, axis=1)[decidable])


# ------------------------------------------ projection + residual + RMSNorm
def _resid_norm_ref(h_bits, x_bits, w_bits, g_bits, eps):
    xv, wv = from_bits(x_bits), from_bits(w_bits)
    acc = xv @ wv.T
    h1 = round_bf16(from_bits(h_bits) + acc)
    y = round_bf16(om.rmsnorm(h1, from_bits(g_bits), eps))
    fp32_err = 4.0 * xv.shape[1] * 2.0 ** -24 * (np.abs(xv) @ np.abs(wv).T)
    return h1, y, fp32_err


def _check_resid_norm(h_got, y_got, h_ref, y_ref, fp32_err, g_bits, eps, name):
    """h: one bf16 ulp of the oracle's value plus twice the fp32 accumulation
    bound (where the residual cancels the product), >= 98% bit-identical.
    The normed rows: one ulp, plus where the GPU's h took the other rounding
    (an fp32-vs-fp64 flip the h check allows) that difference carried through
    the norm; >= 98% bit-identical."""
    assert np.all(np.abs(h_got - h_ref) <= 2.0 ** -7 * np.abs(h_ref) + 2.0 * fp32_err), name
    exact = float(np.mean(h_got == h_ref))
    r = 1.0 / np.sqrt(np.mean(h_ref * h_ref, axis=1, keepdims=True) + eps)
    carried = np.abs(h_got - h_ref) * r * np.abs(from_bits(g_bits))[None, :] * (1.0 + 2.0 ** -7)
    scale = np.abs(y_ref).max(axis=1, keepdims=True)
    ok = np.abs(y_got - y_ref) <= np.maximum(2.0 ** -7 * np.abs(y_ref), 2.0 ** -20 * scale) + carried
    y_exact = float(np.mean(y_got == y_ref))
    print(f"  {name}: h exact={exact:.4f} norm exact={y_exact:.4f} h flips={np.mean(h_got != h_ref):.5f}", flush=True)
    assert exact >= 0.98 and y_exact >= 0.98, name
    assert ok.all(), name


@pytest.fixture(scope="module", params=["o", "down"])
def projection(request, tvp, cuda):
    H = CFG.hidden
    k = CFG.n_heads * CFG.head_dim if request.param == "o" else CFG.ffn
    w, bits = _weight(sub_seed(79, 1 if request.param == "o" else 2), H, k, cuda)
    pw = tvp.w12_pack(tvp.w12_encode(w))
    del w
    x = _acts(sub_seed(79, 3), 32, k)
    h = _acts(sub_seed(79, 4), 32, H)
    g = bf16_bits_numpy((1.0 + 0.1 * torch.randn(H, generator=make_generator(sub_seed(79, 5)))).to(torch.bfloat16))
    h1, y, fp32_err = _resid_norm_ref(h, x, bits, g, CFG.norm_eps)
    return request.param, pw, x, h, g, h1, y, fp32_err


@pytest.mark.parametrize("m", ROWS)
def test_projection_resid_norm_27b_strict(tvp, cuda, projection, m):
    name, pw, x, h, g, h1_ref, y_ref, fp32_err = projection
    H, k = CFG.hidden, x.shape[1]
    print(f"[strict 27b] {name} {H}x{k} + residual + RMSNorm, m={m}", flush=True)
    xp = _dev(pack_rows_host(x[:m]), cuda)
    gd = _dev(g, cuda)
    outs = []
    for _ in range(2):
        hd = _dev(h[:m], cuda).clone()
        yp = tvp.w12_gemm_resid_norm(xp, m, pw, hd, gd, CFG.norm_eps)
        torch.cuda.synchronize()
        outs.append((_u16(hd), unpack_rows_host(_u16(yp), m, H)))  # the rows the call writes
    assert all(np.array_equal(a, b) for a, b in zip(outs[0], outs[1]))
    _check_resid_norm(from_bits(outs[0][0]), from_bits(outs[0][1]), h1_ref[:m], y_ref[:m], fp32_err[:m], g,
                      CFG.norm_eps, f"{name} m={m}")


# --------------------------------------------------- one layer, stage by stage
def test_stages_27b_one_layer(tvp, cuda):
    """One 27B-like decoder layer at 32 nodes over a 4096-token context: each
    GPU stage receives the oracle's input to that stage and must reproduce
    the oracle's output; the stages run in the pass's launch configurations
    (packed activations in and out, K-sliced projections finished by the
    fused residual + RMSNorm)."""
    dev = cuda
    cfg = CFG
    L, n = cfg.ctx_len, cfg.n_nodes
    hq, hkv, d, H, F = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.hidden, cfg.ffn
    s_max = L + 64
    lay = gen_layer(cfg, 81, 0, device=dev, gains="random")
    lb = {k: _u16(v) for k, v in lay.items()}
    w = {k: from_bits(v) for k, v in lb.items()}
    packed = {"wqkv": tvp.w12_pack(tvp.w12_encode(lay["wqkv"]), tvp.TVP_CHAN_QKV, hq, hkv, d),
              "wo": tvp.w12_pack(tvp.w12_encode(lay["wo"])),
              "wgu": tvp.w12_pack(tvp.w12_encode(lay["wgu"]), tvp.TVP_CHAN_GATEUP, F),
              "wdown": tvp.w12_pack(tvp.w12_encode(lay["wdown"]))}
    del lay
    kc0, vc0 = gen_kv_context(cfg, 81, 0, L, s_max)
    rng = np.random.default_rng(81)
    parents = best_first_topology(rng, n)[0]
    pos = L + om._accept.depths(parents)
    vis = np.concatenate([np.ones((n, L), bool), om.ancestor_mask(parents)], axis=1)
    h = round_bf16(np.random.default_rng(82).standard_normal((n, H)))  # a residual stream entering the layer
    post = torch.as_tensor(pos.astype(np.int32), device=dev)
    slot = torch.as_tensor((L + np.arange(n)).astype(np.int32), device=dev)
    par_t = torch.as_tensor(parents.astype(np.int32), device=dev)
    print("[strict 27b] one layer, 32 nodes, ctx 4096", flush=True)
    # QKV with RoPE and the KV write (packed input)
    a = round_bf16(om.rmsnorm(h, w["attn_norm"], cfg.norm_eps))
    qkv = a @ w["wqkv"].T
    q_r = round_bf16(om.rope(qkv[:, : hq * d].reshape(n, hq, d), pos, cfg.rope_theta))
    k_r = round_bf16(om.rope(qkv[:, hq * d: (hq + hkv) * d].reshape(n, hkv, d), pos, cfg.rope_theta))
    v_r = round_bf16(qkv[:, (hq + hkv) * d:].reshape(n, hkv, d))
    kc, vc = kc0.clone().to(dev), vc0.clone().to(dev)
    q = torch.zeros(n, hq * d, dtype=torch.bfloat16, device=dev)
    epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_QKV, y=q.data_ptr(), ldy=hq * d, pos=post.data_ptr(),
                              slot=slot.data_ptr(), k_cache=kc.data_ptr(), v_cache=vc.data_ptr(),
                              s_stride=s_max, rope_theta=cfg.rope_theta)
    tvp.w12_gemm_px(_dev(pack_rows_host(to_bits(a)), dev), n, packed["wqkv"], epi)
    torch.cuda.synchronize()
    _same_bf16(from_bits(_u16(q)), q_r.reshape(n, -1), "q")
    _same_bf16(from_bits(_u16(kc))[:, L: L + n].transpose(1, 0, 2), k_r, "k")
    _same_bf16(from_bits(_u16(vc))[:, L: L + n].transpose(1, 0, 2), v_r, "v")
    # tree attention over the oracle's q, k, v
    kc2, vc2 = kc0.clone(), vc0.clone()
    kc2[:, L: L + n] = _dev(to_bits(k_r.transpose(1, 0, 2)), "cpu")
    vc2[:, L: L + n] = _dev(to_bits(v_r.transpose(1, 0, 2)), "cpu")
    keys = from_bits(bf16_bits_numpy(kc2))[:, : L + n]
    vals = from_bits(bf16_bits_numpy(vc2))[:, : L + n]
    o_r = round_bf16(om.attention(q_r, keys, vals, vis))
    o_g, st = tvp.tree_attention(_dev(to_bits(q_r), dev), kc2.to(dev), vc2.to(dev), L, par_t)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    _same_bf16(from_bits(_u16(o_g)), o_r, "attention")
    # O projection + residual + the FFN norm (K slices, fused residual + RMSNorm)
    h1_ref, b_ref, fp32_err = _resid_norm_ref(to_bits(h), to_bits(o_r.reshape(n, -1)), lb["wo"], lb["ffn_norm"],
                                              cfg.norm_eps)
    hd = _dev(to_bits(h), dev).clone()
    bp = tvp.w12_gemm_resid_norm(_dev(pack_rows_host(to_bits(o_r.reshape(n, -1))), dev), n, packed["wo"], hd,
                                 _dev(lb["ffn_norm"], dev), cfg.norm_eps)
    torch.cuda.synchronize()
    _check_resid_norm(from_bits(_u16(hd)), from_bits(unpack_rows_host(_u16(bp), n, H)), h1_ref, b_ref, fp32_err,
                      lb["ffn_norm"], cfg.norm_eps, "o + residual + ffn norm")
    # gate/up + SwiGLU, packed in and out
    gu = b_ref @ w["wgu"].T
    u_r = round_bf16(om.silu(gu[:, :F]) * gu[:, F:])
    up = torch.zeros(tvp.w12_packed_x_elems(F), dtype=torch.bfloat16, device=dev)
    tvp.w12_gemm_px(_dev(pack_rows_host(to_bits(b_ref)), dev), n, packed["wgu"],
                    tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_SWIGLU, y=up.data_ptr(), y_packed=1))
    torch.cuda.synchronize()
    _same_bf16(from_bits(unpack_rows_host(_u16(up), n, F)), u_r, "swiglu")
    # down projection + residual + the next norm
    h2_ref, a2_ref, fp32_err = _resid_norm_ref(to_bits(h1_ref), to_bits(u_r), lb["wdown"], lb["attn_norm"],
                                               cfg.norm_eps)
    hd = _dev(to_bits(h1_ref), dev).clone()
    ap = tvp.w12_gemm_resid_norm(_dev(pack_rows_host(to_bits(u_r)), dev), n, packed["wdown"], hd,
                                 _dev(lb["attn_norm"], dev), cfg.norm_eps)
    torch.cuda.synchronize()
    _check_resid_norm(from_bits(_u16(hd)), from_bits(unpack_rows_host(_u16(ap), n, H)), h2_ref, a2_ref, fp32_err,
                      lb["attn_norm"], cfg.norm_eps, "down + residual + next norm")
