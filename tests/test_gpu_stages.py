"""Every step of the verification pass on the GPU, fed the oracle's own inputs.

For each layer of the tiny and ragged targets, each GPU stage (fused QKV GEMM
with RoPE and the KV write, tree attention, O projection with the residual,
gate/up GEMM with SwiGLU, down projection with the residual, and the LM head
with its argmax) receives the oracle's input to that stage and must reproduce
the oracle's output: bf16 stage outputs within one bf16 ulp and at least 98%
bit-identical, logits within 2e-3 max-abs-rel (in practice ~1e-7).  The
inputs come from the oracle and the seeded generators only; nothing is fed
back from the GPU.  End-to-end comparisons of the composed pass are in
test_gpu_verify.py.
"""

import numpy as np
import pytest
import torch

from oracle import model as om
from oracle.bf16 import from_bits, round_bf16, to_bits
from synth import best_first_topology
from synth.configs import CONFIGS, gen_kv_context
from synth.weights import bf16_bits_numpy
from tests.helpers import model_bits
from tests.parity import row_max_abs_rel

pytestmark = pytest.mark.gpu


def _T(bits_np, dev):
    return torch.from_numpy(np.ascontiguousarray(bits_np).view(np.int16)).view(torch.bfloat16).to(dev)


def _U(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _same_bf16(got: np.ndarray, ref: np.ndarray, name: str, min_exact: float = 0.98):
    got = np.asarray(got, np.float64).reshape(ref.shape)
    # one bf16 ulp of the value, or a 2^-20 share of its row's scale (values
    # that cancel to almost nothing carry no relative precision)
    scale = np.abs(ref.reshape(ref.shape[0], -1)).max(axis=1).reshape((-1,) + (1,) * (ref.ndim - 1))
    ulp_ok = np.abs(got - ref) <= np.maximum(2.0 ** -7 * np.abs(ref), 2.0 ** -20 * scale)
    exact = float(np.mean(got == ref))
    print(f"  {name:10s} exact={exact:.4f} max_abs_rel={row_max_abs_rel(got.reshape(got.shape[0], -1), ref.reshape(ref.shape[0], -1)).max():.2e}",
          flush=True)
    assert ulp_ok.all(), name
    assert exact >= min_exact, (name, exact)


@pytest.mark.parametrize("cfg_name", ["tiny", "ragged"])
def test_each_stage_matches_oracle(cuda, cfg_name):
    import tree_verification_pass_amd as tvp

    cfg = CONFIGS[cfg_name]
    dev = cuda
    embed, layers, fnorm, lm = model_bits(cfg, 3, "random")
    orc = om.OracleModel.from_bits(om.Dims.of(cfg), embed, layers, fnorm, lm)
    L = cfg.ctx_len
    s_max = L + 64
    hq, hkv, d, H, F = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.hidden, cfg.ffn
    rng = np.random.default_rng(4)
    n = 24
    parents = best_first_topology(rng, n)[0]
    tokens = rng.integers(0, cfg.vocab, n)
    pos = L + om._accept.depths(parents)
    vis = np.concatenate([np.ones((n, L), bool), om.ancestor_mask(parents)], axis=1)
    h = orc.embed[tokens]
    post = torch.as_tensor(pos.astype(np.int32), device=dev)
    slot = torch.as_tensor((L + np.arange(n)).astype(np.int32), device=dev)
    par_t = torch.as_tensor(parents.astype(np.int32), device=dev)
    for li in range(cfg.n_layers):
        print(f"[stages] {cfg_name} layer {li}", flush=True)
        w, lb = orc.layers[li], layers[li]
        kc0, vc0 = gen_kv_context(cfg, 3, li, L, s_max)
        # fused QKV with RoPE and the KV write
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
        wqkv = tvp.w12_pack(tvp.w12_encode(_T(lb["wqkv"], dev)), tvp.TVP_CHAN_QKV, hq, hkv, d)
        tvp.w12_gemm_ex(_T(to_bits(a), dev), wqkv, epi)
        torch.cuda.synchronize()
        _same_bf16(from_bits(_U(q)), q_r.reshape(n, -1), "q")
        _same_bf16(from_bits(_U(kc))[:, L: L + n].transpose(1, 0, 2), k_r, "k")
        _same_bf16(from_bits(_U(vc))[:, L: L + n].transpose(1, 0, 2), v_r, "v")
        # tree attention over the oracle's q, k, v
        kc2, vc2 = kc0.clone(), vc0.clone()
        kc2[:, L: L + n] = _T(to_bits(k_r.transpose(1, 0, 2)), "cpu")
        vc2[:, L: L + n] = _T(to_bits(v_r.transpose(1, 0, 2)), "cpu")
        keys = from_bits(bf16_bits_numpy(kc2))[:, : L + n]
        vals = from_bits(bf16_bits_numpy(vc2))[:, : L + n]
        o_r = round_bf16(om.attention(q_r, keys, vals, vis))
        o_g, st = tvp.tree_attention(_T(to_bits(q_r), dev), kc2.to(dev), vc2.to(dev), L, par_t)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        _same_bf16(from_bits(_U(o_g)), o_r, "attention")
        # O projection + residual
        h1 = round_bf16(h + o_r.reshape(n, -1) @ w["wo"].T)
        y = _T(to_bits(h), dev).clone()
        epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_RESID, y=y.data_ptr(), ldy=H, resid=y.data_ptr(), ldr=H)
        tvp.w12_gemm_ex(_T(to_bits(o_r.reshape(n, -1)), dev), tvp.w12_pack(tvp.w12_encode(_T(lb["wo"], dev))), epi)
        torch.cuda.synchronize()
        _same_bf16(from_bits(_U(y)), h1, "o+resid")
        # gate/up + SwiGLU
        b = round_bf16(om.rmsnorm(h1, w["ffn_norm"], cfg.norm_eps))
        gu = b @ w["wgu"].T
        u_r = round_bf16(om.silu(gu[:, :F]) * gu[:, F:])
        u = torch.zeros(n, F, dtype=torch.bfloat16, device=dev)
        epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_SWIGLU, y=u.data_ptr(), ldy=F)
        tvp.w12_gemm_ex(_T(to_bits(b), dev),
                        tvp.w12_pack(tvp.w12_encode(_T(lb["wgu"], dev)), tvp.TVP_CHAN_GATEUP, F), epi)
        torch.cuda.synchronize()
        _same_bf16(from_bits(_U(u)), u_r, "swiglu")
        # down + residual
        h2 = round_bf16(h1 + u_r @ w["wdown"].T)
        y = _T(to_bits(h1), dev).clone()
        epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_RESID, y=y.data_ptr(), ldy=H, resid=y.data_ptr(), ldr=H)
        tvp.w12_gemm_ex(_T(to_bits(u_r), dev), tvp.w12_pack(tvp.w12_encode(_T(lb["wdown"], dev))), epi)
        torch.cuda.synchronize()
        _same_bf16(from_bits(_U(y)), h2, "down+resid")
        h = h2
    # final norm + LM head with argmax and logits
    f = round_bf16(om.rmsnorm(h, orc.final_norm, cfg.norm_eps))
    lg_r = f @ orc.lm_head.T
    am = torch.zeros(n, dtype=torch.int32, device=dev)
    lg = torch.zeros(n, cfg.vocab, dtype=torch.float32, device=dev)
    epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_ARGMAX, argmax=am.data_ptr(), logits=lg.data_ptr(), ldl=cfg.vocab)
    tvp.w12_gemm_ex(_T(to_bits(f), dev), tvp.w12_pack(tvp.w12_encode(_T(lm, dev))), epi)
    torch.cuda.synchronize()
    err = row_max_abs_rel(lg.cpu().numpy().astype(np.float64), lg_r)
    print(f"  logits max_abs_rel={err.max():.2e}", flush=True)
    assert err.max() <= 2e-3
    part = np.partition(lg_r, -2, axis=1)
    decidable = (part[:, -1] - part[:, -2]) > 2 * np.abs(lg.cpu().numpy() - lg_r).max(axis=1)
    assert np.array_equal(am.cpu().numpy()[decidable], np.argmax(lg_r, axis=1)[decidable])
