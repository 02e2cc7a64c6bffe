// Host-side checks of libtvp's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code only.  Every call here takes a
// path that returns before any HIP call: status strings, layout queries,
// workspace sizes, the host-side W12 format check, plan creation on a model
// description whose device pointers are never dereferenced, and the argument
// validation of the launching entry points.  Exits non-zero on the first
// mismatch (the sanitizers abort on their own findings).
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "tvp.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static void* fake(size_t i) { return (void*)(uintptr_t)(0x100000 + 0x1000 * i); }

static tvp_w12_packed packed(int64_t n, int64_t k, int32_t map, int32_t a = 0, int32_t b = 0, int32_t c = 0,
                             size_t tag = 0) {
  tvp_w12_packed p;
  std::memset(&p, 0, sizeof p);
  EXPECT(w12_pack_size(n, k, n * k / 97, map, a, b, c, &p) == TVP_OK);
  p.blob = fake(tag);
  return p;
}

int main() {
  for (int s = 0; s <= 8; ++s) EXPECT(tvp_status_string(s) != nullptr);
  EXPECT(std::strcmp(tvp_status_string(TVP_OK), "ok") == 0);

  // layout queries
  tvp_w12_packed p;
  EXPECT(w12_pack_size(1000, 1000, 37, TVP_CHAN_PLAIN, 0, 0, 0, &p) == TVP_OK && p.n_tiles == 32);
  EXPECT(w12_pack_size(100, 70000, 0, TVP_CHAN_PLAIN, 0, 0, 0, &p) == TVP_ERR_SHAPE);
  EXPECT(w12_pack_size(2000, 512, 0, TVP_CHAN_GATEUP, 999, 0, 0, &p) == TVP_ERR_SHAPE);
  EXPECT(w12_pack_size(640, 1000, 0, TVP_CHAN_QKV, 6, 2, 64, &p) == TVP_OK && p.n_tiles == 20);
  EXPECT(w12_pack_size(0, 10, 0, TVP_CHAN_PLAIN, 0, 0, 0, &p) == TVP_ERR_ARG);
  EXPECT(w12_packed_x_elems(65) == 4096 && w12_packed_x_elems(-1) == 0);

  // host-side W12 format check
  {
    const int64_t n = 3, k = 100;
    std::vector<uint8_t> base = {100, 1, 239};
    std::vector<uint32_t> ptr = {0, 2, 2, 5};
    std::vector<uint16_t> idx = {3, 99, 0, 1, 50};
    EXPECT(w12_validate(base.data(), ptr.data(), idx.data(), n, k, 5) == TVP_OK);
    base[1] = 0;
    EXPECT(w12_validate(base.data(), ptr.data(), idx.data(), n, k, 5) == TVP_ERR_FORMAT);
    base[1] = 240;
    EXPECT(w12_validate(base.data(), ptr.data(), idx.data(), n, k, 5) == TVP_ERR_FORMAT);
    base[1] = 1;
    idx[1] = 100;
    EXPECT(w12_validate(base.data(), ptr.data(), idx.data(), n, k, 5) == TVP_ERR_FORMAT);
    idx[1] = 3;
    EXPECT(w12_validate(base.data(), ptr.data(), idx.data(), n, k, 5) == TVP_ERR_FORMAT);
    idx[1] = 99;
    ptr[2] = 6;  // decreasing afterwards, and past n_esc
    EXPECT(w12_validate(base.data(), ptr.data(), idx.data(), n, k, 5) == TVP_ERR_FORMAT);
    ptr[2] = 2;
    EXPECT(w12_validate(base.data(), ptr.data(), idx.data(), n, k, 4) == TVP_ERR_FORMAT);
    EXPECT(w12_validate(base.data(), ptr.data(), nullptr, n, k, 5) == TVP_ERR_ARG);
    EXPECT(w12_validate(base.data(), ptr.data(), idx.data(), -1, k, 5) == TVP_ERR_ARG);
    std::vector<uint32_t> zp = {0};
    EXPECT(w12_validate(nullptr, zp.data(), nullptr, 0, 0, 0) == TVP_OK);
  }

  // GEMM and attention workspace queries at every row count
  tvp_w12_packed gu = packed(2 * 17408, 5120, TVP_CHAN_GATEUP, 17408, 0, 0, 1);
  tvp_w12_packed lm = packed(151936, 5120, TVP_CHAN_PLAIN, 0, 0, 0, 2);
  for (int64_t m = 1; m <= 192; ++m) {
    EXPECT(w12_gemm_workspace(m, &gu) > 0);
    EXPECT(w12_gemm_workspace(m, &lm) > 0);
  }
  EXPECT(w12_gemm_workspace(0, &gu) == 0 && w12_gemm_workspace(193, &gu) == 0);
  for (int32_t n = 1; n <= 64; ++n) EXPECT(tree_attention_workspace(n, 40, 128, 4096 + n) > 0);
  EXPECT(tree_attention_workspace(0, 40, 128, 10) == 0);

  // argument validation of launching entry points (returns before any launch)
  tvp_gemm_epilogue epi;
  std::memset(&epi, 0, sizeof epi);
  epi.mode = TVP_EPI_F32;
  EXPECT(w12_gemm_ex(nullptr, 1, 0, nullptr, &epi, nullptr, 0, nullptr) == TVP_ERR_ARG);
  EXPECT(w12_gemm_ex((const uint16_t*)fake(3), 0, 5120, &gu, &epi, fake(4), 1 << 30, nullptr) == TVP_ERR_SHAPE);
  EXPECT(w12_gemm_ex((const uint16_t*)fake(3), 4, 5120, &gu, &epi, fake(4), 16, nullptr) == TVP_ERR_WORKSPACE);
  epi.mode = 42;
  EXPECT(w12_gemm_ex((const uint16_t*)fake(3), 4, 5120, &gu, &epi, fake(4), size_t(1) << 30, nullptr) ==
         TVP_ERR_ARG);
  EXPECT(w12_pack_x((const uint16_t*)fake(3), 33, 64, 64, (uint16_t*)fake(5), nullptr) == TVP_ERR_SHAPE);
  EXPECT(accept_path(nullptr, nullptr, nullptr, 4, nullptr, nullptr, nullptr, nullptr, nullptr) == TVP_ERR_ARG);
  EXPECT(accept_path((const int32_t*)fake(1), (const int32_t*)fake(2), (const int32_t*)fake(3), 1025,
                     (int32_t*)fake(4), (int32_t*)fake(5), (int32_t*)fake(6), (int32_t*)fake(7), nullptr) ==
         TVP_ERR_SHAPE);
  EXPECT(tree_attention((const uint16_t*)fake(1), (const uint16_t*)fake(2), (const uint16_t*)fake(3), 100, 90,
                        (const int32_t*)fake(4), 11, 8, 2, 128, (uint16_t*)fake(5), (int32_t*)fake(6), fake(7),
                        size_t(1) << 30, nullptr) == TVP_ERR_CAPACITY);
  EXPECT(tree_attention((const uint16_t*)fake(1), (const uint16_t*)fake(2), (const uint16_t*)fake(3), 100, 10,
                        (const int32_t*)fake(4), 11, 8, 2, 96, (uint16_t*)fake(5), (int32_t*)fake(6), fake(7),
                        size_t(1) << 30, nullptr) == TVP_ERR_SHAPE);
  EXPECT(tvp_read_probe(nullptr, 64, nullptr, nullptr) == TVP_ERR_ARG);

  // plan creation on a 27B-like description (device pointers never dereferenced)
  const int L = 64, H = 5120, hq = 40, hkv = 8, d = 128, F = 17408, V = 151936;
  std::vector<tvp_layer> layers(L);
  for (int l = 0; l < L; ++l) {
    tvp_layer& y = layers[l];
    std::memset(&y, 0, sizeof y);
    y.wqkv = packed((int64_t)(hq + 2 * hkv) * d, H, TVP_CHAN_QKV, hq, hkv, d, 10 + 8 * l);
    y.wo = packed(H, (int64_t)hq * d, TVP_CHAN_PLAIN, 0, 0, 0, 11 + 8 * l);
    y.wgu = packed(2LL * F, H, TVP_CHAN_GATEUP, F, 0, 0, 12 + 8 * l);
    y.wdown = packed(H, F, TVP_CHAN_PLAIN, 0, 0, 0, 13 + 8 * l);
    y.attn_norm = (const uint16_t*)fake(14 + 8 * l);
    y.ffn_norm = (const uint16_t*)fake(15 + 8 * l);
    y.k_cache = (uint16_t*)fake(16 + 8 * l);
    y.v_cache = (uint16_t*)fake(17 + 8 * l);
  }
  tvp_model_desc md;
  std::memset(&md, 0, sizeof md);
  md.n_layers = L;
  md.hidden = H;
  md.n_heads = hq;
  md.n_kv_heads = hkv;
  md.head_dim = d;
  md.ffn = F;
  md.vocab = V;
  md.rope_theta = 1e6f;
  md.norm_eps = 1e-6f;
  md.s_max = 4096 + 64;
  md.embed = (const uint16_t*)fake(5000);
  md.final_norm = (const uint16_t*)fake(5001);
  md.lm_head = packed(V, H, TVP_CHAN_PLAIN, 0, 0, 0, 5002);
  md.layers = layers.data();
  tvp_plan* plan = nullptr;
  EXPECT(tvp_plan_create(&md, 193, &plan) == TVP_ERR_CAPACITY && plan == nullptr);
  layers[3].wgu.map_a = F - 1;
  EXPECT(tvp_plan_create(&md, 32, &plan) == TVP_ERR_FORMAT);
  layers[3].wgu.map_a = F;
  md.head_dim = 96;
  EXPECT(tvp_plan_create(&md, 32, &plan) == TVP_ERR_SHAPE);
  md.head_dim = d;
  EXPECT(tvp_plan_create(&md, 32, &plan) == TVP_OK && plan != nullptr);
  const size_t ws = verify_step_workspace(plan);
  EXPECT(ws > 0);
  tvp_verify_out out;
  std::memset(&out, 0, sizeof out);
  out.argmax = (int32_t*)fake(6000);
  out.path = (int32_t*)fake(6001);
  out.n_accepted = (int32_t*)fake(6002);
  out.bonus = (int32_t*)fake(6003);
  out.status = (int32_t*)fake(6004);
  const int32_t* tok = (const int32_t*)fake(6005);
  const int32_t* par = (const int32_t*)fake(6006);
  EXPECT(verify_step(plan, 4096, tok, par, 33, 1, &out, fake(6007), ws, nullptr) == TVP_ERR_CAPACITY);
  EXPECT(verify_step(plan, 4096 + 40, tok, par, 32, 1, &out, fake(6007), ws, nullptr) == TVP_ERR_CAPACITY);
  EXPECT(verify_step(plan, 4096, tok, par, 32, 1, &out, fake(6007), ws - 1, nullptr) == TVP_ERR_WORKSPACE);
  EXPECT(verify_step(plan, -1, tok, par, 32, 1, &out, fake(6007), ws, nullptr) == TVP_ERR_SHAPE);
  {
    std::vector<int32_t> ctx = {100, 200}, np = {0, 20, 40};
    EXPECT(verify_step_batched(plan, 2, ctx.data(), np.data(), 2080, tok, par, 1, &out, fake(6007), ws,
                               nullptr) == TVP_ERR_CAPACITY);  // 40 nodes > 32
    np = {0, 10, 20};
    EXPECT(verify_step_batched(plan, 2, ctx.data(), np.data(), 150, tok, par, 1, &out, fake(6007), ws,
                               nullptr) == TVP_ERR_CAPACITY);  // 200 + 10 > s_req
    np = {1, 10, 20};
    EXPECT(verify_step_batched(plan, 2, ctx.data(), np.data(), 2080, tok, par, 1, &out, fake(6007), ws,
                               nullptr) == TVP_ERR_SHAPE);
  }
  tvp_plan_destroy(plan);
  tvp_plan_destroy(nullptr);
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi host checks passed\n");
  return 0;
}
