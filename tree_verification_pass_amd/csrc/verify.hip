// The verification pass: embedding gather, RMSNorm, the per-layer sequence of
// fused W12 GEMMs and tree attention, the LM-head argmax, the acceptance walk
// and the KV commit, for one request or a batch sharing one node budget.
//
// SpecPilot summary (onedev.kr): section 무엇인가 -- the target processes every
// draft token in one forward pass and most of a step is spent reading the
// target's weights; section 무엇과 다른가 -- the pass returns the matched path
// plus a bonus token, and a batch can share one node budget across requests.
// The KV commit is the dense-model counterpart of the page's commit kernel
// (which replays the accepted path into recurrent layers): the accepted
// nodes' keys and values are moved to the committed slots.
#include <math.h>

#include <algorithm>
#include <vector>

#include "internal.h"

namespace tvp {

constexpr int kMaxLayers = 120;

constexpr int kKsplitMax = 16;  // most K slices of the O and down projections (packed path)

// ------------------------------------------------------------ small kernels

__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tokens,
                                                    const uint16_t* __restrict__ embed, int hidden,
                                                    int vocab, uint16_t* __restrict__ h, int ldh,
                                                    int32_t* __restrict__ bad) {
  const int i = blockIdx.x;
  const int32_t t = tokens[i];
  const bool ok = t >= 0 && t < vocab;
  if (threadIdx.x == 0) bad[i] = ok ? 0 : 1;
  const uint16_t* src = embed + (int64_t)(ok ? t : 0) * hidden;
  uint16_t* dst = h + (int64_t)i * ldh;
  if (((uintptr_t)embed % 16) == 0 && hidden % 8 == 0 && ldh % 8 == 0) {  // 16-byte pieces
    for (int c = threadIdx.x; c < hidden / 8; c += 256) ((uint4*)dst)[c] = ((const uint4*)src)[c];
  } else {
    for (int k = threadIdx.x; k < hidden; k += 256) dst[k] = src[k];
  }
}

// Residual update fused with the next RMSNorm, one workgroup per row:
//   h <- bf16(h + (P[0] + P[1] + ... + P[S-1]))   (K-slice partial sums of the
//        preceding projection, added in slice order; nothing when S == 0)
//   y <- bf16(h * (mean(h^2) + eps)^-1/2 * g)       (fp32, fixed reduction order)
// y is the next GEMM's input, row-major or (packed != 0, at most 32 rows) in
// the packed activation layout.  1024 threads: a row of up to 8192 values is
// one 8-element chunk per thread, so every load of the row (h, the slices,
// the gains) is issued before the first is used and the kernel costs about
// one memory round trip.  Longer rows loop; rows whose length or pitches are
// not multiples of 8 go element by element.
constexpr int kNormThreads = 1024;

__global__ __launch_bounds__(kNormThreads) void resid_norm_kernel(const float* __restrict__ P, int S,
                                                                  int64_t pstride, int ldp,
                                                                  uint16_t* __restrict__ h, int ldh,
                                                                  const uint16_t* __restrict__ g, int hidden,
                                                                  float eps, uint16_t* __restrict__ y, int ldy,
                                                                  int packed) {
  constexpr int NT = kNormThreads;
  __shared__ float ws[NT / 64];
  const int i = blockIdx.x, tid = threadIdx.x;
  uint16_t* hr = h + (int64_t)i * ldh;
  const float* pr = P + (int64_t)i * ldp;
  uint16_t* yr = y + (int64_t)i * ldy;
  const bool vec = (hidden % 8) == 0 && (ldh % 8) == 0 && (S == 0 || (ldp % 4) == 0) && (packed || (ldy % 8) == 0);
  float ss = 0.0f;
  // pass 1 on chunk c: residual update (written back) and sum of squares
  auto pass1 = [&](int c, uint32_t (&w)[4]) {
    const uint4 v = *(const uint4*)(hr + 8 * c);
    w[0] = v.x, w[1] = v.y, w[2] = v.z, w[3] = v.w;
    if (S > 0) {
      float acc[8];
      // up to 8 slices per round: all their loads (16 in flight) are issued
      // before the first add, also when fewer than 8 remain; added in slice order
      for (int sl = 0; sl < S; sl += 8) {
        const int cnt = min(8, S - sl);
        float4 q0[8], q1[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (j < cnt) {
            q0[j] = *(const float4*)(pr + (sl + j) * pstride + 8 * c);
            q1[j] = *(const float4*)(pr + (sl + j) * pstride + 8 * c + 4);
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (j < cnt) {
            const float pv[8] = {q0[j].x, q0[j].y, q0[j].z, q0[j].w, q1[j].x, q1[j].y, q1[j].z, q1[j].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = (sl + j) == 0 ? pv[e] : acc[e] + pv[e];
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = f32_to_bf16(bf16_to_f32(w[e] & 0xFFFFu) + acc[2 * e]);
        const uint32_t hi = f32_to_bf16(bf16_to_f32(w[e] >> 16) + acc[2 * e + 1]);
        w[e] = lo | (hi << 16);
      }
      *(uint4*)(hr + 8 * c) = make_uint4(w[0], w[1], w[2], w[3]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a0 = bf16_to_f32(w[e] & 0xFFFFu), a1 = bf16_to_f32(w[e] >> 16);
      ss += a0 * a0 + a1 * a1;
    }
  };
  const int nc = vec ? hidden / 8 : 0;
  uint32_t keep[4] = {0, 0, 0, 0};
  uint4 gkeep = make_uint4(0, 0, 0, 0);
  if (vec) {
    if (tid < nc) {
      gkeep = *(const uint4*)(g + 8 * tid);  // the gains of pass 2, fetched with everything else
      pass1(tid, keep);
    }
    for (int c = tid + NT; c < nc; c += NT) {
      uint32_t w[4];
      pass1(c, w);
    }
  } else {
    for (int k = tid; k < hidden; k += NT) {
      float v = bf16_to_f32(hr[k]);
      if (S > 0) {
        float acc = 0.0f;
        for (int sl = 0; sl < S; ++sl) acc = sl == 0 ? pr[sl * pstride + k] : acc + pr[sl * pstride + k];
        const uint32_t hb = f32_to_bf16(v + acc);
        hr[k] = (uint16_t)hb;
        v = bf16_to_f32(hb);
      }
      ss += v * v;
    }
  }
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((tid & 63) == 0) ws[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < NT / 64; w += 2) tot += ws[w] + ws[w + 1];
  const float r = 1.0f / sqrtf(tot / (float)hidden + eps);
  // pass 2 on chunk c (w: its updated values, gv: its gains)
  auto pass2 = [&](int c, const uint32_t (&w)[4], const uint4& gv) {
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = f32_to_bf16(bf16_to_f32(w[e] & 0xFFFFu) * r * bf16_to_f32(gw[e] & 0xFFFFu));
      const uint32_t hi = f32_to_bf16(bf16_to_f32(w[e] >> 16) * r * bf16_to_f32(gw[e] >> 16));
      o[e] = lo | (hi << 16);
    }
    *(uint4*)(packed ? y + xpack_index(i, 8 * c) : yr + 8 * c) = make_uint4(o[0], o[1], o[2], o[3]);
  };
  if (vec) {
    if (tid < nc) pass2(tid, keep, gkeep);
    for (int c = tid + NT; c < nc; c += NT) {  // re-read this thread's own pass-1 result
      const uint4 v = *(const uint4*)(hr + 8 * c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      pass2(c, w, *(const uint4*)(g + 8 * c));
    }
  } else {
    for (int k = tid; k < hidden; k += NT)
      (packed ? y[xpack_index(i, k)] : yr[k]) = (uint16_t)f32_to_bf16(bf16_to_f32(hr[k]) * r * bf16_to_f32(g[k]));
  }
}

// RMSNorm alone (no residual update): S = 0 of the fused kernel.
static void launch_norm(const float* P, int S, int64_t pstride, int ldp, uint16_t* h, int ldh, const uint16_t* g,
                        int hidden, float eps, uint16_t* y, int ldy, int packed, int rows, hipStream_t stream) {
  resid_norm_kernel<<<dim3(rows), dim3(kNormThreads), 0, stream>>>(P, S, pstride, ldp, h, ldh, g, hidden, eps, y,
                                                                   ldy, packed);
}

// One workgroup per request: its 64 threads stage the request's parents,
// tokens and greedy tokens in LDS and validate the tree, then one thread
// walks the nodes in order (parents[i] < i) from LDS.
__global__ __launch_bounds__(64) void accept_kernel(const int32_t* __restrict__ argmax,
                                                    const int32_t* __restrict__ tokens,
                                                    const int32_t* __restrict__ parents, ReqInfo ri,
                                                    const int32_t* __restrict__ bad_token,
                                                    int32_t* __restrict__ path, int32_t* __restrict__ n_acc,
                                                    int32_t* __restrict__ bonus, int32_t* __restrict__ status) {
  __shared__ int32_t par[1024], tok[1024], am[1024], depth[1024];
  __shared__ uint8_t okf[1024];
  __shared__ int bad_tree, bad_tok;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int nb = ri.node_ptr[r], n = ri.node_ptr[r + 1] - nb;
  const bool sized = n >= 1 && n <= 1024;
  if (tid == 0) {
    bad_tree = sized ? 0 : 1;
    bad_tok = 0;
  }
  __syncthreads();
  if (sized) {
    for (int i = tid; i < n; i += 64) {
      const int p = parents[nb + i];
      par[i] = p;
      tok[i] = tokens[nb + i];
      am[i] = argmax[nb + i];
      if (i == 0 ? p != -1 : (p < 0 || p >= i)) atomicOr(&bad_tree, 1);
      if (bad_token && bad_token[nb + i]) atomicOr(&bad_tok, 1);
    }
  }
  __syncthreads();
  if (tid != 0) return;
  const int st = bad_tree ? TVP_ERR_TREE : (bad_tok ? TVP_ERR_ARG : TVP_OK);
  if (st != TVP_OK) {
    status[r] = st;
    n_acc[r] = 0;
    if (n >= 1) {
      path[nb] = 0;
      bonus[r] = argmax[nb];
    } else {
      bonus[r] = -1;
    }
    return;
  }
  depth[0] = 0;
  okf[0] = 1;
  int best = 0;
  for (int i = 1; i < n; ++i) {
    const int p = par[i];
    depth[i] = depth[p] + 1;
    okf[i] = okf[p] && tok[i] == am[p];
    if (okf[i] && depth[i] > depth[best]) best = i;
  }
  const int a = depth[best];
  int v = best;
  for (int j = a; j >= 0; --j) {
    path[nb + j] = v;
    v = j > 0 ? par[v] : 0;
  }
  n_acc[r] = a;
  bonus[r] = am[best];
  status[r] = TVP_OK;
}

struct CacheTable {
  int n_layers;
  uint16_t* kc[kMaxLayers];
  uint16_t* vc[kMaxLayers];
};

// Moves accepted rows: slot base + L + j <- slot base + L + path[j], j = 1..a,
// for every layer, K and V, kv head.  Reads every source row of a kv head
// before writing any (sources and destinations may overlap).
__global__ __launch_bounds__(256) void kv_commit_kernel(CacheTable ct, ReqInfo ri, int32_t s_req,
                                                        int64_t s_stride, int hkv, int d,
                                                        const int32_t* __restrict__ path,
                                                        const int32_t* __restrict__ n_acc,
                                                        const int32_t* __restrict__ status) {
  constexpr int kBufVec = 1024;  // 16 KB of 16-byte pieces
  __shared__ uint4 buf[kBufVec];
  __shared__ int32_t src[64];     // source slot offset of accepted row j (<= 63 rows)
  const int r = blockIdx.x;
  const int layer = blockIdx.y >> 1, which = blockIdx.y & 1;
  if (status[r] != TVP_OK) return;
  const int a = n_acc[r];
  if (a <= 0) return;
  const int nb = ri.node_ptr[r];
  const int64_t base = (int64_t)r * s_req + ri.ctx_len[r];
  uint16_t* cache = which ? ct.vc[layer] : ct.kc[layer];
  for (int j = threadIdx.x; j <= a; j += 256) src[j] = path[nb + j];
  __syncthreads();
  // Rows j = 1..a of as many heads as the buffer holds per round, in 16-byte
  // pieces: every source row of the round is read before any is written
  // (source and destination slots overlap).
  const int vrow = d / 8, per_head = a * vrow;
  const int hpr = max(1, min(hkv, kBufVec / per_head));
  for (int h0 = 0; h0 < hkv; h0 += hpr) {
    const int nv = min(hpr, hkv - h0) * per_head;
    for (int e = threadIdx.x; e < nv; e += 256) {
      const int hh = e / per_head, rem = e % per_head, j = 1 + rem / vrow, c = rem % vrow;
      const uint4* hc = (const uint4*)(cache + (int64_t)(h0 + hh) * s_stride * d);
      buf[e] = hc[(base + src[j]) * vrow + c];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < nv; e += 256) {
      const int hh = e / per_head, rem = e % per_head, j = 1 + rem / vrow, c = rem % vrow;
      uint4* hc = (uint4*)(cache + (int64_t)(h0 + hh) * s_stride * d);
      hc[(base + j) * vrow + c] = buf[e];
    }
    __syncthreads();
  }
}

}  // namespace tvp

using namespace tvp;

struct tvp_plan {
  tvp_model_desc desc;
  std::vector<tvp_layer> layers;
  int32_t max_nodes;
  int ld_h, ld_q, ld_u;
  bool pack_ok;  // every GEMM takes the skinny path at <= 32 rows
  // workspace layout
  size_t off_h, off_a, off_q, off_o, off_u;
  size_t off_anc, off_pos, off_slot, off_tstat, off_bad, off_rope;
  size_t off_gscr, gscr_bytes;
  size_t off_part;  // K-slice partial sums of the O and down projections (packed path)
  int ks_o, ks_down;  // their K slices at 32 rows
  size_t off_ascr, ascr_bytes;
  size_t off_cnt;  // arrival counters: the GEMMs' (kGemmRemCounters), then the attention's
  int n_cnt;
  size_t bytes;
};

static int check_packed(const tvp_w12_packed& w, int64_t n_out, int64_t k_in, int32_t map) {
  if (!w.blob || w.n_out != n_out || w.k_in != k_in || w.chan_map != map) return TVP_ERR_FORMAT;
  return TVP_OK;
}

extern "C" {

int tvp_plan_create(const tvp_model_desc* d, int32_t max_nodes, tvp_plan** out) {
  if (!d || !out || !d->layers || !d->embed || !d->final_norm) return TVP_ERR_ARG;
  *out = nullptr;
  if (d->n_layers < 1 || d->n_layers > kMaxLayers || d->hidden < 1 || d->n_heads < 1 || d->n_kv_heads < 1 ||
      d->n_heads % d->n_kv_heads || (d->head_dim != 64 && d->head_dim != 128) || d->ffn < 1 || d->vocab < 1 ||
      d->s_max < 1 || !(d->rope_theta > 0) || !(d->norm_eps >= 0))
    return TVP_ERR_SHAPE;
  if (d->hidden > 65536 || d->ffn > 65536 || d->n_heads * d->head_dim > 65536) return TVP_ERR_SHAPE;
  if (max_nodes < 1 || max_nodes > 192) return TVP_ERR_CAPACITY;
  const int hq = d->n_heads, hkv = d->n_kv_heads, hd = d->head_dim, H = d->hidden, F = d->ffn;
  const int G = hq / hkv;
  if (G > 256) return TVP_ERR_SHAPE;  // a one-node request must fit the attention's 256 rows
  if ((uintptr_t)d->final_norm % 16) return TVP_ERR_ARG;
  int st = check_packed(d->lm_head, d->vocab, H, TVP_CHAN_PLAIN);
  if (st) return st;
  for (int l = 0; l < d->n_layers; ++l) {
    const tvp_layer& L = d->layers[l];
    if (!L.attn_norm || !L.ffn_norm || !L.k_cache || !L.v_cache) return TVP_ERR_ARG;
    if ((st = check_packed(L.wqkv, (int64_t)(hq + 2 * hkv) * hd, H, TVP_CHAN_QKV))) return st;
    if (L.wqkv.map_a != hq || L.wqkv.map_b != hkv || L.wqkv.map_c != hd) return TVP_ERR_FORMAT;
    if ((st = check_packed(L.wo, H, (int64_t)hq * hd, TVP_CHAN_PLAIN))) return st;
    if ((st = check_packed(L.wgu, 2LL * F, H, TVP_CHAN_GATEUP))) return st;
    if (L.wgu.map_a != F) return TVP_ERR_FORMAT;
    if ((st = check_packed(L.wdown, H, F, TVP_CHAN_PLAIN))) return st;
    if (((uintptr_t)L.k_cache | (uintptr_t)L.v_cache | (uintptr_t)L.attn_norm | (uintptr_t)L.ffn_norm) % 16)
      return TVP_ERR_ARG;
  }
  tvp_plan* p = new (std::nothrow) tvp_plan();
  if (!p) return TVP_ERR_ARG;
  p->desc = *d;
  p->layers.assign(d->layers, d->layers + d->n_layers);
  p->desc.layers = nullptr;
  p->max_nodes = max_nodes;
  p->ld_h = (int)align_up(H, 8);
  p->ld_q = (int)align_up((size_t)hq * hd, 8);
  p->ld_u = (int)align_up(F, 8);
  const int mn = max_nodes;
  // scratch over every GEMM at every row count up to max_nodes
  int gmax = 1;
  size_t gscr = 256;
  auto need = [&](const tvp_w12_packed& w, bool sliced) {
    for (int m = 1; m <= max_nodes; ++m) {
      int g;
      size_t b;
      gemm_requirements(m, &w, &g, &b);
      gmax = std::max(gmax, g);
      gscr = std::max(gscr, b);
      if (sliced && m <= 32) {  // the O and down projections' K-sliced launches
        gemm_requirements(m, &w, &g, &b, kKsplitMax);
        gmax = std::max(gmax, g);
        gscr = std::max(gscr, b);
      }
    }
  };
  need(d->lm_head, false);
  p->pack_ok = gemm_is_skinny(32, &d->lm_head);
  for (int l = 0; l < d->n_layers; ++l) {
    need(p->layers[l].wqkv, false);
    need(p->layers[l].wo, true);
    need(p->layers[l].wgu, false);
    need(p->layers[l].wdown, true);
    p->pack_ok = p->pack_ok && gemm_is_skinny(32, &p->layers[l].wqkv) && gemm_is_skinny(32, &p->layers[l].wo) &&
                 gemm_is_skinny(32, &p->layers[l].wgu) && gemm_is_skinny(32, &p->layers[l].wdown);
  }
  // activation buffers hold either layout: row-major [mn][ld] or packed
  auto act_bytes = [&](int ld, int64_t k) {
    return std::max((size_t)mn * ld * 2, (size_t)xpack_elems(k) * 2);
  };
  size_t off = 0;
  p->off_h = off;
  off = align_up(off + (size_t)mn * p->ld_h * 2, 256);
  p->off_a = off;
  off = align_up(off + act_bytes(p->ld_h, H), 256);
  p->off_q = off;
  off = align_up(off + (size_t)mn * p->ld_q * 2, 256);
  p->off_o = off;
  off = align_up(off + act_bytes(p->ld_q, (int64_t)hq * hd), 256);
  p->off_u = off;
  off = align_up(off + act_bytes(p->ld_u, F), 256);
  p->off_anc = off;
  off = align_up(off + (size_t)mn * 8, 256);
  p->off_pos = off;
  off = align_up(off + (size_t)mn * 4, 256);
  p->off_slot = off;
  off = align_up(off + (size_t)mn * 4, 256);
  p->off_tstat = off;
  off = align_up(off + (size_t)kMaxReq * 4, 256);
  p->off_bad = off;
  off = align_up(off + (size_t)mn * 4, 256);
  p->off_rope = off;  // (cos, sin) per node and rotated dim, shared by every layer's QKV epilogue
  off = align_up(off + (size_t)mn * (hd / 2) * 8, 256);
  // O and down projections in the packed path: K split over workgroups, the
  // slices' partial sums reduced by the fused residual + RMSNorm kernel
  p->ks_o = 1;
  p->ks_down = 1;
  if (p->pack_ok) {  // the largest slice counts any layer uses (they size the partial buffer)
    for (int l = 0; l < d->n_layers; ++l) {
      p->ks_o = std::max(p->ks_o, gemm_ksplits(32, &p->layers[l].wo, kKsplitMax));
      p->ks_down = std::max(p->ks_down, gemm_ksplits(32, &p->layers[l].wdown, kKsplitMax));
    }
  }
  p->off_part = off;
  off = align_up(off + (size_t)std::max(p->ks_o, p->ks_down) * 32 * H * 4, 256);
  p->off_gscr = off;
  p->gscr_bytes = gscr;
  off = align_up(off + gscr, 256);
  p->off_ascr = off;
  // the attention's split count depends on the largest request's rows, so
  // the scratch covers every per-request node count a pass may bring
  p->ascr_bytes = 0;
  for (int nr = 1; nr <= std::min(mn, 64) && G * nr <= 256; ++nr)
    p->ascr_bytes = std::max(p->ascr_bytes, attention_scratch_bytes(hkv, G, hd, G * nr, mn, d->s_max));
  off = align_up(off + p->ascr_bytes, 256);
  p->off_cnt = off;
  p->n_cnt = kGemmRemCounters + attention_counters(std::min(mn, kMaxReq), hkv);
  off = align_up(off + (size_t)p->n_cnt * 4, 256);
  p->bytes = off;
  *out = p;
  return TVP_OK;
}

void tvp_plan_destroy(tvp_plan* p) { delete p; }

size_t verify_step_workspace(const tvp_plan* p) { return p ? p->bytes : 0; }

}  // extern "C"

// Runs the whole pass for the requests described by `ri`.
static int run_pass(tvp_plan* p, const ReqInfo& ri, int32_t s_req, const int32_t* tokens,
                    const int32_t* parents, int32_t commit, const tvp_verify_out* out, void* ws,
                    hipStream_t stream) {
  const tvp_model_desc& d = p->desc;
  const int hq = d.n_heads, hkv = d.n_kv_heads, hd = d.head_dim, H = d.hidden, F = d.ffn;
  const int G = hq / hkv;
  const int n_total = ri.node_ptr[ri.n_req];
  // up to 32 nodes: GEMM inputs (a, o, u) are produced in the packed layout
  const int pk = (n_total <= 32 && p->pack_ok) ? 1 : 0;
  int max_n = 0, max_keys = 0;
  for (int r = 0; r < ri.n_req; ++r) {
    const int n = ri.node_ptr[r + 1] - ri.node_ptr[r];
    max_n = std::max(max_n, n);
    max_keys = std::max(max_keys, ri.ctx_len[r] + n);
  }
  uint8_t* w = (uint8_t*)ws;
  uint16_t* h = (uint16_t*)(w + p->off_h);
  uint16_t* a = (uint16_t*)(w + p->off_a);
  uint16_t* q = (uint16_t*)(w + p->off_q);
  uint16_t* o = (uint16_t*)(w + p->off_o);
  uint16_t* u = (uint16_t*)(w + p->off_u);
  uint64_t* anc = (uint64_t*)(w + p->off_anc);
  int32_t* pos = (int32_t*)(w + p->off_pos);
  int32_t* slot = (int32_t*)(w + p->off_slot);
  int32_t* tstat = (int32_t*)(w + p->off_tstat);
  int32_t* bad = (int32_t*)(w + p->off_bad);
  void* gscr = w + p->off_gscr;
  void* ascr = w + p->off_ascr;
  uint32_t* gcnt = (uint32_t*)(w + p->off_cnt);  // GEMM arrival counters
  uint32_t* acnt = gcnt + kGemmRemCounters;       // attention arrival counters
  int st;

  if ((st = launch_tree_prep(parents, ri, s_req, anc, pos, slot, tstat, gcnt, p->n_cnt, stream))) return st;
  float* rope = (float*)(w + p->off_rope);
  if ((st = launch_rope_table(pos, n_total, hd, d.rope_theta, rope, stream))) return st;
  embed_kernel<<<dim3(n_total), dim3(256), 0, stream>>>(tokens, d.embed, H, d.vocab, h, p->ld_h, bad);
  TVP_LAUNCH_CHECK();
  float* part = (float*)(w + p->off_part);
  const int64_t pstride = (int64_t)n_total * H;  // one K slice of partial sums [n_total][H]
  // the first layer's attention norm; later norms are fused with the residual update
  launch_norm(part, 0, pstride, H, h, p->ld_h, p->layers[0].attn_norm, H, d.norm_eps, a, p->ld_h, pk, n_total,
              stream);
  TVP_LAUNCH_CHECK();
  for (int l = 0; l < d.n_layers; ++l) {
    const tvp_layer& L = p->layers[l];
    const uint16_t* next_norm = l + 1 < d.n_layers ? p->layers[l + 1].attn_norm : d.final_norm;
    tvp_gemm_epilogue e{};
    e.mode = TVP_EPI_QKV;
    e.y = q;
    e.ldy = p->ld_q;
    e.pos = pos;
    e.slot = slot;
    e.k_cache = L.k_cache;
    e.v_cache = L.v_cache;
    e.s_stride = d.s_max;
    e.rope_theta = d.rope_theta;
    e.counters = gcnt;
    if ((st = gemm_run(a, pk ? a : nullptr, n_total, p->ld_h, &L.wqkv, &e, 0, gscr, p->gscr_bytes,
                       stream, 1, rope)))
      return st;
    if ((st = launch_tree_attention(q, L.k_cache, L.v_cache, d.s_max, ri, s_req, anc, hq, hkv, hd, G * max_n,
                                    max_keys, o, pk, ascr, p->ascr_bytes, acnt, stream)))
      return st;
    // O projection + residual, then the FFN norm
    e = tvp_gemm_epilogue{};
    if (pk) {
      e.mode = kEpiPartial;
      e.y = part;
      e.ldy = H;
      if ((st = gemm_run(o, o, n_total, p->ld_q, &L.wo, &e, 0, gscr, p->gscr_bytes, stream,
                         kKsplitMax)))
        return st;
      launch_norm(part, gemm_ksplits(n_total, &L.wo, kKsplitMax), pstride, H, h, p->ld_h, L.ffn_norm, H,
                  d.norm_eps, a, p->ld_h, 1, n_total, stream);
    } else {  // wide kernel: its split sums stay in the GEMM scratch and the norm adds them in split order
      e.mode = kEpiPartial;
      if ((st = gemm_run(o, nullptr, n_total, p->ld_q, &L.wo, &e, 0, gscr, p->gscr_bytes, stream)))
        return st;
      const int ldp = L.wo.n_tiles * 32;
      launch_norm((const float*)gscr, gemm_ksplits(n_total, &L.wo, 1), (int64_t)n_total * ldp, ldp, h, p->ld_h,
                  L.ffn_norm, H, d.norm_eps, a, p->ld_h, 0, n_total, stream);
    }
    TVP_LAUNCH_CHECK();
    e = tvp_gemm_epilogue{};
    e.mode = TVP_EPI_SWIGLU;
    e.y = u;
    e.ldy = p->ld_u;
    e.counters = gcnt;
    if ((st = gemm_run(a, pk ? a : nullptr, n_total, p->ld_h, &L.wgu, &e, pk, gscr, p->gscr_bytes,
                       stream)))
      return st;
    // down projection + residual, then the next layer's attention norm (or the final norm)
    e = tvp_gemm_epilogue{};
    if (pk) {
      e.mode = kEpiPartial;
      e.y = part;
      e.ldy = H;
      if ((st = gemm_run(u, u, n_total, p->ld_u, &L.wdown, &e, 0, gscr, p->gscr_bytes, stream,
                         kKsplitMax)))
        return st;
      launch_norm(part, gemm_ksplits(n_total, &L.wdown, kKsplitMax), pstride, H, h, p->ld_h, next_norm, H,
                  d.norm_eps, a, p->ld_h, 1, n_total, stream);
    } else {
      e.mode = kEpiPartial;
      if ((st = gemm_run(u, nullptr, n_total, p->ld_u, &L.wdown, &e, 0, gscr, p->gscr_bytes, stream)))
        return st;
      const int ldp = L.wdown.n_tiles * 32;
      launch_norm((const float*)gscr, gemm_ksplits(n_total, &L.wdown, 1), (int64_t)n_total * ldp, ldp, h,
                  p->ld_h, next_norm, H, d.norm_eps, a, p->ld_h, 0, n_total, stream);
    }
    TVP_LAUNCH_CHECK();
  }
  tvp_gemm_epilogue e{};
  e.mode = TVP_EPI_ARGMAX;
  e.argmax = out->argmax;
  e.logits = out->logits;
  e.ldl = d.vocab;
  if ((st = gemm_run(a, pk ? a : nullptr, n_total, p->ld_h, &d.lm_head, &e, 0, gscr, p->gscr_bytes,
                     stream)))
    return st;
  accept_kernel<<<dim3(ri.n_req), dim3(64), 0, stream>>>(out->argmax, tokens, parents, ri, bad, out->path,
                                                         out->n_accepted, out->bonus, out->status);
  TVP_LAUNCH_CHECK();
  if (commit) {
    CacheTable ct{};
    ct.n_layers = d.n_layers;
    for (int l = 0; l < d.n_layers; ++l) {
      ct.kc[l] = p->layers[l].k_cache;
      ct.vc[l] = p->layers[l].v_cache;
    }
    kv_commit_kernel<<<dim3(ri.n_req, 2 * d.n_layers), dim3(256), 0, stream>>>(
        ct, ri, s_req, d.s_max, hkv, hd, out->path, out->n_accepted, out->status);
    TVP_LAUNCH_CHECK();
  }
  (void)tstat;
  return TVP_OK;
}

extern "C" {

int verify_step(tvp_plan* p, int32_t ctx_len, const int32_t* tokens, const int32_t* parents, int32_t n,
                int32_t commit, const tvp_verify_out* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!p || !tokens || !parents || !out) return TVP_ERR_ARG;
  if (!out->argmax || !out->path || !out->n_accepted || !out->bonus || !out->status) return TVP_ERR_ARG;
  if (n < 1 || ctx_len < 0) return TVP_ERR_SHAPE;
  if (n > p->max_nodes || n > 64) return TVP_ERR_CAPACITY;
  if ((int64_t)ctx_len + n > p->desc.s_max) return TVP_ERR_CAPACITY;
  if ((p->desc.n_heads / p->desc.n_kv_heads) * n > 256) return TVP_ERR_SHAPE;  // attention rows per kv head
  if (!ws || ws_bytes < p->bytes) return TVP_ERR_WORKSPACE;
  ReqInfo ri{};
  ri.n_req = 1;
  ri.ctx_len[0] = ctx_len;
  ri.node_ptr[0] = 0;
  ri.node_ptr[1] = n;
  return run_pass(p, ri, 0, tokens, parents, commit, out, ws, stream);
}

int verify_step_batched(tvp_plan* p, int32_t n_req, const int32_t* ctx_len, const int32_t* node_ptr,
                        int32_t s_req, const int32_t* tokens, const int32_t* parents, int32_t commit,
                        const tvp_verify_out* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!p || !ctx_len || !node_ptr || !tokens || !parents || !out) return TVP_ERR_ARG;
  if (!out->argmax || !out->path || !out->n_accepted || !out->bonus || !out->status) return TVP_ERR_ARG;
  if (n_req < 1 || n_req > kMaxReq || s_req < 1) return TVP_ERR_SHAPE;
  if ((int64_t)n_req * s_req > p->desc.s_max) return TVP_ERR_CAPACITY;
  if (node_ptr[0] != 0) return TVP_ERR_SHAPE;
  ReqInfo ri{};
  ri.n_req = n_req;
  for (int r = 0; r < n_req; ++r) {
    const int n = node_ptr[r + 1] - node_ptr[r];
    if (n < 1 || ctx_len[r] < 0) return TVP_ERR_SHAPE;
    if (n > 64 || (int64_t)ctx_len[r] + n > s_req) return TVP_ERR_CAPACITY;
    if ((p->desc.n_heads / p->desc.n_kv_heads) * n > 256) return TVP_ERR_SHAPE;
    ri.ctx_len[r] = ctx_len[r];
    ri.node_ptr[r] = node_ptr[r];
  }
  ri.node_ptr[n_req] = node_ptr[n_req];
  if (node_ptr[n_req] > p->max_nodes) return TVP_ERR_CAPACITY;
  if (!ws || ws_bytes < p->bytes) return TVP_ERR_WORKSPACE;
  return run_pass(p, ri, s_req, tokens, parents, commit, out, ws, stream);
}

static size_t resid_norm_ws_layout(int64_t m, const tvp_w12_packed* w, size_t* off_gemm, size_t* gemm_bytes,
                                   int* slices) {
  int g;
  gemm_requirements(m, w, &g, gemm_bytes, kKsplitMax);
  *slices = gemm_ksplits(m, w, kKsplitMax);
  *off_gemm = align_up((size_t)*slices * m * w->n_out * 4, 256);
  return *off_gemm + align_up(*gemm_bytes, 256);
}

size_t w12_gemm_resid_norm_workspace(int64_t m, const tvp_w12_packed* w) {
  if (!w || m < 1 || m > 32) return 0;
  size_t og, gb;
  int s;
  return resid_norm_ws_layout(m, w, &og, &gb, &s);
}

int w12_gemm_resid_norm(const uint16_t* xp, int64_t m, const tvp_w12_packed* w, uint16_t* h, int64_t ldh,
                        const uint16_t* gain, float eps, uint16_t* yp, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  if (!xp || !w || !w->blob || !h || !gain || !yp) return TVP_ERR_ARG;
  if (m < 1 || m > 32 || w->n_out < 1) return TVP_ERR_SHAPE;
  if (w->chan_map != TVP_CHAN_PLAIN || !gemm_is_skinny(m, w)) return TVP_ERR_SHAPE;
  if (ldh < w->n_out || !(eps >= 0.0f)) return TVP_ERR_ARG;
  if (((uintptr_t)xp | (uintptr_t)yp | (uintptr_t)h | (uintptr_t)gain) % 16) return TVP_ERR_ARG;
  size_t off_g, gb;
  int slices;
  const size_t need = resid_norm_ws_layout(m, w, &off_g, &gb, &slices);
  if (!ws || ws_bytes < need) return TVP_ERR_WORKSPACE;
  float* part = (float*)ws;
  tvp_gemm_epilogue e{};
  e.mode = kEpiPartial;
  e.y = part;
  e.ldy = w->n_out;
  int st = gemm_run(nullptr, xp, m, 0, w, &e, 0, (uint8_t*)ws + off_g, gb, stream, kKsplitMax);
  if (st != TVP_OK) return st;
  launch_norm(part, slices, m * w->n_out, (int)w->n_out, h, (int)ldh, gain, (int)w->n_out, eps, yp, 0, 1, (int)m,
              stream);
  TVP_LAUNCH_CHECK();
  return TVP_OK;
}

int accept_path(const int32_t* argmax, const int32_t* tokens, const int32_t* parents, int32_t n,
                int32_t* path, int32_t* n_accepted, int32_t* bonus, int32_t* status, hipStream_t stream) {
  if (!argmax || !tokens || !parents || !path || !n_accepted || !bonus || !status) return TVP_ERR_ARG;
  if (n < 1 || n > 1024) return TVP_ERR_SHAPE;
  ReqInfo ri{};
  ri.n_req = 1;
  ri.node_ptr[0] = 0;
  ri.node_ptr[1] = n;
  accept_kernel<<<dim3(1), dim3(64), 0, stream>>>(argmax, tokens, parents, ri, nullptr, path, n_accepted, bonus,
                                                  status);
  TVP_LAUNCH_CHECK();
  return TVP_OK;
}

}  // extern "C"
