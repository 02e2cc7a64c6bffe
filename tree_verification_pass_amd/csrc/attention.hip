// Tree preparation (ancestor masks, positions, cache slots, validation) and
// tree-masked attention for gfx950.
//
// SpecPilot summary (onedev.kr), section 무엇인가: the target checks all draft
// tokens in one forward pass, so each node must see the committed context and
// exactly its own root path; section 전제와 한계 names tree attention as one
// of the places where reduction order may flip near-ties.
//
// Design: per (request, kv head, key split) one workgroup of up to 8
// wavefronts; wavefront w owns 32 query rows (row = gq * n + i for query head
// kv_head*G + gq and node i).  Keys are staged 64 at a time through LDS (K
// row-major, V transposed, both XOR-swizzled), scores are computed as
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so each lane owns one query row,
// masked with the node's 64-bit ancestor mask, folded into an online softmax,
// and P V is accumulated with the same MFMA (P as a sum of two bf16 pieces).  Splits
// write (max, sum, O) partials; the last split of each (request, kv head)
// merges them in split order, so the result is deterministic.
#include <math.h>

#include "internal.h"

namespace tvp {

// One workgroup (64 threads) per request.  Nodes of request r are
// node_ptr[r] .. node_ptr[r+1]-1 (at most 64); parents are request-local.
__global__ __launch_bounds__(64) void tree_prep_kernel(const int32_t* __restrict__ parents, ReqInfo ri,
                                                       int32_t s_req, uint64_t* __restrict__ anc,
                                                       int32_t* __restrict__ pos,
                                                       int32_t* __restrict__ slot,
                                                       int32_t* __restrict__ status) {
  __shared__ int32_t par[64];
  const int r = blockIdx.x, i = threadIdx.x;
  const int nb = ri.node_ptr[r], n = ri.node_ptr[r + 1] - nb;
  const int L = ri.ctx_len[r];
  int p = -2;
  if (i < n) p = parents[nb + i];
  const bool ok = i >= n || (i == 0 ? p == -1 : (p >= 0 && p < i));
  const bool all_ok = __all(ok);
  par[i] = (i < n && ok && i > 0) ? p : -1;
  __syncthreads();
  if (i < n) {
    uint64_t m = 1ull << i;
    int depth = 0;
    if (all_ok) {
      int j = par[i];
      while (j >= 0) {  // strictly decreasing, so at most i steps
        m |= 1ull << j;
        ++depth;
        j = par[j];
      }
    }
    anc[nb + i] = m;
    pos[nb + i] = L + depth;
    slot[nb + i] = r * s_req + L + i;
  }
  if (i == 0) status[r] = all_ok ? TVP_OK : TVP_ERR_TREE;
}

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  int64_t s_stride;
  ReqInfo ri;
  int32_t s_req;
  const uint64_t* anc;
  int n_req, hq, hkv, G, max_splits, rows_total, kr;
  float scale_log2;
  float* po;
  float* pm;
  float* pl;
  int row_blocks;  // merge: 16-row blocks per (request, kv head)
  uint16_t* out;
  int out_packed;  // out in the packed activation layout (<= 32 nodes) instead of [node][hq * D]
};

// Output element (global node, column `col` of the node's hq * D row).
template <int D>
__device__ inline int64_t attn_out_index(const AttnArgs& a, int node, int col) {
  return a.out_packed ? xpack_index(node, col) : (int64_t)node * a.hq * D + col;
}

template <int D, int NT>
__global__ __launch_bounds__(NT) void tree_attn_kernel(AttnArgs a) {
  constexpr int KC = 64;        // keys per LDS stage
  constexpr int CH = D / 8;     // 16-byte chunks per K row
  constexpr int NDB = D / 32;   // d blocks of the P V product
  __shared__ uint4 ks[KC * CH];              // K [key][chunk ^ (key % CH)]
  __shared__ uint2 vt[D * (KC / 4)];         // V^T [d][4-key chunk ^ (d % 16)]

  const int split = blockIdx.x % a.max_splits;
  const int kh = (blockIdx.x / a.max_splits) % a.hkv;
  const int r = blockIdx.x / (a.max_splits * a.hkv);
  const int L = a.ri.ctx_len[r], nb = a.ri.node_ptr[r], n = a.ri.node_ptr[r + 1] - nb;
  const int T = L + n, R = a.G * n;
  const int nsplit = (T + a.kr - 1) / a.kr;
  if (split >= nsplit) return;
  const int k0 = split * a.kr, k1 = min(T, k0 + a.kr);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5;
  constexpr int nthr = NT;
  const int row = wave * 32 + (lane & 31);
  const bool row_ok = row < R;
  const int gq = row_ok ? row / n : 0, node = row_ok ? row % n : 0;
  const int64_t cbase = (int64_t)kh * a.s_stride + (int64_t)r * a.s_req;  // slot 0 of this request/head
  const uint16_t* kbase = a.kc + cbase * D;
  const uint16_t* vbase = a.vc + cbase * D;

  // Q fragments (B operand): lane holds q[row][16 ds + 8 h .. +7]
  uint4 qf[D / 16];
  {
    const uint16_t* qp = a.q + ((int64_t)(nb + node) * a.hq + kh * a.G + gq) * D;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds)
      qf[ds] = row_ok ? *(const uint4*)(qp + 16 * ds + 8 * h) : make_uint4(0, 0, 0, 0);
  }
  const uint64_t anc = row_ok ? a.anc[nb + node] : 0ull;

  float m_run = -INFINITY, l_run = 0.0f;
  f32x16_t o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.0f;

  // K/V of the next 64 keys are fetched into registers while the current
  // ones are used (nthr is 256 or 512, so at most PER chunks per thread).
  constexpr int PER = KC * CH / NT;
  uint4 kpre[PER], vpre[PER];
  auto fetch = [&](int sub) {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int idx = tid + it * nthr;
      kpre[it] = make_uint4(0, 0, 0, 0);
      vpre[it] = make_uint4(0, 0, 0, 0);
      if (idx < KC * CH) {
        const int kk = sub + idx % KC, c = idx / KC;
        if (kk < k1) {
          kpre[it] = *(const uint4*)(kbase + (int64_t)kk * D + 8 * c);
          vpre[it] = *(const uint4*)(vbase + (int64_t)kk * D + 8 * c);
        }
      }
    }
  };
  auto stash = [&]() {
    uint16_t* vts = (uint16_t*)vt;
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int idx = tid + it * nthr;
      if (idx >= KC * CH) continue;
      const int key = idx % KC, c = idx / KC;
      ks[key * CH + (c ^ (key % CH))] = kpre[it];
      const uint4 vv = vpre[it];
      const uint32_t hv[8] = {vv.x & 0xFFFFu, vv.x >> 16, vv.y & 0xFFFFu, vv.y >> 16,
                              vv.z & 0xFFFFu, vv.z >> 16, vv.w & 0xFFFFu, vv.w >> 16};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dd = 8 * c + e;
        vts[(dd * (KC / 4) + ((key >> 2) ^ (dd & 15))) * 4 + (key & 3)] = (uint16_t)hv[e];
      }
    }
  };

  fetch(k0);
  for (int sub = k0; sub < k1; sub += KC) {
    __syncthreads();
    stash();
    __syncthreads();
    if (sub + KC < k1) fetch(sub + KC);
    if (wave * 32 >= R) continue;

    // one 32-key block at a time: scores S^T[key][row], online softmax, P V
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16_t sc;
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[v] = 0.0f;
      {
        const int key = kb * 32 + (lane & 31);
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
          const bf16x8_t A = __builtin_bit_cast(bf16x8_t, ks[key * CH + ((2 * ds + h) ^ (key % CH))]);
          const bf16x8_t B = __builtin_bit_cast(bf16x8_t, qf[ds]);
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, sc, 0, 0, 0);
        }
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = sub + kb * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        bool vis = row_ok && key < k1;
        if (vis && key >= L) vis = (anc >> (key - L)) & 1ull;
        const float x = vis ? sc[v] * a.scale_log2 : -INFINITY;
        sc[v] = x;
        mloc = fmaxf(mloc, x);
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float base = m_new == -INFINITY ? 0.0f : m_new;
      const float alpha = exp2f(m_run - base);
      // P is split into two bf16 pieces (hi = bf16(p), lo = bf16(p - hi)) so the
      // P V product on bf16 MFMA keeps 16 significant bits of every weight.
      float lsum = 0.0f;
      uint32_t pk[8], pl[8];
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const float p0 = exp2f(sc[v] - base), p1 = exp2f(sc[v + 1] - base);
        lsum += p0 + p1;
        const uint32_t h0 = f32_to_bf16(p0), h1 = f32_to_bf16(p1);
        pk[v / 2] = h0 | (h1 << 16);
        pl[v / 2] = f32_to_bf16(p0 - bf16_to_f32(h0)) | (f32_to_bf16(p1 - bf16_to_f32(h1)) << 16);
      }
      lsum += __shfl_xor(lsum, 32);
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] *= alpha;

      // O^T[d][row] += V^T[d][key] P^T[key][row]; MFMA q of this key block
      // covers keys kb*32 + 16 q + 8 (i/4) + 4 h + i%4 for k-index 8 h + i.
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const bf16x8_t B = __builtin_bit_cast(bf16x8_t, make_uint4(pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]));
        const bf16x8_t Bl = __builtin_bit_cast(bf16x8_t, make_uint4(pl[4 * q], pl[4 * q + 1], pl[4 * q + 2], pl[4 * q + 3]));
        const int c8 = 8 * kb + 4 * q + h;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int dd = db * 32 + (lane & 31);
          const uint2 lo = vt[dd * (KC / 4) + (c8 ^ (dd & 15))];
          const uint2 hi = vt[dd * (KC / 4) + ((c8 + 2) ^ (dd & 15))];
          const bf16x8_t A = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, o[db], 0, 0, 0);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bl, o[db], 0, 0, 0);
        }
      }
    }
  }

  // single split: normalise and store; otherwise write (max, sum, O) partials
  if (nsplit == 1) {
    if (row_ok) {
      const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
      const int c0 = (kh * a.G + gq) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          a.out[attn_out_index<D>(a, nb + node, c0 + db * 32 + 8 * (v >> 2) + 4 * h + (v & 3))] =
              (uint16_t)f32_to_bf16(o[db][v] * inv);
    }
    return;
  }
  // partial rows: [kv head][split][G * global node], request r's rows start at G * nb
  const int64_t pbase = ((int64_t)kh * a.max_splits + split) * a.rows_total + (int64_t)a.G * nb;
  if (row_ok) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int dd = db * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        a.po[(pbase + row) * D + dd] = o[db][v];
      }
    if (h == 0) {
      a.pm[pbase + row] = m_run;
      a.pl[pbase + row] = l_run;
    }
  }
}

// Merge of the key splits (a separate launch: the kernel boundary makes every
// split's partials visible).  One workgroup per (request, kv head, 16 query
// rows); each row's split weights are formed by 16 lanes with a fixed
// shuffle-tree order, then every output element sums its splits in split
// order, so the result is deterministic.
template <int D>
__global__ __launch_bounds__(256) void tree_attn_merge_kernel(AttnArgs a) {
  __shared__ float wts[16 * 64];  // [row][split], normalised merge weights
  const int rb = blockIdx.x % a.row_blocks;
  const int kh = (blockIdx.x / a.row_blocks) % a.hkv;
  const int r = blockIdx.x / (a.row_blocks * a.hkv);
  const int L = a.ri.ctx_len[r], nb = a.ri.node_ptr[r], n = a.ri.node_ptr[r + 1] - nb;
  const int R = a.G * n;
  const int nsplit = (L + n + a.kr - 1) / a.kr;  // <= 64
  if (nsplit <= 1 || rb * 16 >= R) return;
  const int tid = threadIdx.x;
  const int64_t hb = (int64_t)kh * a.max_splits * a.rows_total + (int64_t)a.G * nb;
  const int r0 = rb * 16, nr = min(16, R - r0);
  {
    const int lr = tid >> 4, s0 = tid & 15;  // 16 lanes per row, 4 rows per wavefront
    const bool rok = lr < nr;
    float pm[4], pl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sp = s0 + 16 * j;
      const bool ok = rok && sp < nsplit;
      const int64_t pr = hb + (int64_t)sp * a.rows_total + r0 + lr;
      pm[j] = ok ? a.pm[pr] : -INFINITY;
      pl[j] = ok ? a.pl[pr] : 0.0f;
    }
    float mx = fmaxf(fmaxf(pm[0], pm[1]), fmaxf(pm[2], pm[3]));
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float bse = mx == -INFINITY ? 0.0f : mx;
    float w[4], den = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[j] = pm[j] == -INFINITY ? 0.0f : exp2f(pm[j] - bse);
      den += pl[j] * w[j];
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) den += __shfl_xor(den, off);
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (rok) wts[lr * 64 + s0 + 16 * j] = w[j] * inv;
  }
  __syncthreads();
  for (int q4 = tid; q4 < nr * (D / 4); q4 += 256) {
    const int lr = q4 / (D / 4), dd = (q4 % (D / 4)) * 4;
    const int rr = r0 + lr;
    const float* src = a.po + (hb + rr) * D + dd;
    const int64_t sstride = (int64_t)a.rows_total * D;
    float4 acc4 = make_float4(0.f, 0.f, 0.f, 0.f);
    int sp = 0;
    for (; sp + 4 <= nsplit; sp += 4) {  // four independent loads in flight
      float4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = *(const float4*)(src + (sp + j) * sstride);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float wj = wts[lr * 64 + sp + j];
        acc4.x += v[j].x * wj;
        acc4.y += v[j].y * wj;
        acc4.z += v[j].z * wj;
        acc4.w += v[j].w * wj;
      }
    }
    for (; sp < nsplit; ++sp) {
      const float4 v = *(const float4*)(src + sp * sstride);
      const float wj = wts[lr * 64 + sp];
      acc4.x += v.x * wj;
      acc4.y += v.y * wj;
      acc4.z += v.z * wj;
      acc4.w += v.w * wj;
    }
    const int g2 = rr / n, nd = rr % n;
    // four consecutive columns stay within one 8-column group of the packed layout
    uint16_t* op = a.out + attn_out_index<D>(a, nb + nd, (kh * a.G + g2) * D + dd);
    op[0] = (uint16_t)f32_to_bf16(acc4.x);
    op[1] = (uint16_t)f32_to_bf16(acc4.y);
    op[2] = (uint16_t)f32_to_bf16(acc4.z);
    op[3] = (uint16_t)f32_to_bf16(acc4.w);
  }
}

#ifndef TVP_ATTN_KR
#define TVP_ATTN_KR 128  // keys per split (doubled while more than 64 splits would be needed)
#endif

struct AttnPlan {
  int kr, max_splits, rows_total, nthreads;
  size_t off_po, off_pm, off_pl, bytes;
};

// max_keys: largest ctx_len + n over the requests; r_max: largest G * n;
// n_total: nodes of all requests.
static AttnPlan attn_plan(int hkv, int G, int d, int r_max, int n_total, int max_keys) {
  AttnPlan p{};
  p.kr = TVP_ATTN_KR;
  while (max_keys > 64 * p.kr) p.kr *= 2;  // at most 64 splits (merge weights live in LDS)
  p.max_splits = max_keys > 0 ? (max_keys + p.kr - 1) / p.kr : 1;
  p.rows_total = G * n_total;
  p.nthreads = r_max <= 128 ? 256 : 512;
  const size_t rows = (size_t)hkv * p.max_splits * p.rows_total;
  size_t off = 0;
  p.off_po = off;
  off = align_up(off + rows * d * 4, 256);
  p.off_pm = off;
  off = align_up(off + rows * 4, 256);
  p.off_pl = off;
  off = align_up(off + rows * 4, 256);
  p.bytes = off;
  return p;
}

int launch_tree_prep(const int32_t* parents, const ReqInfo& ri, int32_t s_req, uint64_t* anc,
                     int32_t* pos, int32_t* slot, int32_t* status, hipStream_t stream) {
  tree_prep_kernel<<<dim3(ri.n_req), dim3(64), 0, stream>>>(parents, ri, s_req, anc, pos, slot, status);
  TVP_LAUNCH_CHECK();
  return TVP_OK;
}

int launch_tree_attention(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, int64_t s_stride,
                          const ReqInfo& ri, int32_t s_req, const uint64_t* anc, int hq, int hkv, int d,
                          int r_max, int max_keys, uint16_t* out, int out_packed, void* scratch,
                          size_t scratch_bytes, hipStream_t stream) {
  if (r_max > 256 || r_max < 1) return TVP_ERR_SHAPE;
  if (out_packed && ri.node_ptr[ri.n_req] > 32) return TVP_ERR_SHAPE;
  const int n_req = ri.n_req;
  const AttnPlan p = attn_plan(hkv, hq / hkv, d, r_max, ri.node_ptr[n_req], max_keys);
  if (scratch_bytes < p.bytes) return TVP_ERR_WORKSPACE;
  AttnArgs a{};
  a.q = q;
  a.kc = kc;
  a.vc = vc;
  a.s_stride = s_stride;
  a.ri = ri;
  a.s_req = s_req;
  a.anc = anc;
  a.n_req = n_req;
  a.hq = hq;
  a.hkv = hkv;
  a.G = hq / hkv;
  a.max_splits = p.max_splits;
  a.rows_total = p.rows_total;
  a.kr = p.kr;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
  uint8_t* sb = (uint8_t*)scratch;
  a.po = (float*)(sb + p.off_po);
  a.pm = (float*)(sb + p.off_pm);
  a.pl = (float*)(sb + p.off_pl);
  a.out = out;
  a.out_packed = out_packed;
  a.row_blocks = (r_max + 15) / 16;
  const dim3 grid((unsigned)(n_req * hkv * p.max_splits));
  const dim3 mgrid((unsigned)(n_req * hkv * a.row_blocks));
  if (d == 128) {
    if (p.nthreads == 256) tree_attn_kernel<128, 256><<<grid, dim3(256), 0, stream>>>(a);
    else tree_attn_kernel<128, 512><<<grid, dim3(512), 0, stream>>>(a);
    if (p.max_splits > 1) tree_attn_merge_kernel<128><<<mgrid, dim3(256), 0, stream>>>(a);
  } else if (d == 64) {
    if (p.nthreads == 256) tree_attn_kernel<64, 256><<<grid, dim3(256), 0, stream>>>(a);
    else tree_attn_kernel<64, 512><<<grid, dim3(512), 0, stream>>>(a);
    if (p.max_splits > 1) tree_attn_merge_kernel<64><<<mgrid, dim3(256), 0, stream>>>(a);
  } else {
    return TVP_ERR_SHAPE;
  }
  TVP_LAUNCH_CHECK();
  return TVP_OK;
}

size_t attention_scratch_bytes(int hkv, int G, int d, int r_max, int n_total, int max_keys) {
  return attn_plan(hkv, G, d, r_max, n_total, max_keys).bytes;
}

}  // namespace tvp

using namespace tvp;

// Standalone layout of the tree_attention workspace:
//   [0, 256)        reserved
//   [256, ...)      anc u64 [64], pos/slot i32 [64]
//   then            attention partials
static size_t ta_layout(int32_t n, int32_t hq, int32_t hkv, int32_t d, int32_t max_keys, size_t* off_part) {
  const size_t off = align_up(256 + 64 * 8 + 2 * 64 * 4, 256);
  *off_part = off;
  const int G = hkv > 0 ? hq / hkv : 1;
  return off + attention_scratch_bytes(hkv, G, d, G * n, n, max_keys);
}

extern "C" {

size_t tree_attention_workspace(int32_t n, int32_t hq, int32_t d, int32_t max_keys) {
  if (n < 1 || hq < 1 || max_keys < 1) return 0;
  size_t offp, best = 0;
  for (int32_t hkv = 1; hkv <= hq; ++hkv) {
    if (hq % hkv) continue;
    const size_t b = ta_layout(n, hq, hkv, d, max_keys, &offp);
    best = b > best ? b : best;
  }
  return best;
}

int tree_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, int64_t s_stride,
                   int32_t ctx_len, const int32_t* parents, int32_t n, int32_t hq, int32_t hkv, int32_t d,
                   uint16_t* out, int32_t* status, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !parents || !out || !status) return TVP_ERR_ARG;
  if (n < 1 || n > 64 || hq < 1 || hkv < 1 || hkv > 64 || hq % hkv || ctx_len < 0) return TVP_ERR_SHAPE;
  if (d != 64 && d != 128) return TVP_ERR_SHAPE;
  if ((int64_t)ctx_len + n > s_stride) return TVP_ERR_CAPACITY;
  if ((hq / hkv) * n > 256) return TVP_ERR_SHAPE;
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache) % 16) return TVP_ERR_ARG;
  size_t offp;
  const size_t need = ta_layout(n, hq, hkv, d, ctx_len + n, &offp);
  if (!ws || ws_bytes < need) return TVP_ERR_WORKSPACE;
  uint8_t* w = (uint8_t*)ws;
  uint64_t* anc = (uint64_t*)(w + 256);
  int32_t* pos = (int32_t*)(w + 256 + 64 * 8);
  int32_t* slot = pos + 64;
  ReqInfo ri{};
  ri.n_req = 1;
  ri.ctx_len[0] = ctx_len;
  ri.node_ptr[0] = 0;
  ri.node_ptr[1] = n;
  int st = launch_tree_prep(parents, ri, 0, anc, pos, slot, status, stream);
  if (st != TVP_OK) return st;
  return launch_tree_attention(q, k_cache, v_cache, s_stride, ri, 0, anc, hq, hkv, d, (hq / hkv) * n,
                               ctx_len + n, out, 0, w + offp, ws_bytes - offp, stream);
}

}  // extern "C"
