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
// kv_head*G + gq and node i).  Keys are staged 64 at a time through LDS with
// fully coalesced 16-byte loads (K and V both row-major there, XOR-swizzled
// per row).  Scores are computed as S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 so each lane owns one query row, masked with the
// node's 64-bit ancestor mask and folded into an online softmax; P V is
// accumulated with the same MFMA, its V^T operand read straight from the
// row-major V tile with the LDS transpose read (ds_read_b64_tr_b16), and P
// applied as a sum of two bf16 pieces.  Splits write (max, sum, O) partials
// in the accumulator's own register layout (one coalesced 256-byte store per
// accumulator register); a separate merge launch sums them in split order,
// so the result is deterministic.
#include <math.h>

#include <algorithm>

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

// Partial rows of request r start at prow[r]: its G * n rows rounded up to a
// multiple of 32, so every wavefront's 32-row block is its own.
struct PartRows {
  int32_t prow[kMaxReq + 1];
};

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
  int row_blocks;  // merge: 32-row blocks per (request, kv head)
  PartRows pr;
  uint16_t* out;
  int out_packed;  // out in the packed activation layout (<= 32 nodes) instead of [node][hq * D]
};

// Output element (global node, column `col` of the node's hq * D row).
template <int D>
__device__ inline int64_t attn_out_index(const AttnArgs& a, int node, int col) {
  return a.out_packed ? xpack_index(node, col) : (int64_t)node * a.hq * D + col;
}

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// Swizzle of V rows in LDS (16-byte chunk index XOR): the transpose reads of
// one MFMA operand touch 8 rows x 64 bytes and spread evenly over the banks.
template <int D>
__device__ inline int v_swz(int key) {
  return D == 128 ? ((key & 3) << 2) : (((key >> 1) & 1) << 2);
}

template <int D, int NT>
__global__ __launch_bounds__(NT) void tree_attn_kernel(AttnArgs a) {
  constexpr int KC = 64;        // keys per LDS stage
  constexpr int CH = D / 8;     // 16-byte chunks per row
  constexpr int NDB = D / 32;   // d blocks of the P V product
  __shared__ uint4 ks[KC * CH];  // K [key][chunk ^ (key % CH)]
  __shared__ uint4 vs[KC * CH];  // V [key][chunk ^ v_swz(key)]

  const int split = blockIdx.x % a.max_splits;
  const int kh = (blockIdx.x / a.max_splits) % a.hkv;
  const int r = blockIdx.x / (a.max_splits * a.hkv);
  const int L = a.ri.ctx_len[r], nb = a.ri.node_ptr[r], n = a.ri.node_ptr[r + 1] - nb;
  const int T = L + n, R = a.G * n;
  const int nsplit = (T + a.kr - 1) / a.kr;
  if (split >= nsplit) return;
  const int k0 = split * a.kr, k1 = min(T, k0 + a.kr);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5;
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

  // K/V of the next 64 keys are fetched into registers while the current ones
  // are used; CH consecutive lanes read one 2*D-byte row.
  constexpr int PER = KC * CH / NT;
  uint4 kpre[PER], vpre[PER];
  auto fetch = [&](int sub) {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int idx = tid + it * NT;
      const int kk = sub + idx / CH, c = idx % CH;
      kpre[it] = make_uint4(0, 0, 0, 0);
      vpre[it] = make_uint4(0, 0, 0, 0);
      if (kk < k1) {
        kpre[it] = *(const uint4*)(kbase + (int64_t)kk * D + 8 * c);
        vpre[it] = *(const uint4*)(vbase + (int64_t)kk * D + 8 * c);
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int idx = tid + it * NT;
      const int key = idx / CH, c = idx % CH;
      ks[key * CH + (c ^ (key % CH))] = kpre[it];
      vs[key * CH + (c ^ v_swz<D>(key))] = vpre[it];
    }
  };
  // transpose-read geometry: in each 16-lane group, source lane s points at
  // key row (s / 4) and 4 d-columns (s % 4) * 4; lane i then receives
  // V[key0 + 0..3][d0 + i]
  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr_key = 4 * h + (s16 >> 2);
  const int tr_d = 16 * (g16 & 1) + 4 * (s16 & 3);
  const char* vs_bytes = (const char*)vs;

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
      // raw scores; the 1/sqrt(d) scale (in log2 units) is applied inside the
      // exponent.  Blocks of context keys only need no mask.
      float mloc = -INFINITY;
      const int kb0 = sub + kb * 32;
      if (kb0 + 32 <= min(L, k1)) {
#pragma unroll
        for (int v = 0; v < 16; ++v) mloc = fmaxf(mloc, sc[v]);
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kb0 + 8 * (v >> 2) + 4 * h + (v & 3);
          bool vis = row_ok && key < k1;
          if (vis && key >= L) vis = (anc >> (key - L)) & 1ull;
          sc[v] = vis ? sc[v] : -INFINITY;
          mloc = fmaxf(mloc, sc[v]);
        }
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float base = m_new == -INFINITY ? 0.0f : m_new;
      const float nbs = -base * a.scale_log2;
      const float alpha = __builtin_amdgcn_exp2f((m_run - base) * a.scale_log2);
      // P is split into two bf16 pieces (hi = bf16(p), lo = bf16(p - hi)) so the
      // P V product on bf16 MFMA keeps 16 significant bits of every weight.
      float lsum = 0.0f;
      uint32_t pk[8], pl[8];
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[v], a.scale_log2, nbs));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[v + 1], a.scale_log2, nbs));
        lsum += p0 + p1;
        const uint32_t hk = pack_bf16x2(p0, p1);
        pk[v / 2] = hk;
        pl[v / 2] = pack_bf16x2(p0 - __uint_as_float(hk << 16), p1 - __uint_as_float(hk & 0xFFFF0000u));
      }
      lsum += __shfl_xor(lsum, 32);
      l_run = l_run * alpha + lsum;
      m_run = m_new;
      if (__ballot(alpha != 1.0f)) {  // the running max moved for some row: rescale
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
      }

      // O^T[d][row] += V^T[d][key] P^T[key][row]; MFMA q of this key block
      // covers keys kb*32 + 16 q + 8 (i/4) + 4 h + i%4 for k-index 8 h + i.
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const bf16x8_t B = __builtin_bit_cast(bf16x8_t, make_uint4(pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]));
        const bf16x8_t Bl = __builtin_bit_cast(bf16x8_t, make_uint4(pl[4 * q], pl[4 * q + 1], pl[4 * q + 2], pl[4 * q + 3]));
        const int r1 = kb * 32 + 16 * q + tr_key, r2 = r1 + 8;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = 32 * db + tr_d;  // 4 columns, 8 bytes inside one 16-byte chunk
          const int off1 = (r1 * CH + ((d >> 3) ^ v_swz<D>(r1))) * 16 + (d & 7) * 2;
          const int off2 = (r2 * CH + ((d >> 3) ^ v_swz<D>(r2))) * 16 + (d & 7) * 2;
          const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(vs_bytes + off1));
          const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(vs_bytes + off2));
          const uint2 lo2 = __builtin_bit_cast(uint2, lo), hi2 = __builtin_bit_cast(uint2, hi);
          const bf16x8_t A = __builtin_bit_cast(bf16x8_t, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, o[db], 0, 0, 0);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bl, o[db], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);  // keeps the operand reads of the two halves apart (register pressure)
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
  if (wave * 32 >= R) return;
  // partial rows: [kv head][split][padded rows]; this wavefront's 32-row block
  // is stored in the accumulator layout: element (db, v) of lane l at
  // block * D + (db * 16 + v) * 64 + l
  const int64_t pbase = ((int64_t)kh * a.max_splits + split) * a.rows_total + a.pr.prow[r] + wave * 32;
  float* pob = a.po + pbase * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) pob[(db * 16 + v) * 64 + lane] = o[db][v];
  if (h == 0) {  // the running max is a raw score (unscaled)
    a.pm[pbase + (lane & 31)] = m_run;
    a.pl[pbase + (lane & 31)] = l_run;
  }
}

// Merge of the key splits (a separate launch: the kernel boundary makes every
// split's partials visible).  One workgroup per (request, kv head, 32-row
// block, quarter of the block's D*32 elements).  Each row's split weights
// come from 8 lanes with a fixed shuffle-tree order; every output element
// sums its splits in split order, so the result is deterministic.
template <int D>
__global__ __launch_bounds__(256) void tree_attn_merge_kernel(AttnArgs a) {
  __shared__ float wts[32 * 64];  // [row][split], normalised merge weights
  const int qt = blockIdx.x & 3;
  const int rb = (blockIdx.x >> 2) % a.row_blocks;
  const int kh = ((blockIdx.x >> 2) / a.row_blocks) % a.hkv;
  const int r = (blockIdx.x >> 2) / (a.row_blocks * a.hkv);
  const int L = a.ri.ctx_len[r], nb = a.ri.node_ptr[r], n = a.ri.node_ptr[r + 1] - nb;
  const int R = a.G * n;
  const int nsplit = (L + n + a.kr - 1) / a.kr;  // <= 64
  if (nsplit <= 1 || rb * 32 >= R) return;
  const int tid = threadIdx.x;
  // row block base of split 0; split sp adds sp * rows_total
  const int64_t hb = (int64_t)kh * a.max_splits * a.rows_total + a.pr.prow[r] + rb * 32;
  {
    const int lr = tid >> 3, s0 = tid & 7;  // 8 lanes per row
    float pm[8], pl[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sp = s0 + 8 * j;
      const bool ok = sp < nsplit;
      const int64_t pr = hb + (int64_t)sp * a.rows_total + lr;
      pm[j] = ok ? a.pm[pr] : -INFINITY;
      pl[j] = ok ? a.pl[pr] : 0.0f;
    }
    float mx = pm[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, pm[j]);
#pragma unroll
    for (int off = 4; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float bse = mx == -INFINITY ? 0.0f : mx;
    float w[8], den = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      w[j] = pm[j] == -INFINITY ? 0.0f : exp2f((pm[j] - bse) * a.scale_log2);  // maxima are raw scores
      den += pl[j] * w[j];
    }
#pragma unroll
    for (int off = 4; off > 0; off >>= 1) den += __shfl_xor(den, off);
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) wts[lr * 64 + s0 + 8 * j] = w[j] * inv;
  }
  __syncthreads();
  const int64_t sstride = (int64_t)a.rows_total * D;
  const float* src = a.po + hb * D;
  constexpr int NE = D / 32;  // elements per thread
  int pe[NE];
  float acc[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    pe[i] = qt * (8 * D) + i * 256 + tid;  // element of the block in accumulator layout
    acc[i] = 0.0f;
  }
  int sp = 0;
  for (; sp + 4 <= nsplit; sp += 4) {  // 4 * NE independent loads in flight
    float v[4][NE];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < NE; ++i) v[j][i] = src[(sp + j) * sstride + pe[i]];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < NE; ++i) acc[i] += v[j][i] * wts[(pe[i] & 31) * 64 + sp + j];
  }
  for (; sp < nsplit; ++sp)
#pragma unroll
    for (int i = 0; i < NE; ++i) acc[i] += src[sp * sstride + pe[i]] * wts[(pe[i] & 31) * 64 + sp];
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int ln = pe[i] & 63, dv = pe[i] >> 6;  // lane, db * 16 + v
    const int rr = rb * 32 + (ln & 31);
    if (rr < R) {
      const int db = dv >> 4, v = dv & 15;
      const int dd = db * 32 + 8 * (v >> 2) + 4 * (ln >> 5) + (v & 3);
      const int g2 = rr / n, nd = rr % n;
      a.out[attn_out_index<D>(a, nb + nd, (kh * a.G + g2) * D + dd)] = (uint16_t)f32_to_bf16(acc[i]);
    }
  }
}

// Key splits are sized so that one launch has about this many workgroups
// (one per compute unit: a workgroup fills a CU's register file).
constexpr int kAttnTargetGroups = 256;

struct AttnPlan {
  int kr, max_splits, rows_total, nthreads;
  size_t off_po, off_pm, off_pl, bytes;
};

// max_keys: largest ctx_len + n over the requests; r_max: largest G * n;
// rows_total: partial rows over all requests (each request's G * n rounded
// up to a multiple of 32).  Splits are multiples of the 64-key stage.
static AttnPlan attn_plan(int hkv, int d, int r_max, int rows_total, int max_keys, int n_req) {
  AttnPlan p{};
  const int target = std::max(1, kAttnTargetGroups / std::max(1, n_req * hkv));
  p.kr = 64 * (int)ceil_div(std::max(max_keys, 1), 64LL * target);
  while (max_keys > 64 * p.kr) p.kr *= 2;  // at most 64 splits (merge weights live in LDS)
  p.max_splits = max_keys > 0 ? (max_keys + p.kr - 1) / p.kr : 1;
  p.rows_total = rows_total;
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
  const int G = hq / hkv;
  AttnArgs a{};
  a.pr.prow[0] = 0;
  for (int i = 0; i < n_req; ++i)
    a.pr.prow[i + 1] = a.pr.prow[i] + (int)align_up((size_t)G * (ri.node_ptr[i + 1] - ri.node_ptr[i]), 32);
  const AttnPlan p = attn_plan(hkv, d, r_max, a.pr.prow[n_req], max_keys, n_req);
  if (scratch_bytes < p.bytes) return TVP_ERR_WORKSPACE;
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
  a.row_blocks = (r_max + 31) / 32;
  const dim3 grid((unsigned)(n_req * hkv * p.max_splits));
  const dim3 mgrid((unsigned)(n_req * hkv * a.row_blocks * 4));
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
  // every request's rows are padded to a multiple of 32; the split count
  // depends on the number of requests
  size_t best = 0;
  for (int nr = 1; nr <= std::min(kMaxReq, std::max(n_total, 1)); ++nr)
    best = std::max(best, attn_plan(hkv, d, r_max, G * n_total + 31 * nr, max_keys, nr).bytes);
  return best;
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
