// Gated DeltaNet layers of a hybrid target over a draft tree, for gfx950:
// every node's output with the recurrent state taken along its own root
// path, two ways, and the replay of the accepted path into the committed
// state.
//
// SpecPilot summary (onedev.kr), section 무엇과 다른가: for hybrid targets the
// recurrent state is recomputed along each path rather than stored per node
// (path verify); a WY-form verify turns the chain of rank-1 updates into
// matrix products solved for all paths at once, with the fp32 state carried
// as three bf16 pieces so its 24-bit significand is kept exactly; after
// acceptance the accepted path is replayed into every recurrent layer
// (commit).  The recurrence is the gated delta rule of Gated DeltaNet (Yang,
// Kautz and Hatamizadeh, ICLR 2025): per value head a dv x dk state S,
//   S <- alpha S + beta (v - alpha S k) k^T,   o = S q   (alpha = exp(g)).
//
// WY form over the tree (G_i: sum of g over node i's root path, node
// included; nodes in topological order so ancestors come first):
//   (I + A) U = B,  A_ij = beta_i e^(G_i - G_j) k_i.k_j  (j a strict ancestor of i),
//                   B_i  = beta_i (v_i - e^(G_i) S0 k_i),
//   o_i = e^(G_i) S0 q_i + sum over j ancestor-or-self of i of e^(G_i - G_j) (q_i.k_j) u_j.
// u_i is node i's write, beta_i (v_i - alpha_i S_parent k_i); unrolling the
// recurrence along any root path gives exactly these equations.  The four
// products K K^T, Q K^T, K S0^T and Q S0^T run on MFMA (bf16 in, fp32
// accumulate, S0 as hi + mid + lo bf16 pieces); the triangular solve and the
// output sums are fp32 on the vector units.
#include <math.h>

#include "internal.h"

namespace tvp {

constexpr int kGdnMaxNodes = 32;
constexpr int kGdnD = 128;  // dk = dv

struct GdnArgs {
  const uint16_t* q;  // [n][hk][dk] bf16
  const uint16_t* k;  // [n][hk][dk] bf16
  const uint16_t* v;  // [n][hv][dv] bf16
  const float* g;     // [n][hv]
  const float* beta;  // [n][hv]
  const float* state; // [hv][dv][dk]
  const int32_t* parents;
  int n, hk, hv;
  uint16_t* out;      // [n][hv][dv] bf16
  int32_t* status;
};

// Ancestor-or-self masks of the tree in LDS, built by the first wavefront
// (lane i: node i).  A tree that breaks parents[0] = -1, 0 <= parents[i] < i
// gets self-only masks (every later access stays in bounds) and
// TVP_ERR_TREE.  Returns whether the tree is valid (same value in every
// thread after the barrier).
__device__ inline bool gdn_tree_masks(const int32_t* __restrict__ parents, int n, int32_t* par,
                                      uint32_t* anc, int* ok_flag) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    // loads stay unconditional (clamped index): a load inside a branch is
    // waited for at the branch's end
    const int pl = parents[min(tid, n - 1)];
    const int p = tid < n ? pl : -2;
    const bool ok = tid >= n || (tid == 0 ? p == -1 : (p >= 0 && p < tid));
    const bool all_ok = __all(ok);
    if (tid < kGdnMaxNodes) par[tid] = (tid < n && all_ok && tid > 0) ? p : -1;
    if (tid == 0) *ok_flag = all_ok ? 1 : 0;
  }
  __syncthreads();
  if (tid < kGdnMaxNodes) {
    uint32_t m = 0;
    if (tid < n) {
      m = 1u << tid;
      for (int j = par[tid]; j >= 0; j = par[j]) m |= 1u << j;  // strictly decreasing
    }
    anc[tid] = m;
  }
  __syncthreads();
  return *ok_flag != 0;
}

// Eight fp32 values as three bf16 operands whose sum is exact: hi is the
// nearest bf16, mid the nearest bf16 to the remainder, lo the rest (at most
// 8 significant bits are left, so exact for every normal value above 2^-110).
__device__ inline void split3(const float4 a, const float4 b, bf16x8_t& hi, bf16x8_t& mid, bf16x8_t& lo) {
  const float s[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    h[e / 2] = pack_bf16x2(s[e], s[e + 1]);
    const float r0 = s[e] - __uint_as_float(h[e / 2] << 16);
    const float r1 = s[e + 1] - __uint_as_float(h[e / 2] & 0xFFFF0000u);
    m[e / 2] = pack_bf16x2(r0, r1);
    l[e / 2] = pack_bf16x2(r0 - __uint_as_float(m[e / 2] << 16), r1 - __uint_as_float(m[e / 2] & 0xFFFF0000u));
  }
  hi = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
  mid = __builtin_bit_cast(bf16x8_t, make_uint4(m[0], m[1], m[2], m[3]));
  lo = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
}

// Eight bf16 (one 16-byte load) to fp32 in LDS.
__device__ inline void unpack8(const uint4 x, float* dst) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    dst[2 * e] = __uint_as_float(w[e] << 16);
    dst[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
  }
}

// Two threads per state row (thread t: row t / 2, columns 64 (t % 2) .. +63,
// held in registers).  Dot product of the row with x (LDS, the same half):
// four interleaved fp32 partial sums per half, added pairwise, then the
// two halves added lower half first (both threads get the same bits).
constexpr int kHalf = kGdnD / 2;
__device__ inline float pair_dot(const float* S, const float* x) {
  float p0 = 0.0f, p1 = 0.0f, p2 = 0.0f, p3 = 0.0f;
#pragma unroll
  for (int c = 0; c < kHalf; c += 4) {
    p0 = fmaf(S[c], x[c], p0);
    p1 = fmaf(S[c + 1], x[c + 1], p1);
    p2 = fmaf(S[c + 2], x[c + 2], p2);
    p3 = fmaf(S[c + 3], x[c + 3], p3);
  }
  const float p = (p0 + p1) + (p2 + p3);
  const float o = __shfl_xor(p, 1);
  return (threadIdx.x & 1) ? o + p : p + o;
}

// One gated delta-rule update of a half row in registers (vr = v at the
// row, x = the key's same half).
__device__ inline void pair_update(float* S, const float* x, float al, float be, float vr) {
  const float t = be * (vr - al * pair_dot(S, x));
#pragma unroll
  for (int c = 0; c < kHalf; ++c) S[c] = fmaf(al, S[c], t * x[c]);
}

// Loads / stores a half row of 64 fp32.
__device__ inline void load_half(const float* src, float* S) {
#pragma unroll
  for (int c = 0; c < kHalf / 4; ++c) {
    const float4 x = ((const float4*)src)[c];
    S[4 * c] = x.x;
    S[4 * c + 1] = x.y;
    S[4 * c + 2] = x.z;
    S[4 * c + 3] = x.w;
  }
}

// u along the root path of node i (mask mk, root first) at value dimension c,
// and o_i's path sum: for path position p (node x), u_x = B_x - sum over
// earlier path positions q of A[x][path q] u_q, then o += E[i][x] u_x.  Fully
// unrolled to P positions with no branch: positions past the path take node 0
// with zero coefficients, so they add nothing.
template <int P>
__device__ inline float wy_path(uint32_t mk, int i, int c, const float (*Am)[33], const float (*Em)[33],
                                const float (*Bm)[33]) {
  int pn[P];
  bool on[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    on[p] = mk != 0;
    pn[p] = on[p] ? __ffs(mk) - 1 : 0;
    mk &= mk - 1;
  }
  float u[P];
  float o = 0.0f;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int x = pn[p];
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < p; ++q) s = fmaf(Am[x][pn[q]], u[q], s);
    u[p] = on[p] ? Bm[x][c] - s : 0.0f;
    o = fmaf(on[p] ? Em[i][x] : 0.0f, u[p], o);
  }
  return o;
}

// ------------------------------------------------------------- WY verify

constexpr int kWyCols = 32;     // value dimensions per workgroup
constexpr int kWyThreads = 512;  // 16 node slots x 32 value dimensions

// One workgroup (eight wavefronts) per (value head, 32 value dimensions).
// Every global load is issued at the start.  Wavefronts 0-3 then form one
// 32 x 32 product each (rows: nodes, zero past n): KK, QK, KS = K S0b^T and
// QS = Q S0b^T (S0b: the block's 32 state rows, as three bf16 pieces).  All
// threads then build the masked coefficients A, E and the right-hand sides
// B, and thread (node i, value dimension c) solves for u along i's own root
// path in registers (root first: each path node's ancestors are the path
// nodes before it) and forms o_i.  A node's u is recomputed, with the same
// operations in the same order, by every thread whose path holds it, so no
// barrier separates tree levels.
__global__ __launch_bounds__(kWyThreads) void gdn_wy_kernel(GdnArgs a) {
  constexpr int D = kGdnD, NC = kWyCols, NS = kWyThreads / NC;
  __shared__ int32_t par[kGdnMaxNodes];
  __shared__ uint32_t anc[kGdnMaxNodes];
  __shared__ float Gs[kGdnMaxNodes], bs[kGdnMaxNodes];
  __shared__ float prod[4][32][33];  // KK, QK, KS, QS
  __shared__ float Am[32][33], Em[32][33], Bm[32][33];
  __shared__ int ok_flag;
  const int nblk = D / NC;
  const int h = blockIdx.x / nblk, c0 = (blockIdx.x % nblk) * NC;
  const int kh = h / (a.hv / a.hk);
  const int n = a.n, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid & 31, slot = tid >> 5;  // nodes slot and slot + NS
  static_assert(NS * 2 == kGdnMaxNodes, "two nodes per thread");

  // ---- loads: v of this thread's nodes, g and beta, the product operands
  float vreg[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int i = slot + NS * m;
    // unconditional, clamped: nodes past n read node n - 1 and are never used
    vreg[m] = __uint_as_float((uint32_t)a.v[((int64_t)min(i, n - 1) * a.hv + h) * D + c0 + c] << 16);
  }
  const int tn = min(tid, n - 1);
  const float gv = a.g[tn * a.hv + h], bv = a.beta[tn * a.hv + h];  // lanes past n: never used
  // product operands (wavefronts 0-3): lane holds row lane % 32 (a node,
  // or a state row of the block) and k values 8 (lane / 32) .. +7 of each
  // 16-wide step; rows past n read node 0 and are zeroed
  const int r = lane & 31, hh = lane >> 5;
  const bool rn = r < n;
  const int rr = rn ? r : 0;
  uint4 xa[D / 16], yb[D / 16];
  float4 sb[D / 8];
  if (wave < 4) {
    const uint16_t* xrow = ((wave & 1) ? a.q : a.k) + ((int64_t)rr * a.hk + kh) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) xa[ks] = *(const uint4*)(xrow + 16 * ks);
    if (wave < 2) {
      const uint16_t* yrow = a.k + ((int64_t)rr * a.hk + kh) * D + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) yb[ks] = *(const uint4*)(yrow + 16 * ks);
    } else {
      const float* srow = a.state + ((int64_t)h * D + c0 + r) * D + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        sb[2 * ks] = *(const float4*)(srow + 16 * ks);
        sb[2 * ks + 1] = *(const float4*)(srow + 16 * ks + 4);
      }
    }
  }

  const bool ok = gdn_tree_masks(a.parents, n, par, anc, &ok_flag);
  if (blockIdx.x == 0 && tid == 0) *a.status = ok ? TVP_OK : TVP_ERR_TREE;
  if (tid < 64) {  // G_i over the root path in node order (lane j holds g_j); beta_i
    const uint32_t m = tid < kGdnMaxNodes ? anc[tid] : 0u;  // bits only below n
    float s = 0.0f;
    for (int j = 0; j < kGdnMaxNodes; ++j) {
      const float gj = __shfl(gv, j);
      if ((m >> j) & 1u) s += gj;
    }
    if (tid < kGdnMaxNodes) {
      Gs[tid] = s;
      bs[tid] = tid < n ? bv : 0.0f;
    }
  }
  if (wave < 4) {
    const uint4 z4 = make_uint4(0, 0, 0, 0);
    f32x16_t acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8_t A = __builtin_bit_cast(bf16x8_t, rn ? xa[ks] : z4);
      if (wave < 2) {
        const bf16x8_t B = __builtin_bit_cast(bf16x8_t, rn ? yb[ks] : z4);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc, 0, 0, 0);
      } else {
        bf16x8_t B0, B1, B2;
        split3(sb[2 * ks], sb[2 * ks + 1], B0, B1, B2);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B1, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B2, acc, 0, 0, 0);
      }
    }
    // D[row][col]: col = lane % 32, row = 8 (e / 4) + 4 (lane / 32) + e % 4
#pragma unroll
    for (int e = 0; e < 16; ++e) prod[wave][8 * (e >> 2) + 4 * hh + (e & 3)][r] = acc[e];
  }
  __syncthreads();
  // ---- masked coefficients and right-hand sides
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int i = slot + NS * m, j = c;  // entry (i, j) of A and E; B_i at value dimension c
    const bool in = ((anc[i] >> j) & 1u) != 0;
    const float d = in ? expf(Gs[i] - Gs[j]) : 0.0f;
    Am[i][j] = (in && j != i) ? bs[i] * d * prod[0][i][j] : 0.0f;
    Em[i][j] = in ? d * prod[1][i][j] : 0.0f;
    Bm[i][c] = i < n ? bs[i] * (vreg[m] - expf(Gs[i]) * prod[2][i][c]) : 0.0f;
  }
  __syncthreads();
  // ---- solve along the root path and output, thread (node i, column c),
  // unrolled to the tree's longest root path
  int maxlen = 1;
  for (int i = 0; i < n; ++i) maxlen = max(maxlen, __popc(anc[i]));
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int i = slot + NS * m;
    if (i >= n) continue;
    float o;
    if (maxlen <= 9) o = wy_path<9>(anc[i], i, c, Am, Em, Bm);
    else if (maxlen <= 16) o = wy_path<16>(anc[i], i, c, Am, Em, Bm);
    else o = wy_path<kGdnMaxNodes>(anc[i], i, c, Am, Em, Bm);
    a.out[((int64_t)i * a.hv + h) * D + c0 + c] = (uint16_t)f32_to_bf16(o + expf(Gs[i]) * prod[3][i][c]);
  }
}

// ------------------------------------------------------------ path verify

// One workgroup (256 threads, two per state row) per (value head, node);
// only workgroups whose node is a leaf work.  The workgroup replays the
// leaf's root path from the committed state and writes the output of every
// path node whose first leaf (the smallest-index leaf below it) is this one,
// so each output is written exactly once.
constexpr int kPairThreads = 2 * kGdnD;
__global__ __launch_bounds__(kPairThreads) void gdn_path_kernel(GdnArgs a) {
  constexpr int D = kGdnD, C8 = D / 8;
  __shared__ int32_t par[kGdnMaxNodes];
  __shared__ uint32_t anc[kGdnMaxNodes];
  __shared__ float ks[kGdnMaxNodes][D], qs[kGdnMaxNodes][D], vs[kGdnMaxNodes][D];
  __shared__ float gl[kGdnMaxNodes], bl[kGdnMaxNodes];
  __shared__ int32_t owner[kGdnMaxNodes];
  __shared__ uint32_t leaves;
  __shared__ int ok_flag;
  const int h = blockIdx.x / a.n, leaf = blockIdx.x % a.n;
  const int kh = h / (a.hv / a.hk);
  const int n = a.n, tid = threadIdx.x, row = tid >> 1, hf = (tid & 1) * kHalf;
  const bool ok = gdn_tree_masks(a.parents, n, par, anc, &ok_flag);
  if (blockIdx.x == 0 && tid == 0) *a.status = ok ? TVP_OK : TVP_ERR_TREE;
  if (tid < 64) {  // leaves: nodes that are nobody's parent
    bool is_leaf = tid < n;
    if (tid < kGdnMaxNodes)
      for (int j = tid + 1; j < n; ++j) is_leaf = is_leaf && par[j] != tid;
    const uint64_t b = __ballot(is_leaf);
    if (tid == 0) leaves = (uint32_t)b;
  }
  __syncthreads();
  if (!((leaves >> leaf) & 1u)) return;  // uniform over the workgroup
  // the half row of this thread, then every node's key, query and value row
  // (16-byte loads), decay and strength, all loads in flight together
  float S[kHalf];
  load_half(a.state + ((int64_t)h * D + row) * D + hf, S);
  // (loads unconditional with clamped indices, stores guarded: a load inside
  // a branch is waited for at the branch's end)
  constexpr int NIT = kGdnMaxNodes * C8 / kPairThreads;
  uint4 kx[NIT], qx[NIT], vx[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int e = tid + kPairThreads * it, j = min(e / C8, n - 1), c8 = e % C8;
    kx[it] = *(const uint4*)(a.k + ((int64_t)j * a.hk + kh) * D + 8 * c8);
    qx[it] = *(const uint4*)(a.q + ((int64_t)j * a.hk + kh) * D + 8 * c8);
    vx[it] = *(const uint4*)(a.v + ((int64_t)j * a.hv + h) * D + 8 * c8);
  }
  const int tn = min(tid, n - 1);
  const float gval = a.g[tn * a.hv + h], bval = a.beta[tn * a.hv + h];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int e = tid + kPairThreads * it, j = e / C8, c8 = e % C8;
    if (j < n) {
      unpack8(kx[it], &ks[j][8 * c8]);
      unpack8(qx[it], &qs[j][8 * c8]);
      unpack8(vx[it], &vs[j][8 * c8]);
    }
  }
  if (tid < n) {
    gl[tid] = expf(gval);
    bl[tid] = bval;
  }
  if (tid < kGdnMaxNodes) {  // the first leaf below each node writes its output
    int o = kGdnMaxNodes;
    for (int l = 0; l < n && o == kGdnMaxNodes; ++l)
      if (((leaves >> l) & 1u) && ((anc[l] >> tid) & 1u)) o = l;
    owner[tid] = o;
  }
  __syncthreads();
  for (uint32_t mk = anc[leaf]; mk; mk &= mk - 1) {  // root first (ancestors have smaller indices)
    const int j = __ffs(mk) - 1;
    pair_update(S, ks[j] + hf, gl[j], bl[j], vs[j][row]);
    if (owner[j] == leaf) {  // uniform
      const float o = pair_dot(S, qs[j] + hf);
      if (hf == 0) a.out[((int64_t)j * a.hv + h) * D + row] = (uint16_t)f32_to_bf16(o);
    }
  }
}

// ------------------------------------------------------------------ commit

struct GdnCommitArgs {
  float* state;        // [L][hv][dv][dk], updated in place
  const uint16_t* k;   // [L][n][hk][dk]
  const uint16_t* v;   // [L][n][hv][dv]
  const float* g;      // [L][n][hv]
  const float* beta;   // [L][n][hv]
  int n, hk, hv;
  const int32_t* path;        // accepted nodes, root first
  const int32_t* n_accepted;  // path holds n_accepted + 1 nodes
  const int32_t* status;
};

// One workgroup (256 threads, two per state row) per (layer, value head):
// the accepted path's updates applied in order to the committed state.  Does
// nothing unless *status is TVP_OK and the path is a valid node list.
__global__ __launch_bounds__(kPairThreads) void gdn_commit_kernel(GdnCommitArgs a) {
  constexpr int D = kGdnD, C8 = D / 8;
  __shared__ float ks[kGdnMaxNodes][D], vs[kGdnMaxNodes][D];
  __shared__ float gl[kGdnMaxNodes], bl[kGdnMaxNodes];
  __shared__ int32_t pj[kGdnMaxNodes];
  __shared__ int len;
  const int layer = blockIdx.x / a.hv, h = blockIdx.x % a.hv;
  const int kh = h / (a.hv / a.hk);
  const int tid = threadIdx.x, n = a.n, row = tid >> 1, hf = (tid & 1) * kHalf;
  if (tid == 0) {
    const int na = *a.n_accepted;
    int m = (*a.status == TVP_OK && na >= 0 && na < n) ? na + 1 : 0;
    for (int i = 0; i < m; ++i) {
      const int j = a.path[i];
      if (j < 0 || j >= n) m = 0;
      else pj[i] = j;
    }
    len = m;
  }
  __syncthreads();
  const int m = len;
  if (m == 0) return;  // uniform
  const int64_t lk = (int64_t)layer * n * a.hk * D, lv = (int64_t)layer * n * a.hv * D;
  const int64_t lg = (int64_t)layer * n * a.hv;
  float* dst = a.state + (((int64_t)layer * a.hv + h) * D + row) * D + hf;
  float S[kHalf];
  load_half(dst, S);
  // (loads unconditional with clamped indices, stores guarded)
  constexpr int NIT = kGdnMaxNodes * C8 / kPairThreads;
  uint4 kx[NIT], vx[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int e = tid + kPairThreads * it, j = pj[min(e / C8, m - 1)], c8 = e % C8;
    kx[it] = *(const uint4*)(a.k + lk + ((int64_t)j * a.hk + kh) * D + 8 * c8);
    vx[it] = *(const uint4*)(a.v + lv + ((int64_t)j * a.hv + h) * D + 8 * c8);
  }
  const int jt = pj[min(tid, m - 1)];
  const float gval = a.g[lg + jt * a.hv + h], bval = a.beta[lg + jt * a.hv + h];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int e = tid + kPairThreads * it, i = e / C8, c8 = e % C8;
    if (i < m) {
      unpack8(kx[it], &ks[i][8 * c8]);
      unpack8(vx[it], &vs[i][8 * c8]);
    }
  }
  if (tid < m) {
    gl[tid] = expf(gval);
    bl[tid] = bval;
  }
  __syncthreads();
  for (int i = 0; i < m; ++i) pair_update(S, ks[i] + hf, gl[i], bl[i], vs[i][row]);
#pragma unroll
  for (int c = 0; c < kHalf / 4; ++c) ((float4*)dst)[c] = make_float4(S[4 * c], S[4 * c + 1], S[4 * c + 2], S[4 * c + 3]);
}

static int gdn_check(const void* q, const void* k, const void* v, const void* g, const void* beta, const void* state,
                     const void* parents, const void* out, const void* status, int32_t n, int32_t hk, int32_t hv,
                     int32_t dk, int32_t dv) {
  if (!q || !k || !v || !g || !beta || !state || !parents || !out || !status) return TVP_ERR_ARG;
  if (n < 1 || n > kGdnMaxNodes || hk < 1 || hv < 1 || hv % hk || hv > 4096) return TVP_ERR_SHAPE;
  if (dk != kGdnD || dv != kGdnD) return TVP_ERR_SHAPE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)state) % 16) return TVP_ERR_ARG;
  return TVP_OK;
}

}  // namespace tvp

using namespace tvp;

extern "C" {

int gdn_tree_verify(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g, const float* beta,
                    const float* state, const int32_t* parents, int32_t n, int32_t hk, int32_t hv, int32_t dk,
                    int32_t dv, uint16_t* out, int32_t* status, hipStream_t stream) {
  int st = gdn_check(q, k, v, g, beta, state, parents, out, status, n, hk, hv, dk, dv);
  if (st) return st;
  GdnArgs a{q, k, v, g, beta, state, parents, n, hk, hv, out, status};
  gdn_wy_kernel<<<dim3((unsigned)(hv * (kGdnD / kWyCols))), dim3(kWyThreads), 0, stream>>>(a);
  TVP_LAUNCH_CHECK();
  return TVP_OK;
}

int gdn_path_verify(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g, const float* beta,
                    const float* state, const int32_t* parents, int32_t n, int32_t hk, int32_t hv, int32_t dk,
                    int32_t dv, uint16_t* out, int32_t* status, hipStream_t stream) {
  int st = gdn_check(q, k, v, g, beta, state, parents, out, status, n, hk, hv, dk, dv);
  if (st) return st;
  GdnArgs a{q, k, v, g, beta, state, parents, n, hk, hv, out, status};
  gdn_path_kernel<<<dim3((unsigned)(hv * n)), dim3(kPairThreads), 0, stream>>>(a);
  TVP_LAUNCH_CHECK();
  return TVP_OK;
}

int gdn_commit(float* state, const uint16_t* k, const uint16_t* v, const float* g, const float* beta,
               int32_t n_layers, int32_t n, int32_t hk, int32_t hv, int32_t dk, int32_t dv, const int32_t* path,
               const int32_t* n_accepted, const int32_t* status, hipStream_t stream) {
  if (!state || !k || !v || !g || !beta || !path || !n_accepted || !status) return TVP_ERR_ARG;
  if (n_layers < 1 || n_layers > 1024 || n < 1 || n > kGdnMaxNodes || hk < 1 || hv < 1 || hv % hk || hv > 4096)
    return TVP_ERR_SHAPE;
  if (dk != kGdnD || dv != kGdnD) return TVP_ERR_SHAPE;
  if (((uintptr_t)state | (uintptr_t)k | (uintptr_t)v) % 16) return TVP_ERR_ARG;
  GdnCommitArgs a{state, k, v, g, beta, n, hk, hv, path, n_accepted, status};
  gdn_commit_kernel<<<dim3((unsigned)(n_layers * hv)), dim3(kPairThreads), 0, stream>>>(a);
  TVP_LAUNCH_CHECK();
  return TVP_OK;
}

}  // extern "C"
