// Tree preparation (ancestor masks, positions, cache slots, validation) and
// tree-masked attention for gfx950.
//
// SpecPilot summary (onedev.kr), section 무엇인가: the target checks all draft
// tokens in one forward pass, so each node must see the committed context and
// exactly its own root path; section 전제와 한계 names tree attention as one
// of the places where reduction order may flip near-ties.
//
// Design: per (request, kv head, 32-row block, key split) one workgroup of
// eight wavefronts.  A row is (query head kv_head*G + gq, node i) at row
// gq * n + i.  Each wavefront streams its own 32-key blocks of the split
// through its own LDS tiles (fully coalesced 16-byte loads, K and V
// row-major, XOR-swizzled per row), with the next blocks in flight in
// registers.  Scores are computed as S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 so each lane owns one query row, masked with the
// node's 64-bit ancestor mask and folded into an online softmax; P V is
// accumulated with the same MFMA, its V^T operand read straight from the
// row-major V tile with the LDS transpose read (ds_read_b64_tr_b16), and P
// applied as a sum of two bf16 pieces.  The wavefronts' (max, sum, O)
// are combined in LDS in a fixed order; with several splits, each split's
// (max, sum, O) goes out in the accumulator's register layout (coalesced
// 256-byte stores, written through to the device's coherence point) and the
// last split of a row block to arrive, counted on a device-scope atomic,
// sums them all in split order, so the result is deterministic.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "internal.h"

namespace tvp {

// One workgroup (64 threads) per request.  Nodes of request r are
// node_ptr[r] .. node_ptr[r+1]-1 (at most 64); parents are request-local.
__global__ __launch_bounds__(64) void tree_prep_kernel(const int32_t* __restrict__ parents, ReqInfo ri,
                                                       int32_t s_req, uint64_t* __restrict__ anc,
                                                       int32_t* __restrict__ pos,
                                                       int32_t* __restrict__ slot,
                                                       int32_t* __restrict__ status,
                                                       uint32_t* __restrict__ cnt, int ncnt) {
  __shared__ int32_t par[64];
  const int r = blockIdx.x, i = threadIdx.x;
  // the in-launch hand-overs' arrival counters start at zero
  for (int c = r * 64 + i; c < ncnt; c += gridDim.x * 64) cnt[c] = 0u;
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
  int units, units8;  // (request, kv head, split) units; rounded up to a multiple of 8
  float scale_log2;
  float* po;
  float* pm;
  float* pl;
  // arrival counters of the key splits, [request][kv head][kAttnRowBlocks]:
  // zero before the launch, and left at zero by the split that merges
  uint32_t* cnt;
  int row_blocks;  // 32-row blocks per (request, kv head)
  // request of each unit slot: longest key range first (batched passes);
  // 32-bit entries, so a uniform index reads one with a scalar load
  int32_t order[kMaxReq];
  int grouped;            // block order: units in groups of 8, row blocks inner (batched passes)
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

// Both halves of a wavefront see {x[l], x[l ^ 32]} after one
// v_permlane32_swap (a VALU op, no LDS round trip); the reductions below
// combine them lower half first, so lanes l and l ^ 32 get identical bits.
__device__ inline float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Word 3 of a raw buffer resource on gfx9 (32-bit data format, no swizzle):
// a load whose per-lane offset (plus the instruction's immediate offset)
// reaches num_records returns zero without touching memory.
constexpr int kBufWord3 = 0x00020000;

// Compiler fence for one wavefront's LDS accesses (they complete in order).
__device__ inline void lds_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// Wavefronts per attention workgroup (two per SIMD).
constexpr int kAttnWaves = 8;

// One workgroup per (request, kv head, 32-row block, key split); its NW
// wavefronts stream disjoint 32-key blocks of the split (wavefront w takes
// blocks w, w + NW, ...) with no workgroup barrier until the end.  Each
// wavefront stages its blocks through its own LDS tiles, keeps the next
// NPF - 1 blocks in flight in registers and runs its own online softmax; the
// NW (max, sum, O) states are combined in LDS in wavefront order at the end.
// Two wavefronts per SIMD hide each other's MFMA, LDS and exp latencies.
template <int D, int NPF>
__global__ __launch_bounds__(kAttnWaves * 64) void tree_attn_kernel(AttnArgs a) {
  constexpr int NW = kAttnWaves;
  constexpr int KB = 32;        // keys per block
  constexpr int CH = D / 8;     // 16-byte chunks per key row
  constexpr int NDB = D / 32;   // d blocks of the P V product
  constexpr int PER = KB * CH / 64;  // 16-byte pieces per lane per block (K or V)
  constexpr int NACC = NDB * 16;     // accumulator registers per lane
  // per wavefront: V [key][chunk ^ v_swz(key)]; at the end the same memory
  // holds the wavefronts' O
  __shared__ uint4 tiles[NW][2][KB * CH];
  __shared__ uint4 qs[32 * CH];    // Q of the row block [row][chunk ^ (row % CH)]
  __shared__ float ml[NW][2][32];  // per wavefront and row: exponent base (a raw score), sum
  static_assert(sizeof(tiles) >= NW * NACC * 64 * sizeof(float), "O of all wavefronts fits the tiles");

  // block -> (row block, unit).  The row blocks of one (request, kv head,
  // split) are a multiple of 8 apart, so they run on one XCD and share its
  // L2.  Batched passes take units in groups of 8 with all their row blocks
  // before the next group (with the longest requests first, their work all
  // starts first); one request takes row block by row block.
  const int u = a.grouped ? (blockIdx.x / (8 * a.row_blocks)) * 8 + blockIdx.x % 8 : blockIdx.x % a.units8;
  const int rb = a.grouped ? (blockIdx.x / 8) % a.row_blocks : blockIdx.x / a.units8;
  if (u >= a.units) return;
  const int split = u % a.max_splits;
  const int kh = (u / a.max_splits) % a.hkv;
  const int r = a.order[u / (a.max_splits * a.hkv)];
  const int L = a.ri.ctx_len[r], nb = a.ri.node_ptr[r], n = a.ri.node_ptr[r + 1] - nb;
  const int T = L + n, R = a.G * n;
  const int nsplit = (T + a.kr - 1) / a.kr;
  if (split >= nsplit || rb * 32 >= R) return;
  const int k0 = split * a.kr, k1 = min(T, k0 + a.kr);
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: block offsets stay scalar
  const int row = rb * 32 + (lane & 31);
  const bool row_ok = row < R;
  const int gq = row_ok ? row / n : 0, node = row_ok ? row % n : 0;
  const int64_t cbase = (int64_t)kh * a.s_stride + (int64_t)r * a.s_req;  // slot 0 of this request/head
  const uint16_t* kbase = a.kc + cbase * D;
  const uint16_t* vbase = a.vc + cbase * D;
  uint4* vs = tiles[wave][0];

  // Q of the row block (zero rows past R), one 16-byte piece per thread,
  // loaded first and stored to LDS once the first K/V loads are in flight;
  // the B operand of the score product is read from there: lane holds
  // q[row][16 ds + 8 h .. +7]
  static_assert(32 * CH <= NW * 64, "one Q piece per thread");
  uint4 qv = make_uint4(0, 0, 0, 0);
  const int qr = tid / CH, qc = tid % CH;
  if (tid < 32 * CH && rb * 32 + qr < R) {
    const int rr = rb * 32 + qr;
    qv = *(const uint4*)(a.q + ((int64_t)(nb + rr % n) * a.hq + kh * a.G + rr / n) * D + 8 * qc);
  }
  const uint64_t anc = row_ok ? a.anc[nb + node] : 0ull;
  const int klim = row_ok ? k1 : 0;  // keys below klim may be visible to this lane's row

  float m_run = -INFINITY, l_run = 0.0f;
  f32x16_t o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.0f;

  const int nblk = (k1 - k0 + KB - 1) / KB;                   // blocks of the split
  const int nbw = nblk > wave ? (nblk - wave + NW - 1) / NW : 0;  // blocks of this wavefront
  auto key0_of = [&](int i) { return k0 + (wave + NW * i) * KB; };

  // Block i of this wavefront into register stage st, with buffer loads whose
  // range ends at the split's last key: keys past it (the split's ragged end,
  // or a whole placeholder block past the wavefront's last) read as zero
  // without touching memory, their scores are masked, and every path keeps
  // the same number of loads in flight.  The block's byte offset is part of
  // the per-lane offset, which is the operand the hardware checks against the
  // range (the scalar offset operand is not checked), so no key at or past
  // the split's end is ever fetched.  K arrives directly in the MFMA
  // A-operand layout (lane: key lane % 32, 16-byte piece 2 ds + h of its
  // row); V with CH consecutive lanes reading one 2*D-byte row, for the LDS
  // tile.
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t kpre[NPF][PER], vpre[NPF][PER];
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, k1 * D * 2, kBufWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, k1 * D * 2, kBufWord3);
  const int koff = (lane & 31) * D * 2 + 16 * h;
  auto fetch = [&](int i, int st) __attribute__((always_inline)) {
    const int boff = key0_of(i) * D * 2;
    const int kv = koff + boff, vv = 16 * lane + boff;
#pragma unroll
    for (int ds = 0; ds < PER; ++ds)
      kpre[st][ds] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(krs, kv + 32 * ds, 0, 0));
#pragma unroll
    for (int it = 0; it < PER; ++it)
      vpre[st][it] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vrs, vv + 1024 * it, 0, 0));
  };
  auto stash = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int pc = lane + 64 * it;
      const int key = pc / CH, c = pc % CH;
      *(u32x4_t*)&vs[key * CH + (c ^ v_swz<D>(key))] = vpre[st][it];
    }
  };
  // transpose-read geometry: in each 16-lane group, source lane s points at
  // key row (s / 4) and 4 d-columns (s % 4) * 4; lane i then receives
  // V[key0 + 0..3][d0 + i]
  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr_key = 4 * h + (s16 >> 2);
  const int tr_d = 16 * (g16 & 1) + 4 * (s16 & 3);
  const char* vs_bytes = (const char*)vs;

  // scores S^T[key][row] of one block, online softmax, P V
  auto compute = [&](int i, int st) __attribute__((always_inline)) {
    f32x16_t sc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sc[v] = 0.0f;
    {
      const int qrow = lane & 31;
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, kpre[st][ds]);
        const bf16x8_t B = __builtin_bit_cast(bf16x8_t, qs[qrow * CH + ((2 * ds + h) ^ (qrow % CH))]);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, sc, 0, 0, 0);
      }
    }
    // raw scores; the 1/sqrt(d) scale (in log2 units) is applied inside the
    // exponent.  Blocks of context keys only need no mask.
    float mloc = -INFINITY;
    const int kb0 = key0_of(i);
    if (kb0 + KB <= min(L, k1)) {
#pragma unroll
      for (int v = 0; v < 16; ++v) mloc = fmaxf(mloc, sc[v]);
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kb0 + 8 * (v >> 2) + 4 * h + (v & 3);
        const bool anc_ok = ((anc >> ((key - L) & 63)) & 1ull) != 0;
        const bool vis = (key < klim) & ((key < L) | anc_ok);  // no branches
        sc[v] = vis ? sc[v] : -INFINITY;
        mloc = fmaxf(mloc, sc[v]);
      }
    }
    mloc = xor32_max(mloc);
    // The exponent base m_run moves only when a row's maximum exceeds it by
    // more than 8 in log2 units (always at the row's first visible key):
    // the weights stay below 2^8, exact to the same relative precision in
    // fp32, and the rescale of O is skipped on almost every block.  O, the
    // sum and the recorded maximum all refer to the same base, so the result
    // is the same softmax.
    const bool grow = (mloc - m_run) * a.scale_log2 > 8.0f;
    const float m_new = grow ? mloc : m_run;
    const float base = m_new == -INFINITY ? 0.0f : m_new;
    const float nbs = -base * a.scale_log2;
    const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - base) * a.scale_log2) : 1.0f;
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
    lsum = xor32_sum(lsum);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
    if (__ballot(grow)) {  // the base moved for some row: rescale
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
    }
    // O^T[d][row] += V^T[d][key] P^T[key][row]; MFMA q of the block covers
    // keys 16 q + 8 (i/4) + 4 h + i%4 for k-index 8 h + i.
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const bf16x8_t B = __builtin_bit_cast(bf16x8_t, make_uint4(pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]));
      const bf16x8_t Bl = __builtin_bit_cast(bf16x8_t, make_uint4(pl[4 * q], pl[4 * q + 1], pl[4 * q + 2], pl[4 * q + 3]));
      const int r1 = 16 * q + tr_key, r2 = r1 + 8;
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
  };

  // The stage index is a compile-time constant (the register ring never
  // moves) and the main loop has no data-dependent branch around its loads,
  // so each stash waits only for its own block.  One wavefront's LDS
  // operations complete in order; the fences keep the compiler from moving
  // a stash across the previous block's reads.
  auto stage = [&](int i, auto stc, bool do_fetch) __attribute__((always_inline)) {
    constexpr int st = decltype(stc)::value;
    lds_fence();
    stash(st);
    lds_fence();
    if (do_fetch) fetch(i + NPF - 1, (st + NPF - 1) % NPF);
    compute(i, st);
  };
#pragma unroll
  for (int st = 0; st < NPF - 1; ++st) fetch(st, st);
  if (tid < 32 * CH) qs[qr * CH + (qc ^ (qr % CH))] = qv;
  __syncthreads();  // Q in LDS
  int c0 = 0;
  for (; c0 + NPF <= nbw; c0 += NPF) {
    stage(c0, std::integral_constant<int, 0>{}, true);
    if constexpr (NPF > 1) stage(c0 + 1, std::integral_constant<int, 1 % NPF>{}, true);
    if constexpr (NPF > 2) stage(c0 + 2, std::integral_constant<int, 2 % NPF>{}, true);
    if constexpr (NPF > 3) stage(c0 + 3, std::integral_constant<int, 3 % NPF>{}, true);
  }
  // the last nbw % NPF blocks are already in flight
  if constexpr (NPF > 1)
    if (c0 < nbw) stage(c0, std::integral_constant<int, 0>{}, false);
  if constexpr (NPF > 2)
    if (c0 + 1 < nbw) stage(c0 + 1, std::integral_constant<int, 1 % NPF>{}, false);
  if constexpr (NPF > 3)
    if (c0 + 2 < nbw) stage(c0 + 2, std::integral_constant<int, 2 % NPF>{}, false);

  // combine the wavefronts' states (wavefront order) in LDS
  __syncthreads();
  float* ob = (float*)&tiles[0][0][0];  // [wave][db * 16 + v][lane]
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) ob[(wave * NACC + db * 16 + v) * 64 + lane] = o[db][v];
  if (h == 0) {
    ml[wave][0][lane & 31] = m_run;
    ml[wave][1][lane & 31] = l_run;
  }
  __syncthreads();
  const int64_t pbase = ((int64_t)kh * a.max_splits + split) * a.rows_total + a.pr.prow[r] + rb * 32;
  // every element of this thread has lane tid % 64, hence row tid % 32
  const int ln = lane, rw = lane & 31;
  float mx = ml[0][0][rw];
#pragma unroll
  for (int w = 1; w < NW; ++w) mx = fmaxf(mx, ml[w][0][rw]);
  const float bse = mx == -INFINITY ? 0.0f : mx;
  float wt[NW], den = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float mw = ml[w][0][rw];
    wt[w] = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((mw - bse) * a.scale_log2);
    den += ml[w][1][rw] * wt[w];
  }
  static_assert(NACC % NW == 0, "whole elements per thread");
#pragma unroll
  for (int it = 0; it < NACC / NW; ++it) {
    const int dv = wave + NW * it;  // element (dv, lane) of the block in accumulator layout
    const int e = dv * 64 + ln;
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) acc += ob[(w * NACC + dv) * 64 + ln] * wt[w];
    const int rr = rb * 32 + rw;
    if (nsplit == 1) {  // normalise and store
      if (rr < R) {
        const int db = dv >> 4, v = dv & 15;
        const int dd = db * 32 + 8 * (v >> 2) + 4 * (ln >> 5) + (v & 3);
        const int g2 = rr / n, nd = rr % n;
        const float inv = den > 0.0f ? 1.0f / den : 0.0f;
        a.out[attn_out_index<D>(a, nb + nd, (kh * a.G + g2) * D + dd)] = (uint16_t)f32_to_bf16(acc * inv);
      }
    } else {  // partial rows [kv head][split][padded rows], accumulator layout
      st_dev(a.po + pbase * D + e, acc);
      if (dv == 0 && ln < 32) {  // the exponent base is a raw score (unscaled)
        st_dev(a.pm + pbase + rw, mx);
        st_dev(a.pl + pbase + rw, den);
      }
    }
  }
  if (nsplit == 1) return;

  // The split of this row block that arrives last merges all of them.
  __shared__ int s_last;
  if (!arrive_last(a.cnt + ((int64_t)r * a.hkv + kh) * kAttnRowBlocks + rb, (uint32_t)nsplit, &s_last)) return;

  // Merge of the row block's splits, in split order with a running exponent
  // base (one pass, so the loads of up to 8 splits are in flight together).
  // This thread's elements are the ones it stored above, all of row rw;
  // every value is read back from the partials, this split's included, so the
  // result does not depend on which split merges.
  const int64_t hb = (int64_t)kh * a.max_splits * a.rows_total + a.pr.prow[r] + rb * 32;  // split 0
  constexpr int NE = NACC / NW;  // elements per thread
  float gb = -INFINITY, gden = 0.0f, macc[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) macc[i] = 0.0f;
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    float pmv[8], plv[8], pv[8][NE];
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // past the last split: its loads repeated, weight zero
      const int64_t sb = hb + (int64_t)min(s0 + j, nsplit - 1) * a.rows_total;
      const float m = ld_dev(a.pm + sb + rw);
      pmv[j] = s0 + j < nsplit ? m : -INFINITY;
      plv[j] = ld_dev(a.pl + sb + rw);
#pragma unroll
      for (int i = 0; i < NE; ++i) pv[j][i] = ld_dev(a.po + sb * D + (wave + NW * i) * 64 + ln);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (pmv[j] == -INFINITY) continue;  // no visible key of this row in the split
      if (pmv[j] > gb) {  // raise the base (maxima are raw scores)
        const float f = gb == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((gb - pmv[j]) * a.scale_log2);
        gden *= f;
#pragma unroll
        for (int i = 0; i < NE; ++i) macc[i] *= f;
        gb = pmv[j];
      }
      const float wj = __builtin_amdgcn_exp2f((pmv[j] - gb) * a.scale_log2);
      gden += plv[j] * wj;
#pragma unroll
      for (int i = 0; i < NE; ++i) macc[i] += pv[j][i] * wj;
    }
  }
  const float ginv = gden > 0.0f ? 1.0f / gden : 0.0f;
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int dv = wave + NW * i;
    const int rr = rb * 32 + rw;
    if (rr < R) {
      const int db = dv >> 4, v = dv & 15;
      const int dd = db * 32 + 8 * (v >> 2) + 4 * (ln >> 5) + (v & 3);
      const int g2 = rr / n, nd = rr % n;
      a.out[attn_out_index<D>(a, nb + nd, (kh * a.G + g2) * D + dd)] = (uint16_t)f32_to_bf16(macc[i] * ginv);
    }
  }
}

// Key splits are sized so that one launch has about this many workgroups
// (one per compute unit).
constexpr int kAttnTargetGroups = 256;
// Blocks of 32 keys per wavefront kept in flight (including the one in LDS).
constexpr int kAttnStages = 2;

struct AttnPlan {
  int kr, max_splits, rows_total, row_blocks;
  size_t off_po, off_pm, off_pl, bytes;
};

// max_keys: largest ctx_len + n over the requests; r_max: largest G * n;
// rows_total: partial rows over all requests (each request's G * n rounded
// up to a multiple of 32).  A split is a multiple of 32 keys (its 32-key
// blocks dealt to the wavefronts in turn), at most 64 splits.
static AttnPlan attn_plan(int hkv, int d, int r_max, int rows_total, int max_keys, int n_req) {
  AttnPlan p{};
  p.row_blocks = (r_max + 31) / 32;
  const int target = std::max(1, kAttnTargetGroups / std::max(1, n_req * hkv * p.row_blocks));
  // whole 32-key blocks, at least one per wavefront: sized in blocks rather
  // than in one block per wavefront, the 4B-like step (6 -> 8 splits, 192 ->
  // 256 workgroups) ran 2.9% faster and the 8-node step (8 -> 15 splits)
  // 1.2%; with fewer keys than one block per wavefront (one-node decoding:
  // 26 splits of 160 keys) decoding ran 1.9% slower, hence the floor
  p.kr = std::max(32 * kAttnWaves, 32 * (int)ceil_div(std::max(max_keys, 1), (int64_t)32 * target));
  while (max_keys > 64 * p.kr) p.kr *= 2;  // at most 64 splits (the merge reads 8 per pass)
  p.max_splits = max_keys > 0 ? (max_keys + p.kr - 1) / p.kr : 1;
  // A last split under a quarter of the others (one-node decoding over 4096
  // context keys: 4097 keys, 17 splits of 256 with one key in the last) is
  // folded into the others, each grown by whole 32-key blocks (15 splits of
  // 288 keys): measured 0.6-0.9% faster verify steps at 1, 8 and 16 nodes.
  if (p.max_splits > 1 && max_keys - (p.max_splits - 1) * p.kr < p.kr / 4) {
    p.kr = 32 * (int)ceil_div(ceil_div(max_keys, p.max_splits - 1), 32);
    p.max_splits = (max_keys + p.kr - 1) / p.kr;
  }
  p.rows_total = rows_total;
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
                     int32_t* pos, int32_t* slot, int32_t* status, uint32_t* cnt, int ncnt,
                     hipStream_t stream) {
  tree_prep_kernel<<<dim3(ri.n_req), dim3(64), 0, stream>>>(parents, ri, s_req, anc, pos, slot, status, cnt,
                                                            ncnt);
  TVP_LAUNCH_CHECK();
  return TVP_OK;
}

int launch_tree_attention(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, int64_t s_stride,
                          const ReqInfo& ri, int32_t s_req, const uint64_t* anc, int hq, int hkv, int d,
                          int r_max, int max_keys, uint16_t* out, int out_packed, void* scratch,
                          size_t scratch_bytes, uint32_t* cnt, hipStream_t stream) {
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
  a.cnt = cnt;
  a.po = (float*)(sb + p.off_po);
  a.pm = (float*)(sb + p.off_pm);
  a.pl = (float*)(sb + p.off_pl);
  a.out = out;
  a.out_packed = out_packed;
  a.row_blocks = p.row_blocks;
  // Workgroups start in index order and run for a time proportional to
  // their request's key range, so the longest requests go first (the tail of
  // the launch is then the shortest work).  Ties keep request order.
  for (int i = 0; i < n_req; ++i) a.order[i] = i;
  std::stable_sort(a.order, a.order + n_req, [&](int32_t x, int32_t y) {
    return ri.ctx_len[x] + (ri.node_ptr[x + 1] - ri.node_ptr[x]) > ri.ctx_len[y] + (ri.node_ptr[y + 1] - ri.node_ptr[y]);
  });
  a.grouped = n_req > 1 ? 1 : 0;
  a.units = n_req * hkv * p.max_splits;
  a.units8 = (int)align_up((size_t)a.units, 8);
  const dim3 grid((unsigned)(a.units8 * p.row_blocks));
  if (d == 128) {
    tree_attn_kernel<128, kAttnStages><<<grid, dim3(kAttnWaves * 64), 0, stream>>>(a);
  } else if (d == 64) {
    tree_attn_kernel<64, kAttnStages><<<grid, dim3(kAttnWaves * 64), 0, stream>>>(a);
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

// Standalone layout of the tree_attention workspace (no initial contents
// needed):
//   [0, 512)        anc u64 [64]
//   [512, 1024)     pos/slot i32 [64] each
//   [1024, ...)     arrival counters u32 [attention_counters(1, hkv)] (cleared by tree preparation)
//   then            attention partials
static size_t ta_layout(int32_t n, int32_t hq, int32_t hkv, int32_t d, int32_t max_keys, size_t* off_part) {
  const size_t off = align_up(64 * 8 + 2 * 64 * 4 + (size_t)attention_counters(1, std::max(hkv, 1)) * 4, 256);
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
  uint64_t* anc = (uint64_t*)w;
  int32_t* pos = (int32_t*)(w + 64 * 8);
  int32_t* slot = pos + 64;
  ReqInfo ri{};
  ri.n_req = 1;
  ri.ctx_len[0] = ctx_len;
  ri.node_ptr[0] = 0;
  ri.node_ptr[1] = n;
  uint32_t* cnt = (uint32_t*)(w + 64 * 8 + 2 * 64 * 4);
  int st = launch_tree_prep(parents, ri, 0, anc, pos, slot, status, cnt, attention_counters(1, hkv), stream);
  if (st != TVP_OK) return st;
  return launch_tree_attention(q, k_cache, v_cache, s_stride, ri, 0, anc, hq, hkv, d, (hq / hkv) * n,
                               ctx_len + n, out, 0, w + offp, ws_bytes - offp, cnt, stream);
}

}  // extern "C"
