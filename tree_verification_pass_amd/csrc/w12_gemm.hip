// Skinny W12 GEMM for gfx950: Y[m][n] = X[m][k] . W[n][k]^T, W streamed as
// 12-bit records and decoded in registers (SpecPilot summary, section
// 무엇과 다른가: the GEMM decodes records in registers so the decode hides
// behind the weight stream; stream-K keeps it deterministic).
//
// MI355X design (not the page's Hopper kernel):
//  * Skinny kernel (up to 32 rows): each wavefront streams whole packed tile
//    blocks (32 channels x 64 k = 3072 B, lane-contiguous 16-byte loads) of
//    one or two tiles through a register ring and reads its activation
//    fragments from the packed activation layout (they stay in L2); a
//    workgroup's wavefronts split K and meet in LDS in wavefront order.
//  * Wide kernel (33..192 rows): a workgroup's four wavefronts walk the same
//    K blocks, one tile each, and share each 64-column block of X through a
//    double-buffered LDS tile.
//  * Decode: 4 VALU ops per pair of weights (rotate, mask, byte spread, add)
//    into bf16 halfwords; the decoded 32x64 tile goes through the wave's LDS
//    scratch so escape values (about 1% of weights) are patched with one
//    16-bit LDS store each, then the fragments feed v_mfma_f32_32x32x16_bf16
//    (m > 16) or v_mfma_f32_16x16x32_bf16 (m <= 16).
//  * K split over workgroups: fp32 partial sums go to the workspace and are
//    added in split order, so results are bitwise reproducible: by the next
//    launch (the wide kernel's fix-up, or the fused residual + RMSNorm), or,
//    for the K slices of a skinny launch's remaining groups, inside the
//    launch by the slice that arrives last on a device-scope counter (the
//    sums travel as device-scope stores and loads).  No float atomics and no
//    device-scope fences.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "internal.h"

namespace tvp {

struct GemmArgs {
  const uint16_t* x;   // row-major activations (wide kernel)
  const uint16_t* xp;  // packed activations (skinny kernel): element (row, k) at (k/8)*256 + row*8 + k%8
  int64_t ldx;
  int m, k_in;
  const uint8_t* rec;
  const uint32_t* escoff;
  const uint32_t* esc;
  const uint32_t* b2;
  const int32_t* rowmap;
  int n_tiles, n_kb, n_pad;
  int groups, splits, kbs, ntasks;
  int kps;    // skinny: K blocks per slice of a split group
  int kbs_split;  // skinny, partial-sum epilogue: K blocks per wavefront of a slice
  float* part;
  unsigned long long* keys;  // ARGMAX: [slot][m] packed (value, -id) maxima, one slot per workgroup that
                             // applies the epilogue (every slot written, no zeroing)
  int key_slots;
  int fmt;  // TVP_FMT_W12, TVP_FMT_HI8 (the 8-bit leading view) or kFmtI8 (int8 values): see decode_*
  // INT8 head (kEpiI8Approx): per-channel scale and bound radius, per-row ||f||_2
  const float* i8_scale;
  const float* i8_r;
  const float* i8_fnorm;
  int mode;
  void* y;
  int64_t ldy;
  const uint16_t* resid;
  int64_t ldr;
  const int32_t* pos;
  const int32_t* slot;
  uint16_t* kc;
  uint16_t* vc;
  int64_t s_stride;
  double theta;
  int hq, hkv, d;
  int32_t* argmax;
  float* logits;
  int64_t ldl;
  int y_packed;  // SWIGLU: write y in the packed activation layout (rows <= 32)
  // Skinny, whole-K epilogues: workgroups 0 .. full_groups-1 take whole
  // groups; the remaining groups are cut into rem_splits K slices of rem_kps
  // blocks (rem_kbs per wavefront) whose sums go to rpart [slice][row][ldrp]
  // (device-scope stores); the slice of a group that arrives last on
  // rcnt[group - full_groups] sums them all and applies the epilogue.
  int full_groups, rem_splits, rem_kps, rem_kbs, rem_tpw;
  float* rpart;
  int ldrp;
  uint32_t* rcnt;
  const float* rope_cs;  // QKV: optional per-pass (cos, sin) table, see gemm_run
  int cache_rowmap;      // epilogue: stage the group's channel rows in LDS first (many rows per thread)
};

constexpr int kArgmaxMaxRows = 192;
// Compute units the skinny decomposition balances over (MI355X: 256).
constexpr int kNumCUs = 256;
constexpr int kRemMaxSplits = 16;  // K slices of a remaining group (whole-K epilogues)

// n arrival counters to zero (one workgroup).
__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* __restrict__ p, int n) {
  for (int i = threadIdx.x; i < n; i += 256) p[i] = 0u;
}

// Row-major x [m][ldx] -> packed (rows >= m and columns >= k_in are zero).
__global__ __launch_bounds__(256) void pack_x_kernel(const uint16_t* __restrict__ x, int64_t ldx, int m,
                                                     int k_in, int nchunks, uint16_t* __restrict__ xp) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over nchunks * 32
  if (idx >= (int64_t)nchunks * 32) return;
  const int row = (int)(idx & 31);
  const int64_t c = idx >> 5;
  const int64_t k = c * 8;
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (row < m && k + e < k_in) ? x[row * ldx + k + e] : 0u;
  *(uint4*)(xp + c * 256 + row * 8) =
      make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

__device__ inline uint32_t rotl32(uint32_t x, int r) { return r == 0 ? x : (x << r) | (x >> (32 - r)); }

// 12 record dwords of one lane -> 16 bf16-pair dwords (K-step s = o[4s..4s+3]).
__device__ inline void decode_block(const uint4 (&r)[3], uint32_t b2, uint32_t (&o)[16]) {
  const uint32_t lb[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
  const uint32_t hn[4] = {r[2].x, r[2].y, r[2].z, r[2].w};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t L = lb[2 * s + q];
      o[4 * s + 2 * q] = (rotl32(hn[s], 8 * q) & 0x87008700u) + (L & 0x00FF00FFu) + b2;
      o[4 * s + 2 * q + 1] = (rotl32(hn[s], 8 * q + 4) & 0x87008700u) + ((L >> 8) & 0x00FF00FFu) + b2;
    }
  }
}

// The 8-bit leading view (record >> 4 per weight): 8 dwords of one lane ->
// 16 bf16-pair dwords, the low four mantissa bits zero.  Each dword holds the
// bytes of weights (4q, 4q+2, 4q+1, 4q+3); sign to bit 15 of each halfword,
// offset and top mantissa bits shifted into place, plus the window base.
__device__ inline void decode_block_hi8(const uint4 (&r)[3], uint32_t b2, uint32_t (&o)[16]) {
  const uint32_t D[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t d = D[2 * s + q];
      o[4 * s + 2 * q] = (((d & 0x007F007Fu) << 4) + b2) | ((d & 0x00800080u) << 8);
      o[4 * s + 2 * q + 1] = (((d >> 4) & 0x07F007F0u) + b2) | (d & 0x80008000u);
    }
  }
}

// Int8 values (the INT8 LM head): 8 dwords of one lane -> 16 bf16-pair
// dwords, each value converted exactly (|q| <= 127 fits bf16's significand).
// Byte order as above: (4q, 4q+2, 4q+1, 4q+3).
__device__ inline void decode_block_i8(const uint4 (&r)[3], uint32_t (&o)[16]) {
  const uint32_t D[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int32_t d = (int32_t)D[2 * s + q];
      const float f0 = (float)((d << 24) >> 24), f2 = (float)((d << 16) >> 24);
      const float f1 = (float)((d << 8) >> 24), f3 = (float)(d >> 24);
      o[4 * s + 2 * q] = pack_bf16x2(f0, f1);
      o[4 * s + 2 * q + 1] = pack_bf16x2(f2, f3);
    }
  }
}

__device__ inline bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ inline float silu_f32(float g) { return g / (1.0f + expf(-g)); }

// Compiler-level ordering of LDS accesses within one wavefront.  The
// wavefront's LDS instructions execute in issue order, so no wait is needed;
// the clobber keeps the compiler from reordering or forwarding across it.
__device__ inline void lds_order() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// (value, id) packed so that a 64-bit unsigned max picks the largest value
// and, among equal values, the smallest id.
__device__ inline unsigned long long argmax_key(float v, int32_t id) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)id);
}

// RoPE angle of rotated dim i (< d/2) at position pos, formed in fp64.
__device__ inline double rope_angle(int pos, double theta, int i, int d) {
  return (double)pos * pow(theta, -2.0 * (double)i / (double)d);
}

// One thread per (row, rotated dim): the (cos, sin) table of a pass.
__global__ __launch_bounds__(256) void rope_table_kernel(const int32_t* __restrict__ pos, int n, int d,
                                                         double theta, float2* __restrict__ cs) {
  const int half = d / 2;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= n * half) return;
  const int r = idx / half, i = idx % half;
  const double ang = rope_angle(pos[r], theta, i, d);
  cs[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

// Epilogue over packed channels [c0, c0+nc) x rows [0, M) by `nthr` threads
// (thread index `tid`), reading fp32 results through V(row, col).
template <int MODE, typename Get>
__device__ inline void epilogue(const GemmArgs& a, int c0, int nc, int M, int tid, int nthr, int key_slot,
                                Get V, int slice = 0) {
  // When each thread walks many (row, column) pairs, the channels' canonical
  // rows come from LDS (no dependent global load per element); the loops are
  // unrolled so independent loads overlap.
  __shared__ int32_t rm_s[128];
  const bool cached = a.cache_rowmap && nc <= 128;  // uniform over the workgroup
  if (cached) {
    for (int i = tid; i < nc; i += nthr) rm_s[i] = a.rowmap[c0 + i];
    __syncthreads();
  }
  auto rowmap_of = [&](int col) { return cached ? rm_s[col - c0] : a.rowmap[col]; };
  if constexpr (MODE == kEpiPartial) {
    float* P = (float*)a.y + (int64_t)slice * M * a.ldy;
    for (int idx = tid; idx < M * nc; idx += nthr) {
      const int row = idx / nc, col = c0 + idx % nc;
      const int32_t r = a.rowmap[col];
      if (r >= 0) P[row * a.ldy + r] = V(row, col);
    }
  } else if constexpr (MODE == TVP_EPI_F32 || MODE == TVP_EPI_BF16 || MODE == TVP_EPI_RESID) {
#pragma unroll 4
    for (int idx = tid; idx < M * nc; idx += nthr) {
      const int row = idx / nc, col = c0 + idx % nc;
      const int32_t r = rowmap_of(col);
      if (r < 0) continue;
      const float v = V(row, col);
      if constexpr (MODE == TVP_EPI_F32) {
        ((float*)a.y)[row * a.ldy + r] = v;
      } else if constexpr (MODE == TVP_EPI_BF16) {
        ((uint16_t*)a.y)[row * a.ldy + r] = (uint16_t)f32_to_bf16(v);
      } else {
        const float rv = bf16_to_f32(a.resid[row * a.ldr + r]);
        ((uint16_t*)a.y)[row * a.ldy + r] = (uint16_t)f32_to_bf16(rv + v);
      }
    }
  } else if constexpr (MODE == TVP_EPI_SWIGLU) {
    const int half = nc / 2;  // nc is a multiple of 32
#pragma unroll 4
    for (int idx = tid; idx < M * half; idx += nthr) {
      const int row = idx / half, p = idx % half;
      const int col = c0 + (p / 16) * 32 + (p % 16);
      const int32_t r = rowmap_of(col);
      if (r < 0) continue;
      const float gv = V(row, col), uv = V(row, col + 16);
      const uint16_t o = (uint16_t)f32_to_bf16(silu_f32(gv) * uv);
      if (a.y_packed) ((uint16_t*)a.y)[xpack_index(row, r)] = o;
      else ((uint16_t*)a.y)[row * a.ldy + r] = o;
    }
  } else if constexpr (MODE == TVP_EPI_QKV) {
    const int d = a.d, tph = d / 32;
    const int rot_tiles = (a.hq + a.hkv) * tph;
#pragma unroll 4
    for (int idx = tid; idx < M * nc; idx += nthr) {
      const int row = idx / nc, col = c0 + idx % nc;
      const int t = col / 32, c = col % 32;
      if (t >= a.n_tiles) continue;
      if (t < rot_tiles) {
        if (c >= 16) continue;
        const int head = t / tph, u = t % tph;
        const int da = 16 * u + c, db = d / 2 + 16 * u + c;
        const float xa = V(row, col), xb = V(row, col + 16);
        float cs, sn;
        if (a.rope_cs) {
          const float2 t = ((const float2*)a.rope_cs)[(int64_t)row * (d / 2) + da];
          cs = t.x;
          sn = t.y;
        } else {
          const double ang = rope_angle(a.pos[row], a.theta, da, d);
          cs = (float)cos(ang);
          sn = (float)sin(ang);
        }
        const float oa = xa * cs - xb * sn, ob = xb * cs + xa * sn;
        if (head < a.hq) {
          uint16_t* q = (uint16_t*)a.y + (int64_t)row * a.ldy + (int64_t)head * d;
          q[da] = (uint16_t)f32_to_bf16(oa);
          q[db] = (uint16_t)f32_to_bf16(ob);
        } else {
          uint16_t* kr = a.kc + ((int64_t)(head - a.hq) * a.s_stride + a.slot[row]) * d;
          kr[da] = (uint16_t)f32_to_bf16(oa);
          kr[db] = (uint16_t)f32_to_bf16(ob);
        }
      } else {
        const int vr = (t - rot_tiles) * 32 + c;
        if (vr >= a.hkv * d) continue;
        const int kh = vr / d, dim = vr % d;
        a.vc[((int64_t)kh * a.s_stride + a.slot[row]) * d + dim] = (uint16_t)f32_to_bf16(V(row, col));
      }
    }
  } else if constexpr (MODE == kEpiI8Approx) {
    // INT8 head: approximate logit a = scale * acc of every channel to
    // logits [row][ldl], and per row the largest a - ||f|| r of this
    // workgroup (the certificate threshold's share) to its key slot
    __shared__ unsigned long long red_i8[8][32];
    for (int row = 0; row < M; ++row) {
      unsigned long long best = 0ull;
      const float fn = a.i8_fnorm[row];
      for (int cc = tid; cc < nc; cc += nthr) {
        const int col = c0 + cc;
        const int32_t r = rowmap_of(col);
        if (r < 0) continue;
        const float v = V(row, col) * a.i8_scale[r];
        a.logits[row * a.ldl + r] = v;
        const unsigned long long k = argmax_key(v - fn * a.i8_r[r], r);
        best = k > best ? k : best;
      }
      for (int off = 32; off > 0; off >>= 1) {
        const unsigned long long o = __shfl_xor(best, off);
        best = o > best ? o : best;
      }
      if ((tid & 63) == 0) red_i8[tid >> 6][row] = best;
    }
    __syncthreads();
    for (int row = tid; row < M; row += nthr) {
      unsigned long long best = 0ull;
      for (int w = 0; w < (nthr >> 6); ++w) best = red_i8[w][row] > best ? red_i8[w][row] : best;
      a.keys[(int64_t)key_slot * M + row] = best;
    }
  } else {  // ARGMAX: per row the best (value, smallest id) of this workgroup, to its key slot
    __shared__ unsigned long long red[8][kArgmaxMaxRows];
    for (int row = 0; row < M; ++row) {
      unsigned long long best = 0ull;
      for (int cc = tid; cc < nc; cc += nthr) {
        const int col = c0 + cc;
        const int32_t r = rowmap_of(col);
        if (r < 0) continue;
        const float v = V(row, col);
        if (a.logits) a.logits[row * a.ldl + r] = v;
        const unsigned long long k = argmax_key(v, r);
        best = k > best ? k : best;
      }
      for (int off = 32; off > 0; off >>= 1) {
        const unsigned long long o = __shfl_xor(best, off);
        best = o > best ? o : best;
      }
      if ((tid & 63) == 0) red[tid >> 6][row] = best;
    }
    __syncthreads();
    for (int row = tid; row < M; row += nthr) {
      unsigned long long best = 0ull;
      for (int w = 0; w < (nthr >> 6); ++w) best = red[w][row] > best ? red[w][row] : best;
      a.keys[(int64_t)key_slot * M + row] = best;
    }
  }
}

// One workgroup per row: argmax[row] from the key slots (max over slots, so
// the order does not matter).
__global__ __launch_bounds__(256) void argmax_finalize_kernel(const unsigned long long* __restrict__ keys,
                                                              int slots, int m, int32_t* __restrict__ argmax) {
  __shared__ unsigned long long wmax[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  unsigned long long k = 0ull;
  for (int s = tid; s < slots; s += 256) {
    const unsigned long long v = keys[(int64_t)s * m + row];
    k = v > k ? v : k;
  }
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned long long o = __shfl_xor(k, off);
    k = o > k ? o : k;
  }
  if ((tid & 63) == 0) wmax[tid >> 6] = k;
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) k = wmax[w] > k ? wmax[w] : k;
    k = wmax[0] > k ? wmax[0] : k;
    argmax[row] = k ? (int32_t)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull)) : 0;
  }
}

// ----------------------------------------------------------------------------
// Skinny kernel (m <= 32): a workgroup owns TPW tiles; its KW wavefronts split
// the K range and stream independently.  Records, escape entries and
// activation fragments for block i + RD - 1 are in flight while block i is
// decoded and multiplied (a register ring, unrolled so no copies tie the
// prefetch to the use).  Activation fragments come straight from global
// memory (a few hundred KB, they stay in L2).  The escape offsets of a
// wave's blocks sit in one VGPR per tile (lane i = block kb0 + i) and are read
// with readlane, so no load in the loop depends on another.  At the end the
// waves' fp32 partial tiles meet in LDS and are summed in wave order: no
// global partial sums, no atomics, no device-scope fences.
template <int MT, int TPW, int RD, int MODE, int FMT>
__global__ __launch_bounds__(512) void w12_skinny_kernel(GemmArgs a) {
  constexpr bool W12 = FMT == TVP_FMT_W12;
  constexpr int NQ = W12 ? 3 : 2;  // 16-byte pieces per lane of one tile block
  constexpr int BB = W12 ? kBlockBytes : kBlockBytesHi8;
  constexpr int NACC = MT == 32 ? 16 : 4;
  constexpr int NCH = MT == 32 ? 1 : 2;
  constexpr int KS = MT == 32 ? 4 : 2;  // MFMA K-steps per 64-column block
  typedef float accv __attribute__((ext_vector_type(NACC)));
  extern __shared__ uint4 dsm[];  // KW x TPW x 4 KB: decode scratch, then the partial tiles
  typedef uint4 scr_t[TPW][256];
  scr_t* scr = (scr_t*)dsm;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KW = blockDim.x >> 6;
  // Workgroup -> work: one workgroup per group of TPW tiles over the whole K
  // range, or, with the partial-sum epilogue, one per (group, K slice).
  // With a whole-K epilogue, workgroups past full_groups take one K slice of
  // a remaining group (so every CU gets the same share of the stream).
  // Workgroups b, b + 256, b + 512, ... start on one CU, one per CU per
  // dispatch round; when whole groups fill several rounds they take
  // consecutive groups, so one CU reads neighbouring tiles of each k block
  // (measured: verify steps at the 27B-like shapes 0.9% faster, with 2 and 9
  // rounds in the gate/up and LM-head launches; the int8 head's 2 KB blocks
  // lost 7% that way and keep the dispatch order).
  int b = blockIdx.x;
  if (MODE != kEpiPartial && FMT != kFmtI8) {
    const int rounds = a.full_groups / kNumCUs;
    if (rounds >= 2 && b < rounds * kNumCUs) b = rounds * (b % kNumCUs) + b / kNumCUs;
  }
  const bool rem = MODE != kEpiPartial && b >= a.full_groups;
  int grp, slice, ks0, ks1, kbs;  // ks0 .. ks1: this workgroup's K range
  if (MODE == kEpiPartial) {
    grp = b / a.splits;
    slice = b % a.splits;
    ks0 = slice * a.kps;
    ks1 = min(a.n_kb, ks0 + a.kps);
    kbs = a.kbs_split;
  } else if (!rem) {
    grp = b;
    slice = 0;
    ks0 = 0;
    ks1 = a.n_kb;
    kbs = a.kbs;
  } else {
    const int rr = b - a.full_groups;
    grp = a.full_groups + rr / a.rem_splits;
    slice = rr % a.rem_splits;
    ks0 = slice * a.rem_kps;
    ks1 = min(a.n_kb, ks0 + a.rem_kps);
    kbs = a.rem_kbs;
  }
  const int t0 = grp * TPW;
  const int kb0 = ks0 + wave * kbs;
  const int kb1 = min(ks1, kb0 + kbs);
  const int nblk = kb1 > kb0 ? kb1 - kb0 : 0;  // <= 63

  // Tiles past the end are computed on a clamped tile and dropped at the end,
  // so the streaming loop has no data-dependent branches around its loads
  // (the compiler's wait counters then stay exact and the ring stays full).
  int tt[TPW];
  uint32_t ewin[TPW], b2v[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    tt[t] = min(t0 + t, a.n_tiles - 1);
    ewin[t] = a.escoff[(int64_t)tt[t] * a.n_kb + min(kb0 + min(lane, nblk), a.n_kb)];
    b2v[t] = a.b2[tt[t] * 32 + (lane & 31)];
  }
  accv acc[TPW][NCH];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int v = 0; v < NACC; ++v) acc[t][ch][v] = 0.0f;

  // activation fragments from the packed layout: rows past m hold zeros or
  // garbage and only feed output rows that are never stored.  In the 16-row
  // shape the lanes of rows past m read row m - 1 again, the same lines: at
  // up to 8 rows a block's fragments touch 8 lines instead of 16 (measured:
  // 1- and 8-node steps 1.9% faster; the 32-row shape, where it would save
  // lines only below 25 rows, keeps every row's own address: +0.2% at 32)
  const int xrow = MT == 32 ? (lane & 31) : min(lane & 15, a.m - 1);
  const int xsub = MT == 32 ? 8 * (lane >> 5) : 8 * (lane >> 4);
  const uint16_t* xr = a.xp + xrow * 8;
  // the last block of a ragged K range is handled on its own, with guards
  const bool ragged_tail = nblk > 0 && kb1 == a.n_kb && (a.k_in & 63) != 0;
  const int nfast = nblk - (ragged_tail ? 1 : 0);

  uint4 R[RD][TPW][3] = {};  // HI8 fills two of the three pieces
  uint4 A[RD][KS];
  uint32_t E[RD][TPW];

  auto issue_rec_only = [&](int i, int slot) {
    const int j = kb0 + i;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const uint4* blk = (const uint4*)(a.rec + rec_block(tt[t], j, a.n_tiles) * BB);
#pragma unroll
      for (int q = 0; q < NQ; ++q) R[slot][t][q] = load_nt(blk + q * 64 + lane);
    }
  };
  auto issue_esc = [&](int i, int slot) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const uint32_t eo = __builtin_amdgcn_readlane(ewin[t], i);
      const uint32_t ec = __builtin_amdgcn_readlane(ewin[t], i + 1) - eo;
      // lanes past the count read a neighbour (the blob continues past the
      // escape list) and are never used
      E[slot][t] = a.esc[(uint32_t)lane < ec ? eo + lane : eo];
    }
  };
  auto issue_recs = [&](int i, int slot) {
    issue_rec_only(i, slot);
    issue_esc(i, slot);
  };
  // full blocks: every activation load is in range
  auto issue_act_fast = [&](int i, int slot) {
    const int j = kb0 + i;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int64_t k = 64LL * j + (MT == 32 ? 16 : 32) * ks + xsub;
      A[slot][ks] = *(const uint4*)(xr + (k >> 3) * 256);
    }
  };
  auto issue_fast = [&](int i, int slot) {
    i = min(i, nfast - 1);  // past the end: re-read the last block (cached), result unused
    issue_recs(i, slot);
    issue_act_fast(i, slot);
  };
  auto issue_tail = [&](int i, int slot) {
    issue_recs(i, slot);
    const int j = kb0 + i;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int64_t k = 64LL * j + (MT == 32 ? 16 : 32) * ks + xsub;
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (k + e < a.k_in) ? xr[(k >> 3) * 256 + e] : 0u;
      A[slot][ks] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    }
  };

  auto process = [&](int i, int slot, auto slow) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      uint32_t o[16];
      if constexpr (FMT == TVP_FMT_HI8) decode_block_hi8(R[slot][t], b2v[t], o);
      else if constexpr (FMT == kFmtI8) decode_block_i8(R[slot][t], o);
      else decode_block(R[slot][t], b2v[t], o);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        scr[wave][t][64 * s + lane] = make_uint4(o[4 * s], o[4 * s + 1], o[4 * s + 2], o[4 * s + 3]);
    }
    lds_order();
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const uint32_t eo = __builtin_amdgcn_readlane(ewin[t], i);
      const uint32_t ec = __builtin_amdgcn_readlane(ewin[t], i + 1) - eo;
      uint16_t* sh = (uint16_t*)&scr[wave][t][0];
      if ((uint32_t)lane < ec) sh[E[slot][t] & 0x7FFu] = (uint16_t)(E[slot][t] >> 16);
      if constexpr (decltype(slow)::value) {  // more escapes than lanes in some tile block
        for (uint32_t e = 64 + lane; e < ec; e += 64) {
          const uint32_t ent = a.esc[eo + e];
          sh[ent & 0x7FFu] = (uint16_t)(ent >> 16);
        }
      }
    }
    lds_order();
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      if constexpr (MT == 32) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8_t B = as_bf16x8(scr[wave][t][64 * ks + lane]);
          acc[t][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(A[slot][ks]), B, acc[t][0], 0, 0, 0);
        }
      } else {
        const int q = lane >> 4;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int ch = 0; ch < 2; ++ch) {
            const bf16x8_t B = as_bf16x8(scr[wave][t][(4 * ks + q) * 32 + 16 * ch + (lane & 15)]);
            acc[t][ch] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(A[slot][ks]), B, acc[t][ch], 0, 0, 0);
          }
      }
    }
    lds_order();
  };

  // The first blocks' records and activations need no escape offsets: they
  // are issued before the wait for the offsets, so that wait overlaps them
  // (all on one straight path, so the wait counts stay exact).
  if (nfast > 0) {
#pragma unroll
    for (int p = 0; p < RD - 1; ++p) {
      issue_rec_only(min(p, nfast - 1), p);
      issue_act_fast(min(p, nfast - 1), p);
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) asm volatile("" ::"v"(ewin[t]), "v"(b2v[t]));  // offsets and bases arrived

    // Tasks where some tile block has more escapes than lanes take a simple
    // unpipelined loop; all others stream through the register ring, whose
    // body then holds no loop with loads of its own.
    uint32_t mx = 0;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const uint32_t nxt = __shfl_down(ewin[t], 1);
      const uint32_t c = lane < nblk ? nxt - ewin[t] : 0u;
      mx = c > mx ? c : mx;
    }
    for (int off = 32; off > 0; off >>= 1) {
      const uint32_t o = __shfl_xor(mx, off);
      mx = o > mx ? o : mx;
    }
    const bool slow = __builtin_amdgcn_readfirstlane(mx) > 64u;
    if (!slow) {
#pragma unroll
      for (int p = 0; p < RD - 1; ++p) issue_esc(min(p, nfast - 1), p);
      for (int i0 = 0; i0 < nfast; i0 += RD) {
#pragma unroll
        for (int r = 0; r < RD; ++r) {
          issue_fast(i0 + r + RD - 1, (r + RD - 1) % RD);
          if (i0 + r < nfast) process(i0 + r, r, std::false_type{});
        }
      }
    } else {
      for (int i = 0; i < nfast; ++i) {
        issue_fast(i, 0);
        process(i, 0, std::true_type{});
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TPW; ++t) asm volatile("" ::"v"(ewin[t]), "v"(b2v[t]));
  if (ragged_tail) {
    issue_tail(nblk - 1, 0);
    process(nblk - 1, 0, std::true_type{});
  }

  // ------------------------------------------------------------- results
  const int M = a.m;
  const int NC = TPW * 32;
  __syncthreads();  // every wave is done with its decode scratch
  float* P = (float*)dsm;  // [KW][M][NC] fp32 partial tiles
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int v = 0; v < NACC; ++v) {
        int row, col;
        if constexpr (MT == 32) {
          row = (v >> 2) * 8 + 4 * (lane >> 5) + (v & 3);
          col = t * 32 + (lane & 31);
        } else {
          row = 4 * (lane >> 4) + v;
          col = t * 32 + 16 * ch + (lane & 15);
        }
        if (row < M) P[(wave * M + row) * NC + col] = acc[t][ch][v];
      }
  __syncthreads();
  auto sum_waves = [&](int row, int col) {
    const int c = col - t0 * 32;
    float v = 0.0f;
    for (int w = 0; w < KW; ++w) v += P[(w * M + row) * NC + c];
    return v;
  };
  const int nc = min(NC, a.n_pad - t0 * 32);
  const int nthr = KW * 64;
  float* S = nullptr;  // set: the epilogue reads the group's slice sums [M][nc] from LDS
  if constexpr (MODE != kEpiPartial && MODE != TVP_EPI_ARGMAX && MODE != kEpiI8Approx) {
    if (rem) {  // this K slice's sums, [slice][row][channel - first remaining channel]
      const int cb = t0 * 32 - a.full_groups * TPW * 32;
      const int ne = M * nc;
      for (int idx = threadIdx.x; idx < ne; idx += nthr) {
        const int row = idx / nc, c = idx % nc;
        st_dev(a.rpart + ((int64_t)slice * M + row) * a.ldrp + cb + c, sum_waves(row, t0 * 32 + c));
      }
      // The slice that arrives last sums the group's slices in slice order
      // (each thread the elements it stored; 8 slices x 8 elements in
      // flight), stages the sums in LDS and applies the group's epilogue.
      __shared__ int s_last;
      if (!arrive_last(a.rcnt + (grp - a.full_groups), (uint32_t)a.rem_splits, &s_last)) return;
      S = (float*)dsm;  // the partial tiles are no longer read
      const int64_t sst = (int64_t)M * a.ldrp;
      for (int e0 = 0; e0 < ne; e0 += 8 * nthr) {
        float acc[8];
        for (int s0 = 0; s0 < a.rem_splits; s0 += 8) {
          float v[8][8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int64_t so = (int64_t)min(s0 + j, a.rem_splits - 1) * sst;  // past the last slice: repeated, unused
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int idx = min(e0 + i * nthr + (int)threadIdx.x, ne - 1);
              v[j][i] = ld_dev(a.rpart + so + (int64_t)(idx / nc) * a.ldrp + cb + idx % nc);
            }
          }
#pragma unroll
          for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              if (s0 + j == 0) acc[i] = v[j][i];
              else if (s0 + j < a.rem_splits) acc[i] += v[j][i];
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int idx = e0 + i * nthr + (int)threadIdx.x;
          if (idx < ne) S[idx] = acc[i];
        }
      }
      __syncthreads();
    }
  }
  // one epilogue instantiation for both sources (its LDS arrays exist once)
  epilogue<MODE>(a, t0 * 32, nc, M, threadIdx.x, nthr, blockIdx.x,
                 [&](int row, int col) { return S ? S[row * nc + (col - t0 * 32)] : sum_waves(row, col); }, slice);
}

// ----------------------------------------------------------------------------
// Wide kernel (33..192 rows): a workgroup owns 4 x TPW tiles (TPW per
// wavefront) and a K range; all four wavefronts walk the same 64-column
// blocks, so one copy of X per block serves them from LDS, and each A
// fragment read from there feeds the MFMAs of the wavefront's TPW tiles.
// Per block: X for the block after next is fetched into registers while this
// block is multiplied, and stored to the other half of a double-buffered LDS
// tile behind one barrier; each wavefront's records sit in a register ring,
// are decoded into its own LDS scratch, patched with the block's escapes, and
// multiplied against RB row blocks of X (v_mfma_f32_32x32x16_bf16).  Rows are
// XOR-swizzled by their 16-byte column group inside the X tile: the
// row-major fill and the column reads of the MFMA A operand are both free of
// bank conflicts.
template <int RB, int TPW, int RD>
__global__ __launch_bounds__(256, TPW == 1 ? 2 : 1) void w12_wide_kernel(GemmArgs a) {
  constexpr int ROWS = 32 * RB;
  // RD: register-ring depth (blocks of records in flight per wavefront).
  __shared__ uint4 xs[2][8 * ROWS];  // X block [k group][row ^ k group]
  __shared__ uint4 scr[4][TPW][256];  // per-wavefront decode scratch: one 32 x 64 block per tile

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  // uniform per wavefront, so the escape offsets below are scalar loads and
  // no vector load in the ring waits on another
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.x / a.splits, sp = blockIdx.x % a.splits;
  const int kb0 = sp * a.kbs;
  const int kb1 = min(a.n_kb, kb0 + a.kbs);
  const int nblk = kb1 > kb0 ? kb1 - kb0 : 0;
  const int tile0 = (g * 4 + wave) * TPW;
  int tt[TPW];
  uint32_t b2v[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    tt[t] = min(tile0 + t, a.n_tiles - 1);  // a tile past the end runs clamped; its results are dropped
    b2v[t] = a.b2[tt[t] * 32 + (lane & 31)];
  }

  f32x16_t acc[TPW][RB];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[t][rb][v] = 0.0f;

  // X block j (row-major x): thread piece i is row (tid + 256 i) / 8,
  // 16-byte group (tid % 8).  A block inside k_in loads without branches:
  // rows past m read row m - 1 and only feed output rows that are never
  // stored.  The ragged last block (a uniform branch) reads zeros past k_in
  // and past m.
  uint4 xr[RB];
  // this thread's row pointers (clamped rows) and LDS slots, formed once
  const uint16_t* xrow[RB];
  int xslot[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    xrow[i] = a.x + (int64_t)min((tid >> 3) + 32 * i, a.m - 1) * a.ldx + 8 * (tid & 7);
    xslot[i] = (tid & 7) * ROWS + (((tid >> 3) + 32 * i) ^ (tid & 7));
  }
  auto load_x = [&](int j) {
    const int64_t k = (int64_t)j * kBlockK + 8 * (tid & 7);
    if ((int64_t)(j + 1) * kBlockK <= a.k_in) {
#pragma unroll
      for (int i = 0; i < RB; ++i) xr[i] = *(const uint4*)(xrow[i] + (int64_t)j * kBlockK);
    } else {
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int row = (tid >> 3) + 32 * i;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < a.m && k < a.k_in) {
          const uint16_t* src = a.x + (int64_t)row * a.ldx + k;
          uint32_t hh[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) hh[e] = (k + e < a.k_in) ? src[e] : 0u;
          v = make_uint4(hh[0] | (hh[1] << 16), hh[2] | (hh[3] << 16), hh[4] | (hh[5] << 16), hh[6] | (hh[7] << 16));
        }
        xr[i] = v;
      }
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RB; ++i) xs[buf][xslot[i]] = xr[i];
  };

  // Escape offsets of a window of 64 blocks, one VGPR per tile (lane l:
  // block wbase + l), read with readlane: no load in the ring waits on
  // another (a dependent offset load per block would make every step wait
  // for all older loads, the ring's included).  A window serves kWin blocks
  // (a multiple of the ring depth) plus the ring's lookahead.
  constexpr int kWin = (64 - RD) / RD * RD;
  static_assert(kWin % RD == 0 && kWin + RD <= 64, "window");
  uint32_t ewin[TPW];
  int wbase = 0;
  auto load_win = [&](int w0) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) ewin[t] = a.escoff[(int64_t)tt[t] * a.n_kb + min(kb0 + w0 + lane, a.n_kb)];
    wbase = w0;
    // consumed here, once per window: the inner loop's header then never
    // waits for it (which would drain the whole ring)
#pragma unroll
    for (int t = 0; t < TPW; ++t) asm volatile("" ::"v"(ewin[t]));
  };

  // records and escape entries of block i into ring slot `slot` (past the
  // end: the last block again, result unused)
  uint4 R[RD][TPW][3];
  uint32_t E[RD][TPW], EO[RD][TPW], EC[RD][TPW];
  auto issue = [&](int i, int slot) {
    const int ic = min(i, max(nblk - 1, 0));
    const int j = kb0 + ic;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const uint32_t eo = __builtin_amdgcn_readlane(ewin[t], ic - wbase);
      const uint32_t ec = __builtin_amdgcn_readlane(ewin[t], ic - wbase + 1) - eo;
      const uint4* blk = (const uint4*)(a.rec + rec_block(tt[t], j, a.n_tiles) * kBlockBytes);
#pragma unroll
      for (int q = 0; q < 3; ++q) R[slot][t][q] = load_nt(blk + q * 64 + lane);
      // lanes past the count read a neighbour (the blob continues past the
      // escape list) and are never used
      E[slot][t] = a.esc[(uint32_t)lane < ec ? eo + lane : eo];
      EO[slot][t] = eo;
      EC[slot][t] = ec;
    }
  };

  auto process = [&](int slot, int buf) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      uint32_t o[16];
      decode_block(R[slot][t], b2v[t], o);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        scr[wave][t][64 * s4 + lane] = make_uint4(o[4 * s4], o[4 * s4 + 1], o[4 * s4 + 2], o[4 * s4 + 3]);
    }
    lds_order();
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      uint16_t* sh = (uint16_t*)&scr[wave][t][0];
      const uint32_t ec = EC[slot][t];
      if ((uint32_t)lane < ec) sh[E[slot][t] & 0x7FFu] = (uint16_t)(E[slot][t] >> 16);
      for (uint32_t e = 64 + lane; e < ec; e += 64) {  // more escapes than lanes (rare)
        const uint32_t ent = a.esc[EO[slot][t] + e];
        sh[ent & 0x7FFu] = (uint16_t)(ent >> 16);
      }
    }
    lds_order();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t B[TPW];
#pragma unroll
      for (int t = 0; t < TPW; ++t) B[t] = as_bf16x8(scr[wave][t][64 * ks + lane]);
      const int kg = 2 * ks + h;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const bf16x8_t A = as_bf16x8(xs[buf][kg * ROWS + ((rb * 32 + (lane & 31)) ^ kg)]);
#pragma unroll
        for (int t = 0; t < TPW; ++t)
          acc[t][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B[t], acc[t][rb], 0, 0, 0);
      }
    }
    lds_order();
  };

  if (nblk > 0) {
    load_win(0);
#pragma unroll
    for (int p = 0; p < RD - 1; ++p) issue(p, p);
    load_x(kb0);
    store_x(0);
    if (nblk > 1) load_x(kb0 + 1);
    __syncthreads();
    // The ring slot is a compile-time constant inside each unrolled group,
    // and the loads run unconditionally (clamped to the last block past the
    // end), so the wait counts stay exact.
    for (int w0 = 0; w0 < nblk; w0 += kWin) {
      if (w0 > 0) load_win(w0);  // blocks issued ahead from the last window are in this one too
      const int wend = min(nblk, w0 + kWin);
      for (int i0 = w0; i0 < wend; i0 += RD) {
#pragma unroll
        for (int r = 0; r < RD; ++r) {
          const int i = i0 + r;
          issue(i + RD - 1, (r + RD - 1) % RD);
          if (i < wend) process(r, i & 1);
          store_x((i + 1) & 1);  // block i + 1, fetched one block ago (its buffer was last read before
                                 // the previous barrier)
          load_x(kb0 + min(i + 2, nblk - 1));
          __syncthreads();
        }
      }
    }
  }

  // this split's sums: part [split][row][packed channel]
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    if (tile0 + t >= a.n_tiles) continue;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = rb * 32 + (v >> 2) * 8 + 4 * h + (v & 3);
        const int col = (tile0 + t) * 32 + (lane & 31);
        if (row < a.m) a.part[((int64_t)sp * a.m + row) * a.n_pad + col] = acc[t][rb][v];
      }
  }
  // The next launch adds the splits in split order and applies the epilogue
  // (w12_wide_fixup_kernel, or the fused residual + RMSNorm for partial-sum
  // epilogues): no device-scope fence or completion counter here (on a part
  // with one L2 per XCD a device-scope release writes back the L2, and one
  // per workgroup serialises the launch).
}

// One workgroup per (group of 4 tiles, 32-row block): the wide kernel's split
// sums (visible here through the kernel boundary) are added in split order
// into LDS, with several pieces' loads of every split in flight together,
// then the epilogue runs on the block's rows (its row-indexed pointers
// offset to the block).  ARGMAX scans a row per thread.
constexpr int kWideSumStride = 33;  // float4 per row of the LDS sums (padded: row-parallel reads spread over banks)
__global__ __launch_bounds__(256) void w12_wide_fixup_kernel(GemmArgs a) {
  __shared__ float4 sums[32 * kWideSumStride];  // [row][128 channels / 4 (+1)]
  const int rbn = (a.m + 31) / 32;
  const int g = blockIdx.x / rbn, r0 = (blockIdx.x % rbn) * 32, tid = threadIdx.x;
  const int c0 = g * 4 * 32;
  const int nc = min(a.n_pad, c0 + 4 * 32) - c0;  // a multiple of 32
  const int M = min(32, a.m - r0), nq = nc / 4;
  const int64_t sstride = (int64_t)a.m * a.n_pad / 4;  // float4 units
  const float4* base = (const float4*)(a.part + (int64_t)r0 * a.n_pad + c0);
  constexpr int U = 4, SJ = 4;  // pieces per thread and splits per round: U x SJ loads in flight
  for (int i0 = 0; i0 < M * nq; i0 += 256 * U) {
    float4 acc[U];
    const float4* src[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = min(i0 + tid + 256 * u, M * nq - 1);  // past the end: a repeat, not stored
      src[u] = base + (int64_t)(idx / nq) * (a.n_pad / 4) + idx % nq;
      acc[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    for (int s0 = 0; s0 < a.splits; s0 += SJ) {
      float4 t[U][SJ];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < SJ; ++j) t[u][j] = src[u][min(s0 + j, a.splits - 1) * sstride];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < SJ; ++j)
          if (s0 + j < a.splits) acc[u].x += t[u][j].x, acc[u].y += t[u][j].y, acc[u].z += t[u][j].z,
                                 acc[u].w += t[u][j].w;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = i0 + tid + 256 * u;
      if (idx < M * nq) sums[(idx / nq) * kWideSumStride + idx % nq] = acc[u];
    }
  }
  __syncthreads();
  const float* sm = (const float*)sums;
  auto red = [&](int row, int col) { return sm[row * (4 * kWideSumStride) + (col - c0)]; };
  if (a.mode == TVP_EPI_ARGMAX) {  // best (value, smallest id) over the group's channels, 8 threads per row
    __shared__ int32_t rmap[128];
    if (tid < nc) rmap[tid] = a.rowmap[c0 + tid];
    __syncthreads();
    const int row = tid >> 3, part = tid & 7;  // part p scans channels p, p + 8, ...
    unsigned long long best = 0ull;
    if (row < M) {
      for (int cc = part; cc < nc; cc += 8) {
        const int32_t r = rmap[cc];
        if (r < 0) continue;
        const float v = red(row, c0 + cc);
        if (a.logits) a.logits[(int64_t)(r0 + row) * a.ldl + r] = v;
        const unsigned long long k = argmax_key(v, r);
        best = k > best ? k : best;
      }
    }
    for (int off = 4; off > 0; off >>= 1) {  // the row's 8 threads are adjacent lanes
      const unsigned long long o = __shfl_xor(best, off);
      best = o > best ? o : best;
    }
    if (row < M && part == 0) a.keys[(int64_t)g * a.m + r0 + row] = best;
    return;
  }
  GemmArgs b = a;  // row-indexed pointers moved to the block's first row
  b.cache_rowmap = 1;
  b.y = a.mode == TVP_EPI_F32 ? (void*)((float*)a.y + (int64_t)r0 * a.ldy)
                              : (void*)((uint16_t*)a.y + (int64_t)r0 * a.ldy);
  if (a.resid) b.resid = a.resid + (int64_t)r0 * a.ldr;
  if (a.pos) b.pos = a.pos + r0;
  if (a.slot) b.slot = a.slot + r0;
  if (a.rope_cs) b.rope_cs = a.rope_cs + (int64_t)r0 * a.d;  // (cos, sin) pairs of d/2 dims per row
  switch (a.mode) {
    case TVP_EPI_F32: epilogue<TVP_EPI_F32>(b, c0, nc, M, tid, 256, g, red); break;
    case TVP_EPI_BF16: epilogue<TVP_EPI_BF16>(b, c0, nc, M, tid, 256, g, red); break;
    case TVP_EPI_RESID: epilogue<TVP_EPI_RESID>(b, c0, nc, M, tid, 256, g, red); break;
    case TVP_EPI_SWIGLU: epilogue<TVP_EPI_SWIGLU>(b, c0, nc, M, tid, 256, g, red); break;
    default: epilogue<TVP_EPI_QKV>(b, c0, nc, M, tid, 256, g, red); break;
  }
}

struct GemmPlan {
  bool skinny;
  int MT, RB, TPW, RD, KW, TG, groups, splits, kbs, kps, ntasks, grid;
  int kbs_split, key_slots;
  int full_groups, rem_groups, rem_splits, rem_kps, rem_kbs;  // whole-K epilogues, see GemmArgs
  size_t keys_off, rem_off, cnt_off, scratch_bytes;
};

// Work decomposition.  Skinny (m <= 32): one workgroup per TPW tiles whose KW
// wavefronts split K (kbs <= 63 blocks each, so a wave's escape offsets fit
// one VGPR).  Wide (m > 32, or K too long for 8 waves of 63 blocks):
// workgroups of 4 x kWideTPW tiles sharing X through LDS, split K over
// workgroups (the splits finished by the next launch).
constexpr int kWideMaxSplits = 32;
// Cost of a split-sum byte against a record byte: the sums are written and
// read back within microseconds, mostly from the caches (measured: 0.5 beat
// 1 by 3.5% on the batched 27B-like step, 0.25 by 2%, 0 lost 50%).
constexpr double kWideSumWeight = 0.5;
constexpr int kWideTPW = 1;    // wide kernel: tiles per wavefront (a workgroup owns 4 x kWideTPW)
constexpr int kWideRD = 4;     // wide kernel: register-ring depth
constexpr int kWideRDBig = 3;  // ... above 128 rows (one tile per wavefront, two wavefronts per SIMD;
                               // measured: 3 beat 4 by 1.1% per batched step, 2 within noise)
constexpr int kTpw2MinTiles = 1024;  // tiles from which a workgroup takes two tiles
constexpr int kWavesPerCU = 12;      // skinny kernel: three wavefronts per SIMD (136-156 VGPRs)
// Waves per workgroup when every workgroup has a CU to itself (4 measured
// 0.8% slower per verify step).
constexpr int kKwOneRound = 8;
// Register-ring depth with one tile per workgroup (106 VGPRs; 3 measured
// 1.5% slower per verify step), the same with 16-row MFMA tiles, and with
// two tiles per workgroup.
constexpr int kRd1 = 2;
constexpr int kRd1M16 = kRd1;
constexpr int kRd2 = 2;

// Per-CU cost, in K blocks, of `gsplit` groups cut into `s` K slices of
// `kps` blocks (partial-sum epilogue): the busiest CU's blocks plus a fixed
// cost per workgroup; a CU holding a single workgroup streams slower.
constexpr double kSliceFixed = 4.0;   // measured: 4 (down in 3 slices) beat 2 (8 slices) by 0.35% per verify step, 1 lost 1%
constexpr double kSliceSingle = 1.5;
static double slice_cost(int gsplit, int s, int kps) {
  const int per_cu = (int)ceil_div((int64_t)gsplit * s, kNumCUs);
  const double cost = (double)per_cu * kps + kSliceFixed * per_cu;
  return per_cu <= 1 ? kSliceSingle * cost : cost;
}

// rem_ok: the epilogue can be applied by the slice of a remaining group that
// arrives last (not argmax, whose per-row reduction over 32 columns would
// run on too few lanes).
static GemmPlan make_plan(int64_t m, const tvp_w12_packed* w, int ksplit = 1, bool rem_ok = true) {
  GemmPlan p{};
  const int64_t n_pad = (int64_t)w->n_tiles * 32;
  const int nkb = w->n_kb;
  const bool partial = ksplit > 1;  // partial-sum epilogue: every group is cut into K slices
  p.MT = m <= 16 ? 16 : 32;
  p.RB = (int)ceil_div(m, p.MT);
  p.skinny = m <= 32 && nkb <= 8 * 63;
  if (p.skinny) {
    p.TPW = w->n_tiles >= kTpw2MinTiles ? 2 : 1;
    p.RD = p.TPW == 2 ? kRd2 : (p.MT == 16 ? kRd1M16 : kRd1);
    p.TG = p.TPW;
    p.groups = (int)ceil_div(w->n_tiles, p.TPW);
    p.splits = 1;
    p.kps = nkb;
    if (partial) {
      // K slices, summed in slice order by the consumer
      int best_s = 1, best_kps = std::max(nkb, 1);
      double best = 1e30;
      for (int sl = 1; sl <= std::min(ksplit, 16) && nkb > 0; ++sl) {
        const int kps = (int)ceil_div(nkb, sl);
        if ((int)ceil_div(nkb, kps) != sl || (sl > 1 && kps < 2)) continue;
        const double c = slice_cost(p.groups, sl, kps);
        if (c < best - 1e-9) best = c, best_s = sl, best_kps = kps;
      }
      p.splits = best_s;
      p.kps = nkb > 0 ? best_kps : 0;
    }
    const int nwg = partial ? p.groups * p.splits : p.groups;
    const int krange = partial ? p.kps : nkb;
    // Waves per workgroup: 4, or 2 when a CU would get more workgroups than it
    // holds at once (kWavesPerCU at this kernel's register use), so that all
    // of a CU's workgroups stream together instead of in two rounds; more
    // when a wave would exceed 63 blocks.
    p.KW = (int)ceil_div(nwg, kNumCUs) * 4 > kWavesPerCU ? 2 : 4;
    if (nwg <= kNumCUs) p.KW = kKwOneRound;  // one workgroup per CU at most
    while (p.KW < 8 && ceil_div(krange, p.KW) > 63) p.KW *= 2;
    p.KW = std::max(1, std::min(p.KW, std::max(krange, 1)));
    p.kbs = nkb > 0 ? (int)ceil_div(nkb, p.KW) : 0;
    p.kbs_split = p.kps > 0 ? (int)ceil_div(p.kps, p.KW) : 0;
    p.ntasks = nwg;
    p.grid = nwg;
    // Whole-K epilogue with more groups than CUs but not a multiple of them:
    // the groups past the last full round go out as K slices, about one
    // slice per CU, so no CU streams a whole extra group at the end.
    p.full_groups = p.groups;
    const int R = p.groups > kNumCUs ? p.groups % kNumCUs : 0;
    if (!partial && rem_ok && R > 0 && nkb >= 4) {
      // slices per remaining group: the fewest that minimise the busiest
      // CU's slices, ceil(R * s / CUs), times each slice's blocks plus the
      // fixed cost of a workgroup (measured: the 4B-like gate/up's 96
      // remaining groups in 2 slices of 20 blocks instead of 8 of 5 made
      // its verify step 3% faster; 27B-like shapes keep 8 slices)
      int sl = 1;
      double best = 1e30;
      for (int c = 2; c <= std::min(kRemMaxSplits, nkb / 2); ++c) {
        const double v = (double)ceil_div((int64_t)R * c, kNumCUs) * ((double)ceil_div(nkb, c) + kSliceFixed);
        if (v < best - 1e-9) best = v, sl = c;
      }
      p.rem_kps = (int)ceil_div(nkb, sl);
      p.rem_splits = (int)ceil_div(nkb, p.rem_kps);
      p.rem_kbs = (int)ceil_div(p.rem_kps, p.KW);
      p.rem_groups = R;
      p.full_groups = p.groups - R;
      p.grid = p.full_groups + R * p.rem_splits;
      p.ntasks = p.grid;
      if (p.rem_splits < 2) {  // no gain: whole groups
        p.rem_groups = 0;
        p.full_groups = p.groups;
        p.grid = p.ntasks = p.groups;
      }
    }
  } else {
    // K splits: the fewest that minimise the busiest CU's bytes -- its
    // workgroups' record blocks (4 tiles x 3 KB each) plus its share of the
    // fp32 split sums written and read back (none for a whole-K group),
    // weighted by kWideSumWeight
    p.TPW = kWideTPW;
    p.RD = 0;
    p.KW = 4;
    p.TG = 4 * kWideTPW;
    p.groups = (int)ceil_div(w->n_tiles, p.TG);
    int best_s = 1;
    double best = 1e300;
    for (int sl = 1; sl <= std::min(kWideMaxSplits, std::max(nkb, 1)); ++sl) {
      const int kbs = (int)ceil_div(std::max(nkb, 1), sl);
      if ((int)ceil_div(std::max(nkb, 1), kbs) != sl) continue;
      const double per_cu = (double)ceil_div((int64_t)p.groups * sl, kNumCUs) * kbs * p.TG * kBlockBytes;
      const double sums = sl > 1 ? kWideSumWeight * 2.0 * sl * m * n_pad * 4 / kNumCUs : 0.0;
      if (per_cu + sums < best - 1e-9) best = per_cu + sums, best_s = sl;
    }
    p.kbs = nkb > 0 ? (int)ceil_div(nkb, best_s) : 0;
    p.splits = best_s;
    p.ntasks = p.groups * p.splits;
    p.grid = p.ntasks;
  }
  // skinny: room to pack row-major activations; wide: split-K partial sums;
  // then the argmax key slots (one per workgroup / group)
  p.key_slots = p.skinny ? p.grid : (int)ceil_div(w->n_tiles, 4);  // wide: one per fix-up group of 4 tiles
  p.keys_off = p.skinny ? align_up((size_t)std::max(nkb, 1) * 4096, 256)
                        : align_up((size_t)p.splits * m * n_pad * 4, 256);
  p.rem_off = p.keys_off + align_up((size_t)std::max(p.key_slots, 1) * m * 8, 256);
  p.cnt_off = p.rem_off + align_up((size_t)p.rem_splits * m * p.rem_groups * p.TPW * 32 * 4, 256);
  p.scratch_bytes = p.cnt_off + align_up((size_t)p.rem_groups * 4, 256);
  return p;
}

template <int MT, int TPW, int RD, int HI8>
static void launch_skinny_fmt(const GemmArgs& a, const GemmPlan& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.grid), block((unsigned)(p.KW * 64));
  const size_t lds = (size_t)p.KW * TPW * 4096;
  if (a.fmt == kFmtI8) {  // the INT8 head: one epilogue
    w12_skinny_kernel<MT, TPW, RD, kEpiI8Approx, kFmtI8><<<grid, block, lds, stream>>>(a);
    return;
  }
  switch (a.mode) {
    case TVP_EPI_F32: w12_skinny_kernel<MT, TPW, RD, TVP_EPI_F32, HI8><<<grid, block, lds, stream>>>(a); break;
    case TVP_EPI_BF16: w12_skinny_kernel<MT, TPW, RD, TVP_EPI_BF16, HI8><<<grid, block, lds, stream>>>(a); break;
    case TVP_EPI_RESID: w12_skinny_kernel<MT, TPW, RD, TVP_EPI_RESID, HI8><<<grid, block, lds, stream>>>(a); break;
    case TVP_EPI_SWIGLU: w12_skinny_kernel<MT, TPW, RD, TVP_EPI_SWIGLU, HI8><<<grid, block, lds, stream>>>(a); break;
    case TVP_EPI_QKV: w12_skinny_kernel<MT, TPW, RD, TVP_EPI_QKV, HI8><<<grid, block, lds, stream>>>(a); break;
    case kEpiPartial: w12_skinny_kernel<MT, TPW, RD, kEpiPartial, HI8><<<grid, block, lds, stream>>>(a); break;
    default: w12_skinny_kernel<MT, TPW, RD, TVP_EPI_ARGMAX, HI8><<<grid, block, lds, stream>>>(a); break;
  }
}

template <int MT, int TPW, int RD>
static void launch_skinny(const GemmArgs& a, const GemmPlan& p, hipStream_t stream) {
  if (a.fmt == TVP_FMT_W12) launch_skinny_fmt<MT, TPW, RD, TVP_FMT_W12>(a, p, stream);
  else launch_skinny_fmt<MT, TPW, RD, TVP_FMT_HI8>(a, p, stream);
}

template <int RB>
static void launch_wide(const GemmArgs& a, int grid, hipStream_t stream) {
  // one tile per wavefront: the deepest ring that fits two wavefronts per
  // SIMD without spills; two tiles: one wavefront per SIMD
  constexpr int rd = kWideTPW == 2 ? kWideRD : (RB <= 4 ? kWideRD : kWideRDBig);
  w12_wide_kernel<RB, kWideTPW, rd><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(a);
  // partial-sum epilogues leave the split sums to their consumer; the fix-up
  // takes groups of 4 tiles (one ARGMAX key slot each)
  if (a.mode != kEpiPartial)
    w12_wide_fixup_kernel<<<dim3((unsigned)(ceil_div(a.n_tiles, 4) * ceil_div(a.m, 32))), dim3(256), 0,
                            stream>>>(a);
}

static int dispatch(const GemmPlan& p, const GemmArgs& a, hipStream_t stream) {
  if (p.grid > 0) {
    if (p.skinny) {
      if (p.MT == 16) {
        if (p.TPW == 2) launch_skinny<16, 2, kRd2>(a, p, stream);
        else launch_skinny<16, 1, kRd1M16>(a, p, stream);
      } else {
        if (p.TPW == 2) launch_skinny<32, 2, kRd2>(a, p, stream);
        else launch_skinny<32, 1, kRd1>(a, p, stream);
      }
    } else {
      switch ((int)ceil_div(a.m, 32)) {  // 32-row blocks
        case 1: launch_wide<1>(a, p.grid, stream); break;
        case 2: launch_wide<2>(a, p.grid, stream); break;
        case 3: launch_wide<3>(a, p.grid, stream); break;
        case 4: launch_wide<4>(a, p.grid, stream); break;
        case 5: launch_wide<5>(a, p.grid, stream); break;
        case 6: launch_wide<6>(a, p.grid, stream); break;
        default: return TVP_ERR_SHAPE;
      }
    }
    TVP_LAUNCH_CHECK();
  }
  if (a.mode == TVP_EPI_ARGMAX) {
    argmax_finalize_kernel<<<dim3((unsigned)a.m), 256, 0, stream>>>(a.keys, a.key_slots, a.m, a.argmax);
    TVP_LAUNCH_CHECK();
  }
  return TVP_OK;
}

int launch_rope_table(const int32_t* pos, int n, int d, double theta, float* rope_cs, hipStream_t stream) {
  if (n <= 0) return TVP_OK;
  const int total = n * (d / 2);
  rope_table_kernel<<<dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, stream>>>(pos, n, d, theta,
                                                                                    (float2*)rope_cs);
  TVP_LAUNCH_CHECK();
  return TVP_OK;
}

bool gemm_is_skinny(int64_t m, const tvp_w12_packed* w) { return make_plan(m, w).skinny; }

int gemm_key_slots(int64_t m, const tvp_w12_packed* w) { return make_plan(m, w, 1, false).key_slots; }
size_t gemm_keys_offset(int64_t m, const tvp_w12_packed* w) { return make_plan(m, w, 1, false).keys_off; }

int gemm_ksplits(int64_t m, const tvp_w12_packed* w, int ksplit) {
  const GemmPlan p = make_plan(m, w, ksplit);
  return p.splits;
}

void gemm_requirements(int64_t m, const tvp_w12_packed* w, int* groups, size_t* scratch_bytes, int ksplit) {
  const GemmPlan p = make_plan(m, w, ksplit);
  *groups = p.groups;
  *scratch_bytes = std::max(p.scratch_bytes, make_plan(m, w, ksplit, false).scratch_bytes);  // argmax: no split
}

int gemm_run(const uint16_t* x, const uint16_t* xp, int64_t m, int64_t ldx, const tvp_w12_packed* w,
             const tvp_gemm_epilogue* epi, int y_packed, void* scratch, size_t scratch_bytes,
             hipStream_t stream, int ksplit, const float* rope_cs, const I8EpiArgs* i8) {
  if (!w || !epi || !w->blob) return TVP_ERR_ARG;
  if (m < 1 || m > 192) return TVP_ERR_SHAPE;
  if (ksplit > 1 && epi->mode != kEpiPartial) return TVP_ERR_ARG;
  const GemmPlan p = make_plan(m, w, ksplit, epi->mode != TVP_EPI_ARGMAX && epi->mode != kEpiI8Approx);
  if (w->format != TVP_FMT_W12 && w->format != TVP_FMT_HI8 && w->format != kFmtI8) return TVP_ERR_FORMAT;
  if (w->format != TVP_FMT_W12 && !p.skinny) return TVP_ERR_SHAPE;  // 8-bit tiles: up to 32 rows
  if ((w->format == kFmtI8) != (epi->mode == kEpiI8Approx)) return TVP_ERR_ARG;
  if (xp) {
    if (!p.skinny || ((uintptr_t)xp) % 16 != 0) return TVP_ERR_ARG;
  } else if (w->k_in > 0) {
    if (!x || ldx < w->k_in) return TVP_ERR_ARG;
    if (((uintptr_t)x) % 16 != 0 || ldx % 8 != 0) return TVP_ERR_ARG;
  }
  if (y_packed && (!p.skinny || epi->mode != TVP_EPI_SWIGLU)) return TVP_ERR_ARG;
  if (!scratch || scratch_bytes < p.scratch_bytes) return TVP_ERR_WORKSPACE;
  GemmArgs a{};
  const uint8_t* blob = (const uint8_t*)w->blob;
  if (p.skinny && !xp) {  // pack the row-major activations into the scratch
    uint16_t* dst = (uint16_t*)scratch;
    const int nchunks = std::max(w->n_kb, 1) * 8;
    pack_x_kernel<<<dim3((unsigned)ceil_div((int64_t)nchunks * 32, 256)), dim3(256), 0, stream>>>(
        x, ldx, (int)m, (int)w->k_in, nchunks, dst);
    TVP_LAUNCH_CHECK();
    xp = dst;
  }
  a.fmt = w->format;
  a.x = x;
  a.xp = xp;
  a.y_packed = y_packed;
  a.ldx = ldx;
  a.m = (int)m;
  a.k_in = (int)w->k_in;
  a.rec = blob + w->off_rec;
  a.escoff = (const uint32_t*)(blob + w->off_escoff);
  a.esc = (const uint32_t*)(blob + w->off_esc);
  a.b2 = (const uint32_t*)(blob + w->off_b2);
  a.rowmap = (const int32_t*)(blob + w->off_rowmap);
  a.n_tiles = w->n_tiles;
  a.n_kb = w->n_kb;
  a.n_pad = w->n_tiles * 32;
  a.groups = p.groups;
  a.splits = p.splits;
  a.kbs = p.kbs;
  a.kps = p.kps;
  a.kbs_split = p.kbs_split;
  a.full_groups = p.full_groups;
  a.rem_splits = std::max(p.rem_splits, 1);
  a.rem_kps = p.rem_kps;
  a.rem_kbs = p.rem_kbs;
  a.rem_tpw = p.TPW;
  a.rpart = (float*)((uint8_t*)scratch + p.rem_off);
  a.ldrp = p.rem_groups * p.TPW * 32;
  a.rcnt = epi->counters;
  if (p.rem_groups > kGemmRemCounters) return TVP_ERR_SHAPE;  // fewer remaining groups than CUs by construction
  if (p.rem_groups > 0 && !a.rcnt) {  // the arrival counters live in the scratch: clear them first
    a.rcnt = (uint32_t*)((uint8_t*)scratch + p.cnt_off);
    zero_u32_kernel<<<dim3(1), dim3(256), 0, stream>>>(a.rcnt, p.rem_groups);
    TVP_LAUNCH_CHECK();
  }
  a.rope_cs = epi->mode == TVP_EPI_QKV ? rope_cs : nullptr;
  a.ntasks = p.ntasks;
  a.keys = (unsigned long long*)((uint8_t*)scratch + p.keys_off);
  a.key_slots = p.key_slots;
  a.part = (float*)scratch;  // wide: split-K partial sums
  a.mode = epi->mode;
  a.y = epi->y;
  a.ldy = epi->ldy;
  a.resid = epi->resid;
  a.ldr = epi->ldr;
  a.pos = epi->pos;
  a.slot = epi->slot;
  a.kc = epi->k_cache;
  a.vc = epi->v_cache;
  a.s_stride = epi->s_stride;
  a.theta = epi->rope_theta;
  a.argmax = epi->argmax;
  a.logits = epi->logits;
  a.ldl = epi->ldl;
  switch (epi->mode) {
    case TVP_EPI_F32:
    case TVP_EPI_BF16:
      if (!epi->y || epi->ldy < w->n_out) return TVP_ERR_ARG;
      break;
    case TVP_EPI_RESID:
      if (!epi->y || !epi->resid || epi->ldy < w->n_out || epi->ldr < w->n_out) return TVP_ERR_ARG;
      break;
    case TVP_EPI_SWIGLU:
      if (w->chan_map != TVP_CHAN_GATEUP) return TVP_ERR_ARG;
      if (!epi->y || (!y_packed && epi->ldy < w->map_a)) return TVP_ERR_ARG;  // packed: ldy unused
      break;
    case TVP_EPI_QKV:
      if (w->chan_map != TVP_CHAN_QKV) return TVP_ERR_ARG;
      if (!epi->y || !epi->pos || !epi->slot || !epi->k_cache || !epi->v_cache) return TVP_ERR_ARG;
      if (epi->ldy < (int64_t)w->map_a * w->map_c || epi->s_stride < 1 || !(epi->rope_theta > 0))
        return TVP_ERR_ARG;
      a.hq = w->map_a;
      a.hkv = w->map_b;
      a.d = w->map_c;
      break;
    case TVP_EPI_ARGMAX:
      if (!epi->argmax) return TVP_ERR_ARG;
      if (epi->logits && epi->ldl < w->n_out) return TVP_ERR_ARG;
      break;
    case kEpiI8Approx:
      if (!epi->logits || epi->ldl < w->n_out || !i8 || !i8->scale || !i8->r || !i8->fnorm || m > 32)
        return TVP_ERR_ARG;
      a.i8_scale = i8->scale;
      a.i8_r = i8->r;
      a.i8_fnorm = i8->fnorm;
      break;
    case kEpiPartial:
      // skinny: slices to y [slice][row][ldy]; wide: the split sums stay in
      // the scratch, [split][row][n_pad] at its start, for the consumer
      if (w->chan_map != TVP_CHAN_PLAIN) return TVP_ERR_ARG;
      if (p.skinny && (!epi->y || epi->ldy < w->n_out)) return TVP_ERR_ARG;
      break;
    default:
      return TVP_ERR_ARG;
  }
  if ((size_t)p.groups > kGemmMaxGroups) return TVP_ERR_SHAPE;
  return dispatch(p, a, stream);
}

}  // namespace tvp

using namespace tvp;

// Standalone GEMM workspace: the scratch of gemm_run, nothing else (no
// initial contents are needed).
static size_t gemm_ws_layout(int64_t m, const tvp_w12_packed* w, size_t* scr_bytes, int* groups) {
  gemm_requirements(m, w, groups, scr_bytes);
  return *scr_bytes;
}

extern "C" {

size_t w12_gemm_workspace(int64_t m, const tvp_w12_packed* w) {
  if (!w || m < 1 || m > 192) return 0;
  size_t b;
  int g;
  return gemm_ws_layout(m, w, &b, &g);
}

int w12_gemm_ex(const uint16_t* x, int64_t m, int64_t ldx, const tvp_w12_packed* w,
                const tvp_gemm_epilogue* epi, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!w || !epi) return TVP_ERR_ARG;
  if (m < 1 || m > 192) return TVP_ERR_SHAPE;
  size_t scr_bytes;
  int groups;
  const size_t need = gemm_ws_layout(m, w, &scr_bytes, &groups);
  if ((size_t)groups > kGemmMaxGroups) return TVP_ERR_SHAPE;
  if (!ws || ws_bytes < need) return TVP_ERR_WORKSPACE;
  if (epi->mode < TVP_EPI_F32 || epi->mode > TVP_EPI_ARGMAX) return TVP_ERR_ARG;
  if (epi->x_packed && !x) return TVP_ERR_ARG;
  return gemm_run(epi->x_packed ? nullptr : x, epi->x_packed ? x : nullptr, m, ldx, w, epi, epi->y_packed, ws,
                  ws_bytes, stream);
}

int64_t w12_packed_x_elems(int64_t k_in) { return k_in < 0 ? 0 : xpack_elems(k_in); }

int w12_pack_x(const uint16_t* x, int64_t m, int64_t ldx, int64_t k_in, uint16_t* xp, hipStream_t stream) {
  if (m < 1 || m > 32 || k_in < 0 || k_in > (1LL << 30)) return TVP_ERR_SHAPE;
  if (!xp || ((uintptr_t)xp) % 16 != 0) return TVP_ERR_ARG;
  if (k_in > 0 && (!x || ldx < k_in)) return TVP_ERR_ARG;
  const int64_t nchunks = xpack_elems(k_in) / 256;
  const int64_t threads = nchunks * 32;
  if (threads == 0) return TVP_OK;
  pack_x_kernel<<<dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0, stream>>>(x, ldx, (int)m, (int)k_in,
                                                                                  (int)nchunks, xp);
  TVP_LAUNCH_CHECK();
  return TVP_OK;
}

int w12_gemm(const uint16_t* x, int64_t m, int64_t ldx, const tvp_w12_packed* w, void* y,
             int64_t ldy, int y_fp32, void* ws, size_t ws_bytes, hipStream_t stream) {
  tvp_gemm_epilogue e{};
  e.mode = y_fp32 ? TVP_EPI_F32 : TVP_EPI_BF16;
  e.y = y;
  e.ldy = ldy;
  return w12_gemm_ex(x, m, ldx, w, &e, ws, ws_bytes, stream);
}

}  // extern "C"
