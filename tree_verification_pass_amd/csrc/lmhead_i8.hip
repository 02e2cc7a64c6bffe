// LM head on INT8 weights with a Cauchy-Schwarz certified candidate filter.
//
// SpecPilot summary (onedev.kr), section 무엇과 다른가: on one GPU the LM head
// filters candidate tokens with INT8 weights and a Cauchy-Schwarz error bound
// (the exact argmax is kept); on another the filter loses to the W12 head.
//
// Per vocabulary row v the 8 largest magnitudes are kept exactly (carried in
// the units of the row's scale, bf16); the rest are int8 at the scale
// s_v = fp32(t_v / 127), t_v the largest remaining magnitude.  With W^_v the
// weights the row stands for and r_v = ||W_v - W^_v||_2, the approximate
// logit a_v = f . W^_v satisfies |f . W_v - a_v| <= ||f||_2 r_v.  The pass:
//  1. ||f||_2 per row;
//  2. the skinny GEMM on the int8 tiles (decoded exactly to bf16, the escapes
//     patched like W12's), whose epilogue writes a_v and the per-workgroup
//     maximum of a_v - ||f|| r'_v, r'_v = r_v plus the fp32 accumulation error
//     of a_v;
//  3. tau = the row's maximum of those; every v with a_v + ||f|| r'_v >= tau
//     is a candidate (the exact argmax always is);
//  4. exact logits of the candidates from the canonical W12 rows of the same
//     weights, and their maximum (ties to the smallest id).
#include <math.h>

#include <algorithm>
#include <vector>

#include "internal.h"

namespace tvp {

constexpr int kI8Esc = 8;  // exact escapes per row

// key of a non-negative bf16 magnitude and a column: the largest magnitude
// wins, the smaller column on ties
__device__ inline uint32_t mag_key(uint32_t mag15, int k) { return (mag15 << 16) | (uint32_t)(0xFFFF - k); }

__device__ inline uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t m = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) m = red[w] > m ? red[w] : m;
  return m;
}

// fp64 sum over the workgroup in a fixed order (thread partials, then a
// shuffle tree, then wavefronts in order)
__device__ inline double block_sum_f64(double v, double* red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) s += red[w];
  return s;
}

// float -> next float toward +inf when x (double) is above it
__device__ inline float round_up_f32(double x) {
  float f = (float)x;
  if ((double)f < x) f = nextafterf(f, INFINITY);
  return f;
}

// One workgroup (256 threads) per row; the row (k_in <= 16384 bf16) in LDS.
__global__ __launch_bounds__(256) void i8_encode_kernel(const uint16_t* __restrict__ w, int k,
                                                        int8_t* __restrict__ q, float* __restrict__ scale,
                                                        uint16_t* __restrict__ esc_col, uint16_t* __restrict__ esc_val,
                                                        float* __restrict__ r, float* __restrict__ r_eff) {
  __shared__ uint16_t row[16384];
  __shared__ uint32_t red[4];
  __shared__ double redd[4];
  __shared__ int sel[kI8Esc];
  const int v = blockIdx.x, tid = threadIdx.x;
  const uint16_t* wr = w + (int64_t)v * k;
  for (int i = tid; i < k; i += 256) row[i] = wr[i];
  __syncthreads();
  const int ne = min(kI8Esc, k);
  // the ne largest magnitudes, one workgroup maximum each
  for (int e = 0; e < ne; ++e) {
    uint32_t best = 0;
    for (int i = tid; i < k; i += 256) {
      bool taken = false;
      for (int j = 0; j < e; ++j) taken |= sel[j] == i;
      if (!taken) {
        const uint32_t key = mag_key(row[i] & 0x7FFFu, i);
        best = key > best ? key : best;
      }
    }
    best = block_max_u32(best, red);
    if (tid == 0) sel[e] = 0xFFFF - (int)(best & 0xFFFFu);
    __syncthreads();
  }
  // largest remaining magnitude -> the scale
  uint32_t t = 0;
  for (int i = tid; i < k; i += 256) {
    bool taken = false;
    for (int j = 0; j < ne; ++j) taken |= sel[j] == i;
    if (!taken) t = max(t, (uint32_t)(row[i] & 0x7FFFu));
  }
  t = block_max_u32(t, red);
  const float tv = bf16_to_f32(t);
  const float s = tv > 0.0f ? tv / 127.0f : 1.0f;
  // int8 values, escapes in the scale's units, and the residual norms
  double err2 = 0.0, b2 = 0.0;
  for (int i = tid; i < k; i += 256) {
    const float x = bf16_to_f32(row[i]);
    const float ratio = x / s;
    bool taken = false;
    for (int j = 0; j < ne; ++j) taken |= sel[j] == i;
    float bv;
    if (taken) {
      bv = bf16_to_f32(f32_to_bf16(ratio));
      q[(int64_t)v * k + i] = 0;
    } else {
      bv = fminf(fmaxf(rintf(ratio), -127.0f), 127.0f);
      q[(int64_t)v * k + i] = (int8_t)bv;
    }
    const double d = (double)x - (double)s * (double)bv;
    err2 += d * d;
    b2 += (double)bv * (double)bv;
  }
  err2 = block_sum_f64(err2, redd);
  b2 = block_sum_f64(b2, redd);
  if (tid == 0) {
    // escapes in ascending column order
    int c[kI8Esc];
    for (int j = 0; j < ne; ++j) c[j] = sel[j];
    for (int a = 1; a < ne; ++a)
      for (int b = a; b > 0 && c[b - 1] > c[b]; --b) {
        const int tmp = c[b - 1];
        c[b - 1] = c[b];
        c[b] = tmp;
      }
    for (int j = 0; j < kI8Esc; ++j) {
      const int cj = j < ne ? c[j] : 0;
      esc_col[(int64_t)v * kI8Esc + j] = (uint16_t)cj;
      esc_val[(int64_t)v * kI8Esc + j] = j < ne ? (uint16_t)f32_to_bf16(bf16_to_f32(row[cj]) / s) : 0;
    }
    scale[v] = s;
    const double rr = sqrt(err2);
    r[v] = round_up_f32(rr);
    // plus a bound of the fp32 accumulation error of the approximate logit
    // (k terms: |f . s B - fl(f . s B)| <= k 2^-24 s ||f|| ||B||, doubled)
    r_eff[v] = round_up_f32(rr * (1.0 + 0x1p-20) + 2.0 * (double)k * 0x1p-24 * (double)s * sqrt(b2));
  }
}

// ||f_m||_2 of every row of the packed activations, slightly rounded up.
__global__ __launch_bounds__(256) void i8_fnorm_kernel(const uint16_t* __restrict__ xp, int k,
                                                       float* __restrict__ fnorm) {
  __shared__ float red[4];
  const int m = blockIdx.x, tid = threadIdx.x;
  float s = 0.0f;
  for (int i = tid; i < k; i += 256) {
    const float x = bf16_to_f32(xp[xpack_index(m, i)]);
    s = fmaf(x, x, s);
  }
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) fnorm[m] = sqrtf(red[0] + red[1] + red[2] + red[3]) * (1.0f + 0x1p-16f);
}

__device__ inline float key_value(unsigned long long k) {
  const uint32_t ord = (uint32_t)(k >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

// tau_m = max over the key slots; the row's result key and count cleared.
__global__ __launch_bounds__(256) void i8_tau_kernel(const unsigned long long* __restrict__ keys, int slots, int m,
                                                     float* __restrict__ tau, unsigned long long* __restrict__ best,
                                                     int32_t* __restrict__ n_cand) {
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
    tau[row] = key_value(k);
    best[row] = 0ull;
    n_cand[row] = 0;
  }
}

struct ExactRows {  // the canonical W12 head
  const uint8_t* hi;
  const uint8_t* lo;
  const uint8_t* base;
  const uint32_t* esc_ptr;
  const uint16_t* esc_idx;
  const uint16_t* esc_val;
  int64_t k_in;
};

// One workgroup (256 threads) per (256 vocabulary ids, row): the certified
// candidates of the chunk go to an LDS list; each wavefront then computes the
// exact logit of its candidates from the canonical W12 rows (fp32, a fixed
// lane and shuffle order) and folds (value, id) into the row's key with an
// atomic maximum, whose result does not depend on the order.
__global__ __launch_bounds__(256) void i8_rescore_kernel(const float* __restrict__ approx, int64_t lda, int vocab,
                                                         const float* __restrict__ r_eff,
                                                         const float* __restrict__ fnorm,
                                                         const float* __restrict__ tau, const uint16_t* __restrict__ xp,
                                                         ExactRows ex, unsigned long long* __restrict__ best,
                                                         int32_t* __restrict__ n_cand) {
  __shared__ int list[256];
  __shared__ int count;
  const int row = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int v = blockIdx.x * 256 + tid;
  if (tid == 0) count = 0;
  __syncthreads();
  if (v < vocab) {
    const float a = approx[row * lda + v];
    if (a + fnorm[row] * r_eff[v] >= tau[row]) list[atomicAdd(&count, 1)] = v;
  }
  __syncthreads();
  const int nc = count;
  if (tid == 0 && nc > 0) atomicAdd(&n_cand[row], nc);
  const int64_t k = ex.k_in, lo_w = (k + 1) / 2;
  for (int c = wave; c < nc; c += 4) {
    const int id = list[c];
    const uint32_t bsh = (uint32_t)ex.base[id] << 7;
    const uint8_t* hr = ex.hi + (int64_t)id * k;
    const uint8_t* lr = ex.lo + (int64_t)id * lo_w;
    float acc = 0.0f;
    for (int64_t i = lane; i < k; i += 64) {
      const uint32_t rec = ((uint32_t)hr[i] << 4) | ((lr[i >> 1] >> ((i & 1) * 4)) & 15u);
      const float wv = bf16_to_f32(((rec & 0x800u) << 4) | ((rec & 0x7FFu) + bsh));
      acc = fmaf(bf16_to_f32(xp[xpack_index(row, i)]), wv, acc);
    }
    // escaped slots decoded record 0; replace that value by the escape's
    const float w0 = bf16_to_f32(bsh);
    for (uint32_t e = ex.esc_ptr[id] + lane; e < ex.esc_ptr[id + 1]; e += 64) {
      const int i = ex.esc_idx[e];
      acc = fmaf(bf16_to_f32(xp[xpack_index(row, i)]), bf16_to_f32(ex.esc_val[e]) - w0, acc);
    }
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) {
      const uint32_t u = __float_as_uint(acc);
      const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
      const unsigned long long key = ((unsigned long long)ord << 32) | (0xFFFFFFFFu - (uint32_t)id);
      __hip_atomic_fetch_max(&best[row], key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

__global__ void i8_out_kernel(const unsigned long long* __restrict__ best, int m, int32_t* __restrict__ argmax) {
  const int row = threadIdx.x;
  if (row < m) argmax[row] = (int32_t)(0xFFFFFFFFu - (uint32_t)(best[row] & 0xFFFFFFFFull));
}

}  // namespace tvp

using namespace tvp;

// Workspace of the argmax: ||f|| [32], tau [32], result keys [32] (u64),
// approximate logits [m][vocab] when the caller gives none, then the GEMM's
// scratch.
struct I8Layout {
  size_t off_fn, off_tau, off_best, off_apx, off_gemm, gemm_bytes, bytes;
};

static I8Layout i8_layout(int64_t m, const tvp_lmhead_i8* h, bool own_approx) {
  I8Layout L{};
  size_t off = 0;
  L.off_fn = off;
  off = align_up(off + 32 * 4, 256);
  L.off_tau = off;
  off = align_up(off + 32 * 4, 256);
  L.off_best = off;
  off = align_up(off + 32 * 8, 256);
  L.off_apx = off;
  if (own_approx) off = align_up(off + (size_t)m * h->vocab * 4, 256);
  L.off_gemm = off;
  int groups;
  gemm_requirements(m, &h->tiles, &groups, &L.gemm_bytes);
  L.bytes = off + align_up(L.gemm_bytes, 256);
  return L;
}

extern "C" {

int lmhead_i8_tiles_size(int64_t vocab, int64_t k_in, tvp_w12_packed* p) {
  if (!p || vocab < 1 || k_in < 1) return TVP_ERR_ARG;
  if (k_in > 16384) return TVP_ERR_SHAPE;
  const int st = w12_pack_hi8_size(vocab, k_in, vocab * std::min<int64_t>(kI8Esc, k_in), TVP_CHAN_PLAIN, 0, 0, 0, p);
  if (st == TVP_OK) p->format = kFmtI8;
  return st;
}

size_t lmhead_i8_encode_workspace(int64_t vocab, int64_t k_in) {
  if (vocab < 1 || k_in < 1) return 0;
  // zero nibble plane, base bytes, escape pointers, then the packer's scratch
  const size_t lo = align_up((size_t)vocab * ((k_in + 1) / 2), 256);
  const size_t bs = align_up((size_t)vocab, 256);
  const size_t ptr = align_up((size_t)(vocab + 1) * 4, 256);
  return lo + bs + ptr + w12_pack_workspace(vocab, k_in);
}

int lmhead_i8_encode(const uint16_t* w, tvp_lmhead_i8* h, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!w || !h || !h->q || !h->scale || !h->esc_col || !h->esc_val || !h->r || !h->r_eff || !h->tiles.blob)
    return TVP_ERR_ARG;
  const int64_t V = h->vocab, k = h->k_in;
  if (V < 1 || k < 1 || k > 16384 || V > 0x7FFFFFFF) return TVP_ERR_SHAPE;
  tvp_w12_packed want;
  if (lmhead_i8_tiles_size(V, k, &want) != TVP_OK || want.bytes != h->tiles.bytes || want.n_tiles != h->tiles.n_tiles)
    return TVP_ERR_SHAPE;
  const size_t need = lmhead_i8_encode_workspace(V, k);
  if (!ws || ws_bytes < need) return TVP_ERR_WORKSPACE;
  i8_encode_kernel<<<dim3((unsigned)V), dim3(256), 0, stream>>>(w, (int)k, h->q, h->scale, h->esc_col, h->esc_val,
                                                                h->r, h->r_eff);
  TVP_LAUNCH_CHECK();
  // pack the int8 values as the 8-bit tile layout: they are the "hi" plane of
  // a record tensor with 8 escapes per row (the scale units' bf16 values)
  uint8_t* b = (uint8_t*)ws;
  const size_t lo = align_up((size_t)V * ((k + 1) / 2), 256), bs = align_up((size_t)V, 256);
  uint8_t* zero_lo = b;
  uint8_t* ones = b + lo;
  uint32_t* ptr = (uint32_t*)(b + lo + bs);
  void* pws = b + lo + bs + align_up((size_t)(V + 1) * 4, 256);
  const int64_t ne = std::min<int64_t>(kI8Esc, k);
  TVP_CHECK_HIP(hipMemsetAsync(zero_lo, 0, (size_t)V * ((k + 1) / 2), stream));
  TVP_CHECK_HIP(hipMemsetAsync(ones, 1, (size_t)V, stream));
  std::vector<uint32_t> hp((size_t)V + 1);
  for (int64_t i = 0; i <= V; ++i) hp[i] = (uint32_t)(i * ne);
  TVP_CHECK_HIP(hipMemcpyAsync(ptr, hp.data(), hp.size() * 4, hipMemcpyHostToDevice, stream));
  // with fewer columns than escapes per row, the rows' escape lists are the
  // first ne entries of each group of 8: compact them first (not needed for
  // k >= 8, the only case of the LM head)
  if (ne != kI8Esc) return TVP_ERR_SHAPE;
  tvp_w12 t{};
  t.n_out = V;
  t.k_in = k;
  t.n_esc = V * ne;
  t.hi = (uint8_t*)h->q;
  t.lo = zero_lo;
  t.base = ones;
  t.esc_ptr = ptr;
  t.esc_idx = h->esc_col;
  t.esc_val = h->esc_val;
  tvp_w12_packed p = h->tiles;
  p.format = TVP_FMT_HI8;
  const int st = pack_tiles(&t, &p, pws, w12_pack_workspace(V, k), stream, TVP_FMT_HI8);
  if (st != TVP_OK) return st;
  p.format = kFmtI8;
  h->tiles = p;
  return TVP_OK;
}

size_t lmhead_i8_argmax_workspace(int64_t m, const tvp_lmhead_i8* h) {
  if (!h || m < 1 || m > 32) return 0;
  return i8_layout(m, h, true).bytes;
}

int lmhead_i8_argmax(const uint16_t* xp, int64_t m, const tvp_lmhead_i8* h, const tvp_w12* exact, int32_t* argmax,
                     int32_t* n_cand, float* approx, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!xp || !h || !exact || !argmax || !n_cand || !h->scale || !h->r_eff || !h->tiles.blob) return TVP_ERR_ARG;
  if (m < 1 || m > 32) return TVP_ERR_SHAPE;
  if (exact->n_out != h->vocab || exact->k_in != h->k_in || h->tiles.format != kFmtI8) return TVP_ERR_SHAPE;
  if (!exact->hi || !exact->lo || !exact->base || !exact->esc_ptr || (exact->n_esc > 0 && !exact->esc_idx))
    return TVP_ERR_ARG;
  if ((uintptr_t)xp % 16) return TVP_ERR_ARG;
  const I8Layout L = i8_layout(m, h, approx == nullptr);
  if (!ws || ws_bytes < L.bytes) return TVP_ERR_WORKSPACE;
  uint8_t* b = (uint8_t*)ws;
  float* fnorm = (float*)(b + L.off_fn);
  float* tau = (float*)(b + L.off_tau);
  unsigned long long* best = (unsigned long long*)(b + L.off_best);
  float* apx = approx ? approx : (float*)(b + L.off_apx);
  const int V = (int)h->vocab;
  i8_fnorm_kernel<<<dim3((unsigned)m), dim3(256), 0, stream>>>(xp, (int)h->k_in, fnorm);
  TVP_LAUNCH_CHECK();
  tvp_gemm_epilogue e{};
  e.mode = kEpiI8Approx;
  e.logits = apx;
  e.ldl = V;
  I8EpiArgs i8{h->scale, h->r_eff, fnorm};
  int st = gemm_run(nullptr, xp, m, 0, &h->tiles, &e, 0, b + L.off_gemm, L.gemm_bytes, stream, 1, nullptr, &i8);
  if (st != TVP_OK) return st;
  // the GEMM's key slots: one per workgroup of its launch, at the scratch's key region
  const int slots = gemm_key_slots(m, &h->tiles);
  const unsigned long long* keys = (const unsigned long long*)(b + L.off_gemm + gemm_keys_offset(m, &h->tiles));
  i8_tau_kernel<<<dim3((unsigned)m), dim3(256), 0, stream>>>(keys, slots, (int)m, tau, best, n_cand);
  TVP_LAUNCH_CHECK();
  ExactRows ex{exact->hi, exact->lo, exact->base, exact->esc_ptr, exact->esc_idx, exact->esc_val, exact->k_in};
  i8_rescore_kernel<<<dim3((unsigned)ceil_div(V, 256), (unsigned)m), dim3(256), 0, stream>>>(
      apx, V, V, h->r_eff, fnorm, tau, xp, ex, best, n_cand);
  TVP_LAUNCH_CHECK();
  i8_out_kernel<<<1, 32, 0, stream>>>(best, (int)m, argmax);
  TVP_LAUNCH_CHECK();
  return TVP_OK;
}

}  // extern "C"
