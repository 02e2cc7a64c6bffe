// W12 conversion on the GPU: encoder (two phases), decoder, and the packer that
// builds the tiled copy the GEMM streams.
//
// Format: SpecPilot summary (onedev.kr), section 무엇과 다른가 -- per output
// channel a 16-binade window of exponents; in-window weights become a 12-bit
// record (sign, 4-bit exponent offset, 7 mantissa bits), everything else is an
// exact escape.  The window holding the most normal exponents wins, the
// smallest base on ties; records are sign<<11 | off<<7 | mantissa, stored as
// a high byte (record >> 4) and a low nibble (two per byte, even k low).
#include <algorithm>
#include <vector>

#include "common.h"

namespace tvp {

// ---------------------------------------------------------------- encoder

// One workgroup per channel: exponent histogram in LDS, then the best window.
__global__ __launch_bounds__(256) void w12_count_kernel(const uint16_t* __restrict__ w,
                                                        int64_t k_in, uint8_t* __restrict__ base,
                                                        uint32_t* __restrict__ counts) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t best[4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  hist[tid] = 0;
  __syncthreads();
  const uint16_t* wr = w + row * k_in;
  for (int64_t k = tid; k < k_in; k += 256) {
    uint32_t e = (wr[k] >> 7) & 0xFFu;
    if (e >= 1 && e <= 254) atomicAdd(&hist[e], 1u);
  }
  __syncthreads();
  // key = in-window count * 256 + (255 - b): the max picks the largest count,
  // then the smallest b.
  uint32_t key = 0;
  if (tid >= 1 && tid <= 239) {
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += hist[tid + i];
    key = s * 256u + (255u - (uint32_t)tid);
  }
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = __shfl_xor(key, off);
    key = o > key ? o : key;
  }
  if ((tid & 63) == 0) best[tid >> 6] = key;
  __syncthreads();
  if (tid == 0) {
    uint32_t m = best[0];
    for (int i = 1; i < 4; ++i) m = best[i] > m ? best[i] : m;
    const uint32_t b = 255u - (m & 255u);
    base[row] = (uint8_t)b;
    counts[row] = (uint32_t)(k_in - (int64_t)(m >> 8));
  }
}

// Exclusive scan of n counts into out[0..n] with one workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void scan_u32_kernel(const uint32_t* __restrict__ in, int64_t n,
                                                         uint32_t* __restrict__ out) {
  __shared__ uint32_t wsum[16];
  __shared__ uint32_t carry;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int64_t b0 = 0; b0 < n; b0 += 1024) {
    const int64_t i = b0 + tid;
    const uint32_t v = i < n ? in[i] : 0u;
    uint32_t x = v;
    for (int off = 1; off < 64; off <<= 1) {
      uint32_t y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    uint32_t pre = carry;
    for (int j = 0; j < wv; ++j) pre += wsum[j];
    if (i < n) out[i] = pre + x - v;
    __syncthreads();
    if (tid == 1023) carry = pre + x;
    __syncthreads();
  }
  if (tid == 0) out[n] = carry;
}

// One workgroup per channel; each pass covers 512 columns, two per thread.
__global__ __launch_bounds__(256) void w12_encode_kernel(const uint16_t* __restrict__ w,
                                                         int64_t k_in, const uint8_t* __restrict__ base,
                                                         const uint32_t* __restrict__ esc_ptr,
                                                         uint8_t* __restrict__ hi, uint8_t* __restrict__ lo,
                                                         uint16_t* __restrict__ esc_idx,
                                                         uint16_t* __restrict__ esc_val) {
  __shared__ uint32_t wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t row = blockIdx.x;
  const uint32_t b = base[row];
  const uint16_t* wr = w + row * k_in;
  const int64_t lo_w = (k_in + 1) / 2;
  uint32_t run = esc_ptr[row];
  for (int64_t k0 = 0; k0 < k_in; k0 += 512) {
    const int64_t k = k0 + 2 * tid;
    uint32_t rec[2] = {0, 0}, esc[2] = {0, 0}, val[2] = {0, 0};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (k + q < k_in) {
        const uint32_t u = wr[k + q];
        const uint32_t e = (u >> 7) & 0xFFu;
        if (e >= b && e <= b + 15u) {
          rec[q] = ((u >> 15) << 11) | ((e - b) << 7) | (u & 0x7Fu);
        } else {
          esc[q] = 1;
          val[q] = u;
        }
      }
    }
    if (k < k_in) hi[row * k_in + k] = (uint8_t)(rec[0] >> 4);
    if (k + 1 < k_in) hi[row * k_in + k + 1] = (uint8_t)(rec[1] >> 4);
    if (k < k_in) lo[row * lo_w + k / 2] = (uint8_t)((rec[0] & 15u) | ((rec[1] & 15u) << 4));
    // exclusive prefix of escapes across the workgroup, in column order
    const uint32_t c = esc[0] + esc[1];
    uint32_t x = c;
    for (int off = 1; off < 64; off <<= 1) {
      uint32_t y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    uint32_t pre = run;
    for (int j = 0; j < wv; ++j) pre += wsum[j];
    pre += x - c;
    if (esc[0]) {
      esc_idx[pre] = (uint16_t)k;
      esc_val[pre] = (uint16_t)val[0];
      ++pre;
    }
    if (esc[1]) {
      esc_idx[pre] = (uint16_t)(k + 1);
      esc_val[pre] = (uint16_t)val[1];
    }
    run += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
}

// ---------------------------------------------------------------- decoder

__global__ __launch_bounds__(256) void w12_decode_kernel(const uint8_t* __restrict__ hi,
                                                         const uint8_t* __restrict__ lo,
                                                         const uint8_t* __restrict__ base,
                                                         const uint32_t* __restrict__ esc_ptr,
                                                         const uint16_t* __restrict__ esc_idx,
                                                         const uint16_t* __restrict__ esc_val,
                                                         int64_t k_in, uint16_t* __restrict__ out) {
  const int64_t row = blockIdx.x;
  const uint32_t b = base[row];
  const int64_t lo_w = (k_in + 1) / 2;
  uint16_t* o = out + row * k_in;
  for (int64_t k = threadIdx.x; k < k_in; k += 256) {
    const uint32_t nib = (lo[row * lo_w + k / 2] >> ((k & 1) * 4)) & 15u;
    const uint32_t r = ((uint32_t)hi[row * k_in + k] << 4) | nib;
    o[k] = (uint16_t)(((r & 0x800u) << 4) | ((r & 0x7FFu) + (b << 7)));
  }
  __syncthreads();
  for (uint32_t e = esc_ptr[row] + threadIdx.x; e < esc_ptr[row + 1]; e += 256) o[esc_idx[e]] = esc_val[e];
}

// ----------------------------------------------------------------- packer
// Packed tile block (tile t = 32 packed channels, block j = 64 columns):
// lane l (channel c = l & 31, half h = l >> 5) owns 48 bytes, as dwords
// D[0..11] at byte offsets s*1024 + l*16 + 4*i (s = i / 4).  The lane's
// 32 weights are w[s][i] = column 16 s + 8 h + i (s, i < 4, 8).
//  - D[2s+q] (q = 0, 1) holds the low record bytes of w[s][4q..4q+3] in byte
//    order (4q, 4q+2, 4q+1, 4q+3), so masking with 0x00FF00FF (after a shift
//    by 8 for the odd pair) puts a pair in the low bytes of two halfwords;
//  - D[8+s] holds, for each pair p of w[s], the bits (sign, off>>1) of both
//    records placed so that rotl(D, 4p) & 0x87008700 lands them in the high
//    bytes of the two halfwords.
// Decode of pair p:  (rotl(D[8+s],4p) & 0x87008700) + lowbytes + (base<<7)*0x10001.
// Escaped slots hold record 0 and are overwritten from the escape list, whose
// entries are (bf16 << 16) | halfword index in the 32x64 bf16 tile laid out
// as [column/8][channel][column%8].

__device__ inline uint32_t rotr32(uint32_t x, int r) { return r == 0 ? x : (x >> r) | (x << (32 - r)); }

__global__ __launch_bounds__(64) void pack_count_kernel(const uint32_t* __restrict__ esc_ptr,
                                                        const uint16_t* __restrict__ esc_idx,
                                                        const int32_t* __restrict__ rowmap,
                                                        int32_t n_kb, uint32_t* __restrict__ counts) {
  const int64_t unit = blockIdx.x;
  const int64_t t = unit / n_kb;
  const int j = (int)(unit % n_kb);
  const int c = threadIdx.x;
  uint32_t cnt = 0;
  if (c < 32) {
    const int32_t r = rowmap[t * 32 + c];
    if (r >= 0) {
      uint32_t a = esc_ptr[r], z = esc_ptr[r + 1];
      // lower bounds of columns 64 j and 64 (j+1) in the ascending list
      uint32_t lo0 = a, hi0 = z;
      while (lo0 < hi0) { uint32_t m = (lo0 + hi0) / 2; if (esc_idx[m] < 64u * j) lo0 = m + 1; else hi0 = m; }
      uint32_t lo1 = lo0, hi1 = z;
      while (lo1 < hi1) { uint32_t m = (lo1 + hi1) / 2; if (esc_idx[m] < 64u * (j + 1)) lo1 = m + 1; else hi1 = m; }
      cnt = lo1 - lo0;
    }
  }
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
  if (c == 0) counts[unit] = cnt;
}

// HI8 (the 8-bit leading view): each lane owns 32 bytes, dwords D[0..7] at
// byte offsets s*1024 + l*16 + 4*i (s = i / 4), D[2s+q] holding the hi bytes
// (record >> 4) of w[s][4q..4q+3] in the same byte order (4q, 4q+2, 4q+1,
// 4q+3), so masking with 0x00FF00FF (after a shift by 8 for the odd pair)
// spreads a pair into two halfwords.  Decode of such a pair x:
//   (((x & 0x007F007F) << 4) + (base<<7)*0x10001) | ((x & 0x00800080) << 8).
template <bool HI8>
__global__ __launch_bounds__(64) void pack_write_kernel(const uint8_t* __restrict__ hi,
                                                        const uint8_t* __restrict__ lo,
                                                        const uint8_t* __restrict__ base,
                                                        const uint32_t* __restrict__ esc_ptr,
                                                        const uint16_t* __restrict__ esc_idx,
                                                        const uint16_t* __restrict__ esc_val,
                                                        const int32_t* __restrict__ rowmap,
                                                        int64_t k_in, int32_t n_kb,
                                                        const uint32_t* __restrict__ escoff,
                                                        uint8_t* __restrict__ rec_out,
                                                        uint32_t* __restrict__ esc_out) {
  const int64_t unit = blockIdx.x;
  const int64_t t = unit / n_kb;
  const int j = (int)(unit % n_kb);
  const int l = threadIdx.x, c = l & 31, h = l >> 5;
  const int32_t r = rowmap[t * 32 + c];
  const int64_t lo_w = (k_in + 1) / 2;
  uint32_t D[12];
#pragma unroll
  for (int i = 0; i < 12; ++i) D[i] = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint32_t recs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t k = 64LL * j + 16 * s + 8 * h + i;
      uint32_t rc = 0;
      if (r >= 0 && k < k_in) {
        const uint32_t nib = (lo[(int64_t)r * lo_w + k / 2] >> ((k & 1) * 4)) & 15u;
        rc = ((uint32_t)hi[(int64_t)r * k_in + k] << 4) | nib;
      }
      recs[i] = rc;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      D[2 * s + q] = (recs[4 * q] & 0xFFu) | ((recs[4 * q + 2] & 0xFFu) << 8) |
                     ((recs[4 * q + 1] & 0xFFu) << 16) | ((recs[4 * q + 3] & 0xFFu) << 24);
    }
    uint32_t hn = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t ra = recs[2 * p], rb = recs[2 * p + 1];
      const uint32_t hba = (((ra >> 11) & 1u) << 7) | ((ra >> 8) & 7u);
      const uint32_t hbb = (((rb >> 11) & 1u) << 7) | ((rb >> 8) & 7u);
      hn |= rotr32((hba << 8) | (hbb << 24), 4 * p);
    }
    D[8 + s] = hn;
  }
  const int64_t n_tiles = (int64_t)gridDim.x / n_kb;  // one workgroup per (tile, k-block)
  if constexpr (HI8) {
    uint32_t Q[8];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t h8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t k = 64LL * j + 16 * s + 8 * h + i;
        h8[i] = (r >= 0 && k < k_in) ? (uint32_t)hi[(int64_t)r * k_in + k] : 0u;
      }
#pragma unroll
      for (int q = 0; q < 2; ++q)
        Q[2 * s + q] = h8[4 * q] | (h8[4 * q + 2] << 8) | (h8[4 * q + 1] << 16) | (h8[4 * q + 3] << 24);
    }
    uint4* blk = (uint4*)(rec_out + rec_block(t, j, n_tiles) * (int64_t)kBlockBytesHi8);
#pragma unroll
    for (int s = 0; s < 2; ++s) blk[s * 64 + l] = make_uint4(Q[4 * s], Q[4 * s + 1], Q[4 * s + 2], Q[4 * s + 3]);
  } else {
    uint4* blk = (uint4*)(rec_out + rec_block(t, j, n_tiles) * (int64_t)kBlockBytes);
#pragma unroll
    for (int s = 0; s < 3; ++s) blk[s * 64 + l] = make_uint4(D[4 * s], D[4 * s + 1], D[4 * s + 2], D[4 * s + 3]);
  }

  // escape entries, channel by channel in packed order, ascending column
  uint32_t lo0 = 0, lo1 = 0;
  if (h == 0 && r >= 0) {
    uint32_t a = esc_ptr[r], z = esc_ptr[r + 1];
    uint32_t x0 = a, y0 = z;
    while (x0 < y0) { uint32_t m = (x0 + y0) / 2; if (esc_idx[m] < 64u * j) x0 = m + 1; else y0 = m; }
    uint32_t x1 = x0, y1 = z;
    while (x1 < y1) { uint32_t m = (x1 + y1) / 2; if (esc_idx[m] < 64u * (j + 1)) x1 = m + 1; else y1 = m; }
    lo0 = x0;
    lo1 = x1;
  }
  const uint32_t cnt = lo1 - lo0;
  uint32_t x = cnt;
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_up(x, off);
    if (l >= off) x += y;
  }
  uint32_t pos = escoff[unit] + x - cnt;
  for (uint32_t e = lo0; e < lo1; ++e) {
    const uint32_t kk = esc_idx[e] - 64u * j;
    const uint32_t half = ((kk >> 3) * 32u + (uint32_t)c) * 8u + (kk & 7u);
    esc_out[pos++] = ((uint32_t)esc_val[e] << 16) | half;
  }
}

__global__ void pack_b2_kernel(const uint8_t* __restrict__ base, const int32_t* __restrict__ rowmap,
                               int64_t n_pad, uint32_t* __restrict__ b2) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= n_pad) return;
  const int32_t r = rowmap[p];
  const uint32_t b = r >= 0 ? base[r] : 1u;
  b2[p] = (b << 7) * 0x10001u;
}

static int build_rowmap(const tvp_w12_packed* p, std::vector<int32_t>& map) {
  const int64_t n_pad = (int64_t)p->n_tiles * kTileN;
  map.assign(n_pad, -1);
  if (p->chan_map == TVP_CHAN_PLAIN) {
    for (int64_t i = 0; i < p->n_out; ++i) map[i] = (int32_t)i;
  } else if (p->chan_map == TVP_CHAN_GATEUP) {
    const int64_t F = p->map_a;
    for (int64_t t = 0; t < p->n_tiles; ++t)
      for (int c = 0; c < 32; ++c) {
        const int64_t j = 16 * t + (c & 15);
        if (j < F) map[t * 32 + c] = (int32_t)(c < 16 ? j : F + j);
      }
  } else if (p->chan_map == TVP_CHAN_QKV) {
    const int64_t hq = p->map_a, hkv = p->map_b, d = p->map_c;
    const int64_t tph = d / 32;  // tiles per head
    const int64_t rot_heads = hq + hkv;
    for (int64_t t = 0; t < p->n_tiles; ++t)
      for (int c = 0; c < 32; ++c) {
        int64_t row;
        if (t < rot_heads * tph) {
          const int64_t head = t / tph, u = t % tph;
          const int64_t dim = c < 16 ? 16 * u + c : d / 2 + 16 * u + (c - 16);
          row = head * d + dim;
        } else {
          row = rot_heads * d + (t - rot_heads * tph) * 32 + c;
        }
        if (row < p->n_out) map[t * 32 + c] = (int32_t)row;
      }
  } else {
    return TVP_ERR_ARG;
  }
  return TVP_OK;
}

}  // namespace tvp

using namespace tvp;

extern "C" {

const char* tvp_status_string(int s) {
  switch (s) {
    case TVP_OK: return "ok";
    case TVP_ERR_ARG: return "invalid argument";
    case TVP_ERR_SHAPE: return "invalid or unsupported shape";
    case TVP_ERR_TREE: return "malformed draft tree";
    case TVP_ERR_CAPACITY: return "capacity exceeded";
    case TVP_ERR_FORMAT: return "malformed W12 tensor";
    case TVP_ERR_WORKSPACE: return "workspace missing or too small";
    case TVP_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int w12_encode_count(const uint16_t* w, int64_t n_out, int64_t k_in, uint8_t* base,
                     uint32_t* esc_ptr, int64_t* h_n_esc, hipStream_t stream) {
  if (!h_n_esc || n_out < 0 || k_in < 0) return TVP_ERR_ARG;
  if (k_in > 65536) return TVP_ERR_SHAPE;
  if (n_out == 0) { *h_n_esc = 0; return TVP_OK; }
  if (!w || !base || !esc_ptr) return TVP_ERR_ARG;
  if (n_out > 0x7FFFFFFF) return TVP_ERR_SHAPE;
  // Per-channel escape counts land in esc_ptr[1..n]; the scan then turns them
  // into offsets in place (each pass reads index i+1 before a barrier and
  // writes index i after it).
  w12_count_kernel<<<dim3((unsigned)n_out), dim3(256), 0, stream>>>(w, k_in, base, esc_ptr + 1);
  TVP_LAUNCH_CHECK();
  scan_u32_kernel<<<1, 1024, 0, stream>>>(esc_ptr + 1, n_out, esc_ptr);
  TVP_LAUNCH_CHECK();
  uint32_t total = 0;
  TVP_CHECK_HIP(hipMemcpyAsync(&total, esc_ptr + n_out, 4, hipMemcpyDeviceToHost, stream));
  TVP_CHECK_HIP(hipStreamSynchronize(stream));
  *h_n_esc = total;
  return TVP_OK;
}

int w12_encode(const uint16_t* w, const tvp_w12* t, hipStream_t stream) {
  if (!t || t->n_out < 0 || t->k_in < 0) return TVP_ERR_ARG;
  if (t->k_in > 65536) return TVP_ERR_SHAPE;
  if (t->n_out == 0 || t->k_in == 0) return TVP_OK;
  if (!w || !t->hi || !t->lo || !t->base || !t->esc_ptr) return TVP_ERR_ARG;
  if (t->n_esc > 0 && (!t->esc_idx || !t->esc_val)) return TVP_ERR_ARG;
  w12_encode_kernel<<<dim3((unsigned)t->n_out), dim3(256), 0, stream>>>(
      w, t->k_in, t->base, t->esc_ptr, t->hi, t->lo, t->esc_idx, t->esc_val);
  TVP_LAUNCH_CHECK();
  return TVP_OK;
}

int w12_decode(const tvp_w12* t, uint16_t* out, hipStream_t stream) {
  if (!t || t->n_out < 0 || t->k_in < 0) return TVP_ERR_ARG;
  if (t->n_out == 0 || t->k_in == 0) return TVP_OK;
  if (!out || !t->hi || !t->lo || !t->base || !t->esc_ptr) return TVP_ERR_ARG;
  w12_decode_kernel<<<dim3((unsigned)t->n_out), dim3(256), 0, stream>>>(
      t->hi, t->lo, t->base, t->esc_ptr, t->esc_idx, t->esc_val, t->k_in, out);
  TVP_LAUNCH_CHECK();
  return TVP_OK;
}

int w12_validate(const uint8_t* base, const uint32_t* esc_ptr, const uint16_t* esc_idx, int64_t n_out,
                 int64_t k_in, int64_t n_esc) {
  if (n_out < 0 || k_in < 0 || n_esc < 0) return TVP_ERR_ARG;
  if (k_in > 65536 || n_esc > 0xFFFFFFFFll) return TVP_ERR_FORMAT;
  if (!esc_ptr || (n_out > 0 && !base) || (n_esc > 0 && !esc_idx)) return TVP_ERR_ARG;
  if (esc_ptr[0] != 0 || (int64_t)esc_ptr[n_out] != n_esc) return TVP_ERR_FORMAT;
  for (int64_t r = 0; r < n_out; ++r) {
    if (base[r] < 1 || base[r] > 239) return TVP_ERR_FORMAT;
    const uint32_t a = esc_ptr[r], z = esc_ptr[r + 1];
    if (z < a || z > (uint64_t)n_esc) return TVP_ERR_FORMAT;
    for (uint32_t e = a; e < z; ++e) {
      if ((int64_t)esc_idx[e] >= k_in) return TVP_ERR_FORMAT;
      if (e > a && esc_idx[e] <= esc_idx[e - 1]) return TVP_ERR_FORMAT;
    }
  }
  return TVP_OK;
}

static int pack_size_fmt(int64_t n_out, int64_t k_in, int64_t n_esc, int32_t chan_map, int32_t map_a,
                         int32_t map_b, int32_t map_c, int32_t format, tvp_w12_packed* p) {
  if (!p || n_out < 1 || k_in < 0 || n_esc < 0) return TVP_ERR_ARG;
  if (k_in > 65536) return TVP_ERR_SHAPE;
  int64_t n_tiles;
  if (chan_map == TVP_CHAN_PLAIN) {
    n_tiles = ceil_div(n_out, 32);
  } else if (chan_map == TVP_CHAN_GATEUP) {
    if (map_a < 1 || (int64_t)map_a * 2 != n_out) return TVP_ERR_SHAPE;
    n_tiles = ceil_div(map_a, 16);
  } else if (chan_map == TVP_CHAN_QKV) {
    if (map_a < 1 || map_b < 1 || map_c < 32 || map_c % 32 || map_a % map_b) return TVP_ERR_SHAPE;
    if ((int64_t)(map_a + 2 * map_b) * map_c != n_out) return TVP_ERR_SHAPE;
    n_tiles = (int64_t)(map_a + map_b) * (map_c / 32) + ceil_div((int64_t)map_b * map_c, 32);
  } else {
    return TVP_ERR_ARG;
  }
  if (n_tiles > (1 << 26)) return TVP_ERR_SHAPE;
  const int64_t n_kb = ceil_div(k_in, kBlockK);
  const int64_t units = n_tiles * n_kb;
  p->n_out = n_out;
  p->k_in = k_in;
  p->n_esc = n_esc;
  p->n_tiles = (int32_t)n_tiles;
  p->n_kb = (int32_t)n_kb;
  p->chan_map = chan_map;
  p->map_a = map_a;
  p->map_b = map_b;
  p->map_c = map_c;
  p->format = format;
  size_t off = 0;
  p->off_rec = off;
  off = align_up(off + (size_t)units * block_bytes(format), 256);
  p->off_escoff = off;
  off = align_up(off + (size_t)(units + 1) * 4, 256);
  p->off_esc = off;
  off = align_up(off + (size_t)n_esc * 4, 256);
  p->off_b2 = off;
  off = align_up(off + (size_t)n_tiles * 32 * 4, 256);
  p->off_rowmap = off;
  off = align_up(off + (size_t)n_tiles * 32 * 4, 256);
  p->bytes = off;
  return TVP_OK;
}

int w12_pack_size(int64_t n_out, int64_t k_in, int64_t n_esc, int32_t chan_map, int32_t map_a,
                  int32_t map_b, int32_t map_c, tvp_w12_packed* p) {
  return pack_size_fmt(n_out, k_in, n_esc, chan_map, map_a, map_b, map_c, TVP_FMT_W12, p);
}

int w12_pack_hi8_size(int64_t n_out, int64_t k_in, int64_t n_esc, int32_t chan_map, int32_t map_a,
                      int32_t map_b, int32_t map_c, tvp_w12_packed* p) {
  return pack_size_fmt(n_out, k_in, n_esc, chan_map, map_a, map_b, map_c, TVP_FMT_HI8, p);
}

size_t w12_pack_workspace(int64_t n_out, int64_t k_in) {
  // per-unit escape counts for the worst map (GATEUP/QKV add at most a few tiles)
  const int64_t tiles = ceil_div(n_out, 16) + 64;
  return align_up((size_t)(tiles * ceil_div(k_in, kBlockK) + 1) * 4, 256);
}

static int pack_fmt(const tvp_w12* t, tvp_w12_packed* p, void* ws, size_t ws_bytes, hipStream_t stream,
                    int32_t format) {
  if (!t || !p || !p->blob) return TVP_ERR_ARG;
  if (p->format != format) return TVP_ERR_FORMAT;
  if (t->n_out != p->n_out || t->k_in != p->k_in || t->n_esc != p->n_esc) return TVP_ERR_SHAPE;
  const int64_t units = (int64_t)p->n_tiles * p->n_kb;
  if (!ws || ws_bytes < (size_t)(units + 1) * 4 || ws_bytes < w12_pack_workspace(t->n_out, t->k_in))
    return TVP_ERR_WORKSPACE;
  // The packer's binary searches and the GEMM's escape patch rely on the
  // side data being well formed: check it on the host first (this call
  // synchronises anyway), and launch nothing if it is not.
  {
    std::vector<uint8_t> hb((size_t)t->n_out);
    std::vector<uint32_t> hp((size_t)t->n_out + 1);
    std::vector<uint16_t> hi((size_t)std::max<int64_t>(t->n_esc, 1));
    if (!t->base || !t->esc_ptr || (t->n_esc > 0 && !t->esc_idx)) return TVP_ERR_ARG;
    TVP_CHECK_HIP(hipMemcpyAsync(hb.data(), t->base, hb.size(), hipMemcpyDeviceToHost, stream));
    TVP_CHECK_HIP(hipMemcpyAsync(hp.data(), t->esc_ptr, hp.size() * 4, hipMemcpyDeviceToHost, stream));
    if (t->n_esc > 0)
      TVP_CHECK_HIP(hipMemcpyAsync(hi.data(), t->esc_idx, (size_t)t->n_esc * 2, hipMemcpyDeviceToHost, stream));
    TVP_CHECK_HIP(hipStreamSynchronize(stream));
    const int vs = w12_validate(hb.data(), hp.data(), hi.data(), t->n_out, t->k_in, t->n_esc);
    if (vs != TVP_OK) return vs;
  }
  std::vector<int32_t> map;
  int st = build_rowmap(p, map);
  if (st != TVP_OK) return st;
  uint8_t* blob = (uint8_t*)p->blob;
  int32_t* rowmap = (int32_t*)(blob + p->off_rowmap);
  TVP_CHECK_HIP(hipMemcpyAsync(rowmap, map.data(), map.size() * 4, hipMemcpyHostToDevice, stream));
  TVP_CHECK_HIP(hipStreamSynchronize(stream));
  const int64_t n_pad = (int64_t)p->n_tiles * 32;
  pack_b2_kernel<<<dim3((unsigned)ceil_div(n_pad, 256)), dim3(256), 0, stream>>>(
      t->base, rowmap, n_pad, (uint32_t*)(blob + p->off_b2));
  TVP_LAUNCH_CHECK();
  uint32_t* counts = (uint32_t*)ws;
  uint32_t* escoff = (uint32_t*)(blob + p->off_escoff);
  if (units == 0) {
    TVP_CHECK_HIP(hipMemsetAsync(escoff, 0, 4, stream));
    return TVP_OK;
  }
  pack_count_kernel<<<dim3((unsigned)units), dim3(64), 0, stream>>>(t->esc_ptr, t->esc_idx, rowmap,
                                                                   p->n_kb, counts);
  TVP_LAUNCH_CHECK();
  scan_u32_kernel<<<1, 1024, 0, stream>>>(counts, units, escoff);
  TVP_LAUNCH_CHECK();
  if (format == TVP_FMT_HI8)
    pack_write_kernel<true><<<dim3((unsigned)units), dim3(64), 0, stream>>>(
        t->hi, t->lo, t->base, t->esc_ptr, t->esc_idx, t->esc_val, rowmap, t->k_in, p->n_kb, escoff,
        blob + p->off_rec, (uint32_t*)(blob + p->off_esc));
  else
    pack_write_kernel<false><<<dim3((unsigned)units), dim3(64), 0, stream>>>(
        t->hi, t->lo, t->base, t->esc_ptr, t->esc_idx, t->esc_val, rowmap, t->k_in, p->n_kb, escoff,
        blob + p->off_rec, (uint32_t*)(blob + p->off_esc));
  TVP_LAUNCH_CHECK();
  return TVP_OK;
}

int w12_pack(const tvp_w12* t, tvp_w12_packed* p, void* ws, size_t ws_bytes, hipStream_t stream) {
  return pack_fmt(t, p, ws, ws_bytes, stream, TVP_FMT_W12);
}

int w12_pack_hi8(const tvp_w12* t, tvp_w12_packed* p, void* ws, size_t ws_bytes, hipStream_t stream) {
  return pack_fmt(t, p, ws, ws_bytes, stream, TVP_FMT_HI8);
}

}  // extern "C"

namespace tvp {
// The packer for other entry points of the library (the INT8 head packs its
// int8 values as the 8-bit tile layout).
int pack_tiles(const tvp_w12* t, tvp_w12_packed* p, void* ws, size_t ws_bytes, hipStream_t stream,
               int32_t layout) {
  return pack_fmt(t, p, ws, ws_bytes, stream, layout);
}
}  // namespace tvp
