// Entry points shared between the library's translation units (not part of the ABI).
#pragma once

#include "common.h"

namespace tvp {

// Largest number of channel groups one GEMM launch takes (grid sizes and the
// argmax key slots stay well inside 32-bit indexing).
constexpr size_t kGemmMaxGroups = 32768;

// W12 GEMM with caller-provided scratch (which also holds the argmax key
// slots).  Activations come row-major in `x` or, for
// m <= 32, already in the packed layout in `xp` (then `x` is unused).
// `y_packed`: the SwiGLU epilogue writes its output packed (m <= 32).
// `ksplit` > 1 (skinny path, epilogue kEpiPartial only) also splits K over
// workgroups.
// rope_cs (QKV epilogue, optional): per GEMM row r and rotated dim i < d/2,
// (cos, sin) of pos[r] * theta^(-2i/d) at rope_cs[2 * (r * d/2 + i)] -- the
// values the epilogue would otherwise compute itself, formed once per pass.
// Record format of packed int8 values (the INT8 LM head): same tiles as
// TVP_FMT_HI8, each byte a signed int8; only the kEpiI8Approx epilogue.
constexpr int kFmtI8 = 2;
struct I8EpiArgs {
  const float* scale;  // [n_out] per-channel scale
  const float* r;      // [n_out] bound radius
  const float* fnorm;  // [m] ||f_row||_2
};
// epi->counters (optional): TVP_GEMM_COUNTERS zero arrival counters for the
// K slices of the remaining groups; without them they live in the scratch and
// a small launch clears them first.
int gemm_run(const uint16_t* x, const uint16_t* xp, int64_t m, int64_t ldx, const tvp_w12_packed* w,
             const tvp_gemm_epilogue* epi, int y_packed, void* scratch, size_t scratch_bytes,
             hipStream_t stream, int ksplit = 1, const float* rope_cs = nullptr, const I8EpiArgs* i8 = nullptr);
// (cos, sin) table of the QKV epilogue for rows 0..n-1 at positions pos[].
int launch_rope_table(const int32_t* pos, int n, int d, double theta, float* rope_cs, hipStream_t stream);

// Internal epilogue (not part of the ABI): each K slice's fp32 partial result
// goes to y = P[slice][m][ldy] (canonical columns); the consumer sums the
// slices in slice order.  Needs the plain channel map and the skinny path.
constexpr int kEpiPartial = 16;
// Internal epilogue of the INT8 head: approximate logits (epi->logits, ldl)
// and per-workgroup key slots of max(a - ||f|| r) per row.
constexpr int kEpiI8Approx = 17;

// Packed activation layout for up to 32 rows: 16-byte groups of 8 columns,
// [k / 8][row (32)][k % 8].  One MFMA A-fragment load of a wavefront is then
// 1 KB contiguous instead of 32 rows of 16 bytes.  Columns are padded to a
// multiple of 64; rows >= m and padding columns are never used.
__host__ __device__ inline int64_t xpack_index(int row, int64_t k) { return (k >> 3) * 256 + row * 8 + (k & 7); }
inline int64_t xpack_elems(int64_t k_in) { return ((k_in + 63) / 64) * 2048; }

// Key slots (one per workgroup) of an argmax-like epilogue and their offset
// in gemm_run's scratch, for m rows.
int gemm_key_slots(int64_t m, const tvp_w12_packed* w);
size_t gemm_keys_offset(int64_t m, const tvp_w12_packed* w);
// Whether gemm_run takes the skinny path (and so accepts packed input) for m rows.
bool gemm_is_skinny(int64_t m, const tvp_w12_packed* w);
// Number of K slices gemm_run uses for `ksplit` (clamped so none is empty).
int gemm_ksplits(int64_t m, const tvp_w12_packed* w, int ksplit);
// Channel groups and scratch bytes gemm_run needs for m rows (and `ksplit`).
void gemm_requirements(int64_t m, const tvp_w12_packed* w, int* groups, size_t* scratch_bytes, int ksplit = 1);

// The W12 packer with the tile layout of `layout` (TVP_FMT_W12 or
// TVP_FMT_HI8): p->format must equal it.
int pack_tiles(const tvp_w12* t, tvp_w12_packed* p, void* ws, size_t ws_bytes, hipStream_t stream,
               int32_t layout);

// Arrival counters (see arrive_last) of the in-launch hand-overs: they must
// be zero when a launch starts, and every launch leaves them at zero.  Tree
// preparation sets the ncnt counters at cnt to zero first.
int launch_tree_prep(const int32_t* parents, const ReqInfo& ri, int32_t s_req, uint64_t* anc,
                     int32_t* pos, int32_t* slot, int32_t* status, uint32_t* cnt, int ncnt,
                     hipStream_t stream);
// cnt: attention_counters(n_req, hkv) arrival counters, zero.
int launch_tree_attention(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, int64_t s_stride,
                          const ReqInfo& ri, int32_t s_req, const uint64_t* anc, int hq, int hkv, int d,
                          int r_max, int max_keys, uint16_t* out, int out_packed, void* scratch,
                          size_t scratch_bytes, uint32_t* cnt, hipStream_t stream);
size_t attention_scratch_bytes(int hkv, int G, int d, int r_max, int n_total, int max_keys);
// 32-row blocks per (request, kv head) at most (256 rows), and the attention's
// arrival counters for n_req requests: one per (request, kv head, row block).
constexpr int kAttnRowBlocks = 8;
inline int attention_counters(int n_req, int hkv) { return n_req * hkv * kAttnRowBlocks; }
// Arrival counters a skinny GEMM launch with remaining-group K slices uses
// at most (one per remaining group: fewer groups than compute units).
constexpr int kGemmRemCounters = TVP_GEMM_COUNTERS;

}  // namespace tvp
