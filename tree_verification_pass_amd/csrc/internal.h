// Entry points shared between the library's translation units (not part of the ABI).
#pragma once

#include "common.h"

namespace tvp {

// Zero region of a GEMM: completion counters (kGemmMaxGroups entries), then
// argmax buckets (192 rows x 64 u64).  Zero on entry, left zero by every call.
constexpr size_t kGemmMaxGroups = 32768;
constexpr size_t kGemmKeyBytes = 192 * 64 * 8;
constexpr size_t kGemmZeroBytes = 256 * 1024;
static_assert(kGemmMaxGroups * 4 + kGemmKeyBytes <= kGemmZeroBytes, "zero region");

// W12 GEMM with caller-provided counters (`cnt`, groups entries), argmax
// buckets (`keys`) and scratch for partial sums.
int gemm_run(const uint16_t* x, int64_t m, int64_t ldx, const tvp_w12_packed* w,
             const tvp_gemm_epilogue* epi, uint32_t* cnt, unsigned long long* keys, void* scratch,
             size_t scratch_bytes, hipStream_t stream);
// Counter entries and scratch bytes gemm_run needs for m rows.
void gemm_requirements(int64_t m, const tvp_w12_packed* w, int* groups, size_t* scratch_bytes);

int launch_tree_prep(const int32_t* parents, const ReqInfo& ri, int32_t s_req, uint64_t* anc,
                     int32_t* pos, int32_t* slot, int32_t* status, hipStream_t stream);
int launch_tree_attention(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, int64_t s_stride,
                          const ReqInfo& ri, int32_t s_req, const uint64_t* anc, int hq, int hkv, int d,
                          int r_max, int max_keys, uint16_t* out, uint32_t* attn_cnt, void* scratch,
                          size_t scratch_bytes, hipStream_t stream);
size_t attention_scratch_bytes(int hkv, int G, int d, int r_max, int n_total, int max_keys);

}  // namespace tvp
