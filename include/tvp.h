/*
 * tvp.h -- C ABI of the tree-verification pass with W12 weights on MI355X (gfx950).
 *
 * Sources (cited by page and section; "SpecPilot summary" is the onedev.kr
 * page on SpecPilot, "SpecPilot review" the blog.secrett2633.cloud review):
 *   - W12, its per-channel escape list and the register-decode GEMM kept
 *     deterministic by stream-K: SpecPilot summary, section 무엇과 다른가;
 *   - one forward pass of the target over every draft-tree token, then the
 *     matched path and one bonus token: SpecPilot summary, sections 무엇인가
 *     and 무엇과 다른가; SpecPilot review, section 3;
 *   - "lossless" up to near-tie flips from reduction order (GEMM tiling, tree
 *     attention): SpecPilot summary, section 전제와 한계.
 *
 * Conventions for every entry point:
 *   - Pointers named in comments as "device" point to GPU memory; "host" to
 *     CPU memory.  All device buffers are owned by the caller; the library
 *     never allocates device memory (scratch comes in through `ws`, and no
 *     workspace needs any initial contents).
 *   - Work is enqueued on `stream` and is complete when the stream is.  Only
 *     w12_encode_count and w12_pack synchronise (documented there).
 *   - Shapes, nulls and capacities are validated on the host before anything
 *     is launched; a failure returns an error code and launches nothing.
 *     Launch failures return TVP_ERR_HIP.  No C++ exception crosses the ABI.
 *   - Handles are not thread-safe; calls that share a workspace must not
 *     overlap in time.
 *   - bf16 values are passed as their raw 16-bit patterns (uint16_t).
 */
#ifndef TVP_H
#define TVP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status codes */
enum {
  TVP_OK = 0,
  TVP_ERR_ARG = 1,       /* null pointer or invalid scalar argument */
  TVP_ERR_SHAPE = 2,     /* dimensions inconsistent or unsupported */
  TVP_ERR_TREE = 3,      /* malformed draft tree (also reported on device) */
  TVP_ERR_CAPACITY = 4,  /* more nodes / context than the plan was built for */
  TVP_ERR_FORMAT = 5,    /* W12 tensor fields out of range */
  TVP_ERR_WORKSPACE = 6, /* workspace missing or too small */
  TVP_ERR_HIP = 7        /* a HIP runtime call or kernel launch failed */
};

/* Static string naming a status code. */
const char* tvp_status_string(int status);

/* ------------------------------------------------------------- W12 tensors
 * Canonical W12 layout of a bf16 weight W[n_out][k_in] (one "channel" is one
 * output row).  SpecPilot summary, section 무엇과 다른가: a per-channel
 * 16-binade window [base, base+15] of normal exponents; each in-window weight
 * is the 12-bit record  sign<<11 | (exp-base)<<7 | mantissa ; zeros,
 * subnormals, infinities, NaNs and out-of-window values are escapes whose raw
 * bf16 bits are listed per channel (escaped slots hold record 0).
 *   hi      device uint8  [n_out][k_in]          record >> 4
 *   lo      device uint8  [n_out][(k_in+1)/2]    record & 15, even k in the low nibble
 *   base    device uint8  [n_out]                window base, 1..239
 *   esc_ptr device uint32 [n_out+1]              CSR offsets into esc_idx/esc_val
 *   esc_idx device uint16 [n_esc]                column, ascending per channel
 *   esc_val device uint16 [n_esc]                raw bf16 bits
 * The window is the one holding the most weights, the smallest base on ties.
 * k_in must be <= 65536 (uint16 escape columns). */
typedef struct tvp_w12 {
  int64_t n_out;
  int64_t k_in;
  int64_t n_esc;
  uint8_t* hi;
  uint8_t* lo;
  uint8_t* base;
  uint32_t* esc_ptr;
  uint16_t* esc_idx;
  uint16_t* esc_val;
} tvp_w12;

/* Phase 1 of the offline conversion (SpecPilot summary, section 무엇과 다른가:
 * models are converted to W12 ahead of serving).  From device bf16 weights
 * `w` [n_out][k_in] (row-major), writes device `base` [n_out] and `esc_ptr`
 * [n_out+1], then synchronises `stream` and returns the total number of
 * escapes in *h_n_esc (host).  The caller sizes esc_idx/esc_val from it. */
int w12_encode_count(const uint16_t* w, int64_t n_out, int64_t k_in, uint8_t* base,
                     uint32_t* esc_ptr, int64_t* h_n_esc, hipStream_t stream);

/* Phase 2: writes t->hi, t->lo, t->esc_idx, t->esc_val of the tensor whose
 * base/esc_ptr w12_encode_count produced (t->n_esc must equal its count). */
int w12_encode(const uint16_t* w, const tvp_w12* t, hipStream_t stream);

/* Exact decode back to bf16 bits, device `out` [n_out][k_in] (test hook). */
int w12_decode(const tvp_w12* t, uint16_t* out, hipStream_t stream);

/* Checks the side data of a canonical W12 tensor given in HOST memory:
 * base[n_out], esc_ptr[n_out+1], esc_idx[n_esc] (SpecPilot summary, section
 * 무엇과 다른가: a per-channel window and a per-channel escape list; the
 * window of normal exponents fixes 1 <= base <= 239).  TVP_ERR_FORMAT when a
 * base is outside 1..239, esc_ptr does not run from 0 up to n_esc without
 * decreasing, or a channel's escape columns are not strictly ascending and
 * below k_in (or k_in > 65536); TVP_ERR_ARG on a negative size or a null
 * array that is needed.  Pure host code: no HIP call, no allocation beyond
 * the stack.  w12_pack runs the same check before it launches anything. */
int w12_validate(const uint8_t* base, const uint32_t* esc_ptr, const uint16_t* esc_idx, int64_t n_out,
                 int64_t k_in, int64_t n_esc);

/* -------------------------------------------------- packed (GPU) W12 layout
 * SpecPilot summary, section 무엇과 다른가: the GEMM decodes W12 records in
 * registers behind the weight stream.  The records keep the canonical bits;
 * only their order in memory is chosen here, for that stream.
 * The GEMM streams W12 from a tiled copy of the same records: tiles of 32
 * channels x 64 k, each 3072 contiguous bytes laid out in the order the
 * 64 lanes of a wavefront load and decode them, plus per-tile-block escape
 * lists.  Tile blocks are stored k-block-major (block j of tile t at
 * (j * n_tiles + t) * 3072 bytes), so workgroups that stream the same k range
 * of neighbouring tiles at the same time read neighbouring memory.
 * It decodes to exactly the same bf16 values as the canonical layout
 * (checked by w12_gemm parity).  `chan_map` chooses which canonical row lands
 * in each packed channel, so fused epilogues find their operands in one tile:
 *   TVP_CHAN_PLAIN   packed channel p = row p
 *   TVP_CHAN_GATEUP  rows [gate F | up F]: tile t = gate rows 16t..16t+15 then
 *                    up rows 16t..16t+15 (map_a = F)
 *   TVP_CHAN_QKV     rows [q heads | k heads | v heads] of head size d:
 *                    q/k tiles pair dims i and i+d/2 (16 each) for RoPE, v
 *                    tiles are plain (map_a = n_heads, map_b = n_kv_heads,
 *                    map_c = d; d % 32 == 0)                                  */
enum { TVP_CHAN_PLAIN = 0, TVP_CHAN_GATEUP = 1, TVP_CHAN_QKV = 2 };

/* Record format of a packed tensor.  TVP_FMT_W12: the full 12-bit records
 * (3072-byte tile blocks).  TVP_FMT_HI8: only the 8-bit leading view of each
 * record, record >> 4 (2048-byte tile blocks), for the Q pass of two-level
 * verification (SpecPilot summary, section 무엇과 다른가: the Q pass runs on
 * the 8-bit view of the front of the W12 records): an in-window weight is
 * read with its low four mantissa bits cleared; escapes stay exact.         */
enum { TVP_FMT_W12 = 0, TVP_FMT_HI8 = 1 };

typedef struct tvp_w12_packed {
  int64_t n_out, k_in, n_esc;
  int32_t n_tiles, n_kb; /* ceil over 32 packed channels, ceil(k_in/64) */
  int32_t chan_map, map_a, map_b, map_c;
  int32_t format;        /* TVP_FMT_W12 or TVP_FMT_HI8 */
  void* blob;            /* device, `bytes` long, caller-owned, 256-B aligned */
  size_t bytes;
  size_t off_rec, off_escoff, off_esc, off_b2, off_rowmap; /* offsets in blob */
} tvp_w12_packed;

/* Fills every field of *p except `blob` for the given shape and map
 * (format TVP_FMT_W12). */
int w12_pack_size(int64_t n_out, int64_t k_in, int64_t n_esc, int32_t chan_map, int32_t map_a,
                  int32_t map_b, int32_t map_c, tvp_w12_packed* p);

/* Builds the packed copy of canonical tensor `t` into p->blob (p from
 * w12_pack_size with p->blob set), part of the offline conversion of the
 * model (SpecPilot summary, section 무엇과 다른가).  Device scratch `ws` of
 * w12_pack_workspace() bytes.  Synchronises `stream`: the tensor's side data
 * is first checked on the host as w12_validate does (TVP_ERR_FORMAT, nothing
 * launched), then the channel map is uploaded. */
size_t w12_pack_workspace(int64_t n_out, int64_t k_in);
int w12_pack(const tvp_w12* t, tvp_w12_packed* p, void* ws, size_t ws_bytes, hipStream_t stream);

/* The same two calls for the 8-bit leading view (format TVP_FMT_HI8): the
 * tiles hold record >> 4 of every weight in the same lane order, the escape
 * lists are the same.  The GEMM reads such a tensor at up to 32 rows
 * (TVP_ERR_SHAPE above); w12_pack_workspace sizes the scratch of both. */
int w12_pack_hi8_size(int64_t n_out, int64_t k_in, int64_t n_esc, int32_t chan_map, int32_t map_a,
                      int32_t map_b, int32_t map_c, tvp_w12_packed* p);
int w12_pack_hi8(const tvp_w12* t, tvp_w12_packed* p, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ W12 GEMM
 * Y[m][n_out] = X[m][k_in] . W^T with bf16 inputs and fp32 accumulation, the
 * weights decoded from W12 in registers (SpecPilot summary, section
 * 무엇과 다른가).  Split-K partial sums are reduced in a fixed order, so the
 * result is bitwise identical from run to run (the page's deterministic
 * stream-K requirement).  1 <= m <= 192.
 *   x      device bf16 [m][ldx], 16-byte aligned, ldx >= k_in, ldx % 8 == 0
 *   y      device, [m][ldy] fp32 if y_fp32 else bf16 (ldy >= n_out); rows
 *          follow the canonical channel order whatever p->chan_map is
 *   ws     device scratch of w12_gemm_workspace() bytes (any contents; a
 *          call may overwrite all of it).  Calls that share a workspace must
 *          not overlap in time.                                               */
size_t w12_gemm_workspace(int64_t m, const tvp_w12_packed* w);
int w12_gemm(const uint16_t* x, int64_t m, int64_t ldx, const tvp_w12_packed* w, void* y,
             int64_t ldy, int y_fp32, void* ws, size_t ws_bytes, hipStream_t stream);

/* Same GEMM with a fused epilogue (used by verify_step; exposed for tests). */
enum {
  TVP_EPI_F32 = 0,     /* y fp32 */
  TVP_EPI_BF16 = 1,    /* y bf16 */
  TVP_EPI_RESID = 2,   /* y bf16 = bf16(resid + acc); resid may alias y */
  TVP_EPI_SWIGLU = 3,  /* TVP_CHAN_GATEUP: y bf16 [m][F] = bf16(silu(gate) * up) */
  TVP_EPI_QKV = 4,     /* TVP_CHAN_QKV: RoPE on q and k at positions pos[m];
                          q -> y bf16 [m][n_heads][d]; k, v -> caches at slot[m] */
  TVP_EPI_ARGMAX = 5   /* argmax (int32 [m], ties -> smallest id) + optional fp32 logits */
};

typedef struct tvp_gemm_epilogue {
  int32_t mode;
  void* y;                 /* F32/BF16/RESID/SWIGLU/QKV output (see modes) */
  int64_t ldy;
  const uint16_t* resid;   /* RESID: bf16 [m][ldr] */
  int64_t ldr;
  const int32_t* pos;      /* QKV: device int32 [m] RoPE positions */
  const int32_t* slot;     /* QKV: device int32 [m] cache slots for k and v */
  uint16_t* k_cache;       /* QKV: device bf16 [n_kv_heads][s_stride][d] */
  uint16_t* v_cache;
  int64_t s_stride;
  double rope_theta;
  int32_t* argmax;         /* ARGMAX: device int32 [m] */
  float* logits;           /* ARGMAX: optional device fp32 [m][ldl] (NULL = none) */
  int64_t ldl;
  int32_t x_packed;        /* x is in the packed activation layout (ldx unused) */
  int32_t y_packed;        /* SWIGLU: y is written in the packed layout (ldy unused) */
  uint32_t* counters;      /* optional device uint32 [TVP_GEMM_COUNTERS], all zero: arrival counters
                              of the channel groups whose K range is cut into slices (the slice that
                              arrives last applies the epilogue); the call leaves them at zero, so one
                              array serves any number of calls in stream order.  NULL: the counters
                              live in ws and one small launch clears them before the GEMM. */
} tvp_gemm_epilogue;
#define TVP_GEMM_COUNTERS 256

/* x_packed and y_packed need m <= 32 and every k_in <= 32256 (the
 * single-pass path); otherwise TVP_ERR_ARG. */
int w12_gemm_ex(const uint16_t* x, int64_t m, int64_t ldx, const tvp_w12_packed* w,
                const tvp_gemm_epilogue* epi, void* ws, size_t ws_bytes, hipStream_t stream);

/* The same GEMM for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no workspace argument; the scratch is a library-owned device array of
 * TVP_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends.  The call
 * allocates nothing.  Shapes whose w12_gemm_workspace() exceeds that size
 * return TVP_ERR_WORKSPACE (e.g. the wide path at many rows over large
 * weights); every 27B-like projection and LM head at up to 32 rows fits.
 * `stream` must belong to the current device (TVP_ERR_ARG otherwise).  All
 * calls on one GPU share the array, so calls that overlap in time on one
 * GPU (other streams, other threads) race; nothing in it needs to start at
 * zero.  Arguments and results otherwise as w12_gemm_ex. */
#define TVP_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int w12_gemm_ex_noalloc(const uint16_t* x, int64_t m, int64_t ldx, const tvp_w12_packed* w,
                        const tvp_gemm_epilogue* epi, hipStream_t stream);

/* Packed activation layout, the GEMM's input format for up to 32 rows (and
 * what verify_step produces internally; the pages leave the activation
 * layout open, so it is chosen for the GEMM's MFMA operand loads): bf16 element (row, k) lives at
 * (k/8)*256 + row*8 + k%8, so a wavefront's MFMA A-fragment of 32 rows x 8
 * columns is 512 contiguous bytes.  k is padded to a multiple of 64:
 * w12_packed_x_elems(k_in) elements.  w12_pack_x converts row-major
 * x (device bf16 [m][ldx], ldx >= k_in) into xp (device, 16-byte aligned,
 * caller-owned), zero-filling rows m..31 and the padding columns.
 * 1 <= m <= 32, k_in >= 0; TVP_ERR_SHAPE / TVP_ERR_ARG otherwise. */
int64_t w12_packed_x_elems(int64_t k_in);
int w12_pack_x(const uint16_t* x, int64_t m, int64_t ldx, int64_t k_in, uint16_t* xp, hipStream_t stream);

/* Projection + residual add + RMSNorm, the stage that follows the attention
 * and the FFN in every layer of verify_step, in the same launch
 * configuration (K split over workgroups, the slices' fp32 sums added in
 * slice order by the fused residual + RMSNorm kernel).  The residual add
 * follows from the decoder layer the pages' targets use; RMSNorm is the
 * norm of the model configurations (eps given here).
 *   xp     device bf16, packed activation layout of m rows x w->k_in
 *   w      TVP_CHAN_PLAIN packed weight, w->k_in <= 32256
 *   h      device bf16 [m][ldh] residual stream, updated in place:
 *          h = bf16(h + xp . W^T)  (fp32 sum, one rounding)
 *   gain   device bf16 [w->n_out]
 *   yp     device bf16, packed layout of m rows x w->n_out:
 *          bf16(h * (mean(h^2) + eps)^-1/2 * gain), fp32 inside
 *   ws     device scratch of w12_gemm_resid_norm_workspace() bytes
 * 1 <= m <= 32 (TVP_ERR_SHAPE otherwise); 16-byte aligned pointers.       */
size_t w12_gemm_resid_norm_workspace(int64_t m, const tvp_w12_packed* w);
int w12_gemm_resid_norm(const uint16_t* xp, int64_t m, const tvp_w12_packed* w, uint16_t* h, int64_t ldh,
                        const uint16_t* gain, float eps, uint16_t* yp, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* ------------------------------------------------ INT8 certified LM head
 * SpecPilot summary, section 무엇과 다른가: the LM head can filter candidate
 * tokens with INT8 weights and a Cauchy-Schwarz error bound while keeping the
 * exact argmax.  Per vocabulary row v: the 8 largest magnitudes (ties to the
 * smaller column) are escapes, carried as bf16(w / s_v); the rest are
 * q = clip(rint(fp32(w) / s_v), -127, 127) with s_v = fp32(t_v / 127), t_v the
 * largest remaining magnitude (1 when it is 0); r_v = ||W_v - s_v B_v||_2 (B_v:
 * the int8 values with the escapes in place) rounded up to fp32, and r_eff_v
 * = r_v plus a bound of the fp32 accumulation error of the approximate logit.
 * The argmax computes a_v = f . s_v B_v (bf16 MFMA on the int8 values, fp32
 * accumulation), tau = max_v (a_v - ||f|| r_eff_v), and exact logits -- from
 * the canonical W12 rows of the same weights -- only for the v with
 * a_v + ||f|| r_eff_v >= tau, a set that always holds the exact argmax.
 * Keeping the largest magnitudes out of the scale follows W12's escapes: on
 * weights with rare large outliers, a scale set by the outliers would leave
 * a large share of the vocabulary as candidates.                            */
typedef struct tvp_lmhead_i8 {
  int64_t vocab, k_in;  /* k_in <= 16384 */
  int8_t* q;            /* device [vocab][k_in], 0 at the escaped columns */
  float* scale;         /* device [vocab] */
  uint16_t* esc_col;    /* device [vocab][8], ascending */
  uint16_t* esc_val;    /* device [vocab][8], bf16 of w / scale */
  float* r;             /* device [vocab] */
  float* r_eff;         /* device [vocab] */
  tvp_w12_packed tiles; /* the int8 values in the GEMM's tiled layout (blob caller-owned) */
} tvp_lmhead_i8;

/* Sizes the tiles (every field of *p but `blob`). */
int lmhead_i8_tiles_size(int64_t vocab, int64_t k_in, tvp_w12_packed* p);
/* Encodes device bf16 `w` [vocab][k_in] into every array of *h and packs the
 * tiles (h->tiles from lmhead_i8_tiles_size, its blob set).  Device scratch
 * of lmhead_i8_encode_workspace() bytes.  Synchronises `stream` (offline
 * conversion, like w12_pack). */
size_t lmhead_i8_encode_workspace(int64_t vocab, int64_t k_in);
int lmhead_i8_encode(const uint16_t* w, tvp_lmhead_i8* h, void* ws, size_t ws_bytes, hipStream_t stream);
/* Greedy token of every row of the packed activations xp (m <= 32 rows of
 * k_in): argmax (int32 [m], ties to the smallest id) and the number of
 * certified candidates per row (int32 [m]); `approx` (optional fp32
 * [m][vocab]) receives the approximate logits.  `exact` is the canonical W12
 * tensor of the same weights.  Scratch: lmhead_i8_argmax_workspace() bytes. */
size_t lmhead_i8_argmax_workspace(int64_t m, const tvp_lmhead_i8* h);
int lmhead_i8_argmax(const uint16_t* xp, int64_t m, const tvp_lmhead_i8* h, const tvp_w12* exact, int32_t* argmax,
                     int32_t* n_cand, float* approx, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------- tree attention
 * Attention of n draft-tree nodes over a committed context and their own
 * ancestors (SpecPilot summary, section 전제와 한계 names tree attention as
 * one of the reduction orders that may flip near-ties).  Node i attends to
 * cache slots [0, ctx_len) and to tree slots ctx_len + j for every ancestor
 * j of i and i itself, where the tree's own keys/values are already in the
 * cache at slots ctx_len + j.  Scores q.k/sqrt(d), softmax in fp32, GQA
 * q-head h -> kv-head h / (hq/hkv).  Split over the keys with a fixed-order
 * merge: deterministic.
 *   q        device bf16 [n][hq][d] (already rotated)
 *   k_cache  device bf16 [hkv][s_stride][d] (v_cache likewise)
 *   parents  device int32 [n]: parents[0] = -1, 0 <= parents[i] < i
 *   out      device bf16 [n][hq][d]
 *   status   device int32 [1]: TVP_OK or TVP_ERR_TREE (then out is zero)
 * n <= 64, d in {64, 128}, hq % hkv == 0, n * hq / hkv <= 256.
 * ws: tree_attention_workspace() bytes of device scratch (any contents).     */
size_t tree_attention_workspace(int32_t n, int32_t hq, int32_t d, int32_t max_keys);
int tree_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                   int64_t s_stride, int32_t ctx_len, const int32_t* parents, int32_t n, int32_t hq,
                   int32_t hkv, int32_t d, uint16_t* out, int32_t* status, void* ws,
                   size_t ws_bytes, hipStream_t stream);

/* ----------------------------------------------------------- acceptance
 * Greedy acceptance (SpecPilot summary, section 무엇과 다른가: the matched
 * path plus a bonus token).  acc[0] = 1; acc[i] = acc[parents[i]] and
 * tokens[i] == argmax[parents[i]].  The deepest accepted node (smallest index
 * on ties) ends the path; bonus = argmax at that node.  One workgroup.
 *   argmax, tokens, parents  device int32 [n], n <= 1024
 *   path        device int32 [n]: path[0..n_accepted] = root .. deepest node
 *   n_accepted, bonus, status  device int32 [1]
 * A malformed tree sets *status = TVP_ERR_TREE, n_accepted = 0, path[0] = 0,
 * bonus = argmax[0].                                                          */
int accept_path(const int32_t* argmax, const int32_t* tokens, const int32_t* parents, int32_t n,
                int32_t* path, int32_t* n_accepted, int32_t* bonus, int32_t* status,
                hipStream_t stream);

/* ------------------------------------------------------ the verify pass */
typedef struct tvp_layer {
  tvp_w12_packed wqkv;   /* TVP_CHAN_QKV, [(hq+2hkv)d][hidden] */
  tvp_w12_packed wo;     /* TVP_CHAN_PLAIN, [hidden][hq d] */
  tvp_w12_packed wgu;    /* TVP_CHAN_GATEUP, [2 ffn][hidden] */
  tvp_w12_packed wdown;  /* TVP_CHAN_PLAIN, [hidden][ffn] */
  const uint16_t* attn_norm; /* device bf16 [hidden] */
  const uint16_t* ffn_norm;  /* device bf16 [hidden] */
  uint16_t* k_cache;     /* device bf16 [hkv][s_max][d] */
  uint16_t* v_cache;     /* device bf16 [hkv][s_max][d] */
} tvp_layer;

typedef struct tvp_model_desc {
  int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab;
  float rope_theta, norm_eps;
  int32_t s_max;               /* KV slots per layer and head */
  const uint16_t* embed;       /* device bf16 [vocab][hidden] */
  const uint16_t* final_norm;  /* device bf16 [hidden] */
  tvp_w12_packed lm_head;      /* TVP_CHAN_PLAIN, [vocab][hidden] */
  const tvp_layer* layers;     /* host array [n_layers]; copied by tvp_plan_create */
} tvp_model_desc;

typedef struct tvp_plan tvp_plan;

/* Validates the description and builds host state for trees of up to
 * max_nodes nodes in total (all requests of a batch together, <= 192): the
 * target model whose forward pass verifies every draft-tree token at once
 * (SpecPilot summary, section 무엇인가), its weights already converted to
 * packed W12 (section 무엇과 다른가), and one KV cache per layer.  Device
 * pointers in `desc` are stored, not dereferenced; the plan owns host memory
 * only.  TVP_ERR_SHAPE / TVP_ERR_FORMAT / TVP_ERR_ARG / TVP_ERR_CAPACITY on
 * an inconsistent description. */
int tvp_plan_create(const tvp_model_desc* desc, int32_t max_nodes, tvp_plan** plan);
void tvp_plan_destroy(tvp_plan* plan);

/* Device scratch needed by verify_step / verify_step_batched on this plan
 * (any contents; every call overwrites what it uses).  Calls sharing a
 * workspace must not overlap in time. */
size_t verify_step_workspace(const tvp_plan* plan);

typedef struct tvp_verify_out {
  int32_t* argmax;     /* device int32 [n] */
  int32_t* path;       /* device int32 [n] */
  int32_t* n_accepted; /* device int32 [1] */
  int32_t* bonus;      /* device int32 [1] */
  int32_t* status;     /* device int32 [1] */
  float* logits;       /* optional device fp32 [n][vocab] (NULL = not written) */
} tvp_verify_out;

/* One verification pass of draft tree (tokens, parents) after ctx_len
 * committed tokens -- SpecPilot summary, section 무엇인가 (every draft token
 * goes through the target in one forward pass) and section 무엇과 다른가
 * (the pass returns the matched path plus a bonus token): every node's next-token logits in one forward pass
 * (node i at position ctx_len + depth(i), its K/V written to cache slot
 * ctx_len + i), greedy acceptance, and -- if `commit` -- the accepted nodes'
 * K/V moved to slots ctx_len .. ctx_len + n_accepted, so the next committed
 * length is ctx_len + n_accepted + 1 and the bonus token is the next root.
 *   tokens, parents  device int32 [n]; tokens[0] is the root token (the last
 *                    committed-but-unprocessed token, e.g. the previous bonus)
 * Requires ctx_len + n <= s_max and n <= min(max_nodes, 64)
 * (TVP_ERR_CAPACITY otherwise), (n_heads / n_kv_heads) * n <= 256 (the
 * attention's rows per kv head; TVP_ERR_SHAPE otherwise); depth <= 63.     */
int verify_step(tvp_plan* plan, int32_t ctx_len, const int32_t* tokens, const int32_t* parents,
                int32_t n, int32_t commit, const tvp_verify_out* out, void* ws, size_t ws_bytes,
                hipStream_t stream);

/* Batched pass (SpecPilot summary, section 무엇과 다른가: requests share one
 * node budget): n_req requests, request r owning nodes node_ptr[r] ..
 * node_ptr[r+1]-1 of the concatenated tokens/parents (parents are
 * request-local), its own context length ctx_len[r] and its own KV cache
 * region: slots [r*s_req, (r+1)*s_req) of every layer's cache.  Every GEMM
 * runs once over all Σ n_r rows; attention, acceptance and commit run per
 * request.  Outputs are per request: path [node_ptr[r] ..] (request-local
 * node indices), n_accepted/bonus/status [r]; argmax/logits per global node.
 *   ctx_len, node_ptr  host int32 arrays ([n_req], [n_req+1])
 * Per request the limits of verify_step hold, with ctx_len[r] + n_r <= s_req;
 * n_req * s_req <= s_max and Σ n_r <= max_nodes.                           */
int verify_step_batched(tvp_plan* plan, int32_t n_req, const int32_t* ctx_len,
                        const int32_t* node_ptr, int32_t s_req, const int32_t* tokens,
                        const int32_t* parents, int32_t commit, const tvp_verify_out* out,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------- Gated DeltaNet layers (hybrid targets)
 * SpecPilot summary, section 무엇과 다른가: for a target whose recurrent
 * layers are Gated DeltaNet, verification takes each node's recurrent state
 * along its own root path (recomputed, not stored per node); a WY-form
 * verify solves all paths at once with matrix products, the fp32 state split
 * into three bf16 pieces that hold its 24-bit significand exactly; after
 * acceptance the accepted path is replayed into every recurrent layer.  The
 * recurrence (gated delta rule, Gated DeltaNet, Yang, Kautz and Hatamizadeh,
 * ICLR 2025), per value head with state S [dv][dk]:
 *   S <- exp(g) S + beta (v - exp(g) S k) k^T,   o = S q
 * for every new token in root-first order; value head h reads q and k of key
 * head h / (hv / hk).  q and k arrive as the recurrence consumes them (after
 * the layer's projections, convolution and normalisation).
 *
 * gdn_tree_verify (WY form) and gdn_path_verify (each leaf's root path
 * replayed from the committed state) compute the same outputs:
 *   q, k     device bf16 [n][hk][dk]       v  device bf16 [n][hv][dv]
 *   g, beta  device fp32 [n][hv] (log decay <= 0, write strength)
 *   state    device fp32 [hv][dv][dk], the committed state (read only)
 *   parents  device int32 [n], parents[0] = -1, 0 <= parents[i] < i
 *   out      device bf16 [n][hv][dv] (caller-owned; every element written)
 *   status   device int32 [1]: TVP_OK, or TVP_ERR_TREE for a malformed tree
 *            (the outputs are then unspecified)
 * Limits: 1 <= n <= 32, dk = dv = 128, hv a multiple of hk; q, k, v and
 * state 16-byte aligned.  TVP_ERR_ARG / TVP_ERR_SHAPE before any launch.  No
 * workspace.  Deterministic: the same inputs give the same bits.           */
int gdn_tree_verify(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g, const float* beta,
                    const float* state, const int32_t* parents, int32_t n, int32_t hk, int32_t hv, int32_t dk,
                    int32_t dv, uint16_t* out, int32_t* status, hipStream_t stream);
int gdn_path_verify(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g, const float* beta,
                    const float* state, const int32_t* parents, int32_t n, int32_t hk, int32_t hv, int32_t dk,
                    int32_t dv, uint16_t* out, int32_t* status, hipStream_t stream);

/* Commit of the accepted path into n_layers recurrent layers at once:
 * state [n_layers][hv][dv][dk] (device fp32, updated in place) gets the
 * updates of nodes path[0 .. *n_accepted] in that order, with each layer's
 * k [n_layers][n][hk][dk], v [n_layers][n][hv][dv] (bf16) and
 * g, beta [n_layers][n][hv] (fp32).  path, n_accepted and status are device
 * int32 as accept_path writes them; nothing is changed unless *status is
 * TVP_OK, 0 <= *n_accepted < n and every path entry is in [0, n).  Limits as
 * above (n_layers <= 1024; state, k and v 16-byte aligned).               */
int gdn_commit(float* state, const uint16_t* k, const uint16_t* v, const float* g, const float* beta,
               int32_t n_layers, int32_t n, int32_t hk, int32_t hv, int32_t dk, int32_t dv, const int32_t* path,
               const int32_t* n_accepted, const int32_t* status, hipStream_t stream);

/* ------------------------------------------------------- measurement
 * Streaming-read probe: the HBM read rate a plain sequential stream reaches
 * on this GPU, the practical ceiling the weight stream of the pass (SpecPilot
 * summary, section 무엇인가: most of a step is reading the target's weights)
 * is compared against, next to the nominal bandwidth.  Reads the first bytes/16*16 bytes of src once, as a
 * plain sequential stream, and writes 4096 words to sink.  Nothing else is
 * touched; time it with events on `stream`.
 *   src   device, 16-byte aligned, >= 16 bytes (caller-owned)
 *   sink  device uint32 [4096] (caller-owned; contents meaningless)
 * TVP_ERR_ARG on a null or misaligned pointer.                             */
int tvp_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TVP_H */
