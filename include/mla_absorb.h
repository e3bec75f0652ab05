/*
 * mla_absorb.h -- C ABI of the MI355X (gfx950) library for DeepSeek-V2
 * Multi-head Latent Attention decode with matrix absorption.
 *
 * What is computed (sources cited by page title and section):
 *   Every request caches, per token and layer, only the joint K/V latent
 *   c^KV (width d_c) and the shared, already-rotated RoPE key k^R (width
 *   d_h^R), stored as one row [c^KV | k^R]  (DeepSeek-V3 technical report
 *   read-through, 2kiu.com/news/6340724, sections 2.2 and 2.4; DeepSeek-V2
 *   read-through, 2kiu.com/news/6085339, section 5.1).
 *   W^UK is absorbed into the query, q_lat,i = W^UK_i^T q^C_i, so scores are
 *   taken directly against the cached row; the softmax-weighted sum stays in
 *   latent space and W^UV is applied last  (V2 read-through, section 2.3;
 *   zeeklog "Transformer 15: DeepSeek-V2 architecture", equations 9-11 and
 *   the absorption paragraph after them).
 *   A decode step of one layer is three calls:
 *     mla_absorb_q    q_cat[b,i] = [ W^UK_i^T q^C[b,i] | q^R[b,i] ]
 *     mla_decode_attn o_lat[b,i] = sum_j softmax_j(scale * q_cat[b,i] . row_j) c_j
 *     mla_out_uv      o[b,i,h]   = sum_c o_lat[b,i,c] W^UV[i,c,h]
 *
 * Conventions shared by every call:
 *   - Every pointer to tensor data is a DEVICE pointer (HIP memory on the
 *     current device), unless the argument says "host".  The caller owns and
 *     frees all memory, including the workspace; the library never allocates
 *     device memory and never synchronises the stream.
 *   - Tensors are dense, row-major, innermost dimension contiguous.  Float
 *     tensors use the storage type dims->dtype (fp32 or bf16); lse, split
 *     partials and all accumulation are fp32.  Integer tensors are int32.
 *   - Device pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     All work is enqueued asynchronously on it; pointers must stay valid
 *     until that work completes.
 *   - Arguments are checked on the host before anything is enqueued; on
 *     failure a non-zero status is returned and nothing is launched.  A
 *     launch the runtime rejects returns MLA_ERR_LAUNCH.  Device-side data
 *     (seq_lens, page_table) is trusted: values outside the documented
 *     ranges are undefined behaviour.
 *   - Calls on different streams may run concurrently; the library keeps no
 *     mutable global state apart from a per-device property cache.
 */
#ifndef MLA_ABSORB_H
#define MLA_ABSORB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,      /* a required pointer is NULL                        */
  MLA_ERR_DIMS = 2,      /* a size is out of range or sizes are inconsistent  */
  MLA_ERR_DTYPE = 3,     /* unsupported storage type                          */
  MLA_ERR_WORKSPACE = 4, /* workspace NULL or smaller than the plan needs     */
  MLA_ERR_ALIGN = 5,     /* a device pointer is not 16-byte aligned           */
  MLA_ERR_LAUNCH = 6,    /* the HIP runtime rejected a kernel launch          */
  MLA_ERR_DEVICE = 7     /* no current HIP device, or it is not gfx950        */
} mla_status_t;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype_t;

/* How the cache stores its rows (mla_cache_t.row_format).  MLA_ROWS_NATIVE:
 * elements of dims->dtype.  MLA_ROWS_FP8: the low-bit cache of deployment
 * (ai-library "DeepSeek-V2" notes, "Training and Inference Efficiency" /
 * "Inference cost": the KV cache quantised to about 6 bits per element; V3
 * read-through section 4.4: scales computed online from the data): each row
 * is d_latent + d_rope OCP E4M3 bytes (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits, largest finite value 448) with one fp32 scale per row, the
 * element value being code * scale (see mla_quantize_rows). */
typedef enum { MLA_ROWS_NATIVE = 0, MLA_ROWS_FP8 = 1 } mla_row_format_t;

/* Model dimensions of one MLA layer (DeepSeek-V2: 128, 128, 64, 512; zeeklog
 * notes, the remark under the cache table: d_c = 4 d_h, d_h^R = d_h / 2). */
typedef struct {
  int32_t n_heads;  /* n_h, 1..1024                                        */
  int32_t d_head;   /* d_h, content width per head, 1..1024                */
  int32_t d_rope;   /* d_h^R, width of q^R and of the shared k^R, 0..1024  */
  int32_t d_latent; /* d_c, width of c^KV, 1..2048                         */
  int32_t dtype;    /* mla_dtype_t: storage type of every float tensor     */
} mla_dims_t;

/* The latent cache of one layer.  Row = d_latent + d_rope elements,
 * [c^KV | k^R].  Rows [0, seq_lens[b]) of request b are attended; the
 * current token's row must already be appended (the query attends positions
 * 1..t, zeeklog notes, decode paragraphs). */
typedef struct {
  const void* data;          /* contiguous: [batch, max_len, row];
                                paged:      [num_pages, page_size, row]        */
  const int32_t* seq_lens;   /* device [batch], each in [0, max_len]           */
  const int32_t* page_table; /* device [batch, max_len / page_size] physical
                                page ids in [0, num_pages); NULL = contiguous  */
  int32_t page_size;         /* tokens per page (paged only; 0 = contiguous)   */
  int32_t max_len;           /* host-known bound on every seq_lens[b]; the row
                                stride between requests of a contiguous cache;
                                a multiple of page_size when paged            */
  int64_t num_pages;         /* paged: pages in the pool; ignored otherwise    */
  const float* scales;       /* MLA_ROWS_FP8: device, one fp32 per row, indexed
                                like the rows of data ([batch, max_len] or
                                [num_pages, page_size]); NULL otherwise       */
  int32_t row_format;        /* mla_row_format_t                               */
} mla_cache_t;

/* Split-KV plan: each request's tokens are cut into partitions that run on
 * different compute units and are merged by their log-sum-exp weights.
 * Produced by mla_decode_plan or mla_decode_plan_mq; every decode call takes
 * its query count from it.
 * Uniform plan (split_tokens > 0): partitions of split_tokens tokens, the
 * same cut for every batch, sized from max_len.
 * Length-balanced plan (split_tokens == 0; the MFMA kernel's default when the
 * batch alone does not fill the compute units, at most 256 requests and
 * max_len <= 2^22): the decode kernel reads seq_lens on the device and picks
 * one partition length c (a multiple of 32 tokens) per call, the smallest
 * for which the requests' partition counts ceil(seq_lens[b] / c) add up to
 * at most one workgroup per compute unit; no host synchronisation.  The
 * split of a request's rows changes only the rounding of the result. */
typedef struct {
  int32_t split_tokens;   /* tokens per partition; 0: length-balanced plan     */
  int32_t num_splits;     /* uniform: partitions per request,
                             ceil(max_len/split_tokens); balanced: the most
                             partitions one request can get                   */
  int32_t kernel;         /* 0 = generic fp32-VALU kernel; bf16 MFMA kernel with
                             1 = 128 or 2 = 64 query rows per workgroup (2:
                             chosen for several splits of at most 256 tokens;
                             the four waves then split the score contraction
                             and the latent output in halves)                 */
  int32_t head_groups;    /* query rows (q_len * n_heads) are processed in this
                             many groups                                      */
  int32_t q_len;          /* query tokens per request (1 = plain decode)       */
  size_t workspace_bytes; /* device bytes mla_decode_attn needs                */
  int32_t partitions;     /* (request, partition) pairs one call has room for:
                             batch * num_splits (uniform) or the balanced
                             plan's capacity                                  */
} mla_decode_plan_t;

/* Device bytes of workspace mla_decode_attn needs for `batch` requests of
 * at most max_len cached rows and one query token each, with the plan
 * mla_decode_plan would choose (split_tokens = 0) for a contiguous cache of
 * native rows on the current device: plan.workspace_bytes of that plan.
 * Host only; allocates nothing and enqueues nothing.  Returns 0 for invalid
 * dims, batch < 0, max_len < 0 or no current gfx950 device.  (A paged or
 * low-bit cache, several query tokens or an explicit split size can need a
 * different amount: take plan->workspace_bytes from mla_decode_plan or
 * mla_decode_plan_mq for those.) */
size_t mla_decode_workspace_bytes(const mla_dims_t* dims, int32_t batch, int32_t max_len);

/* Human-readable name of a status code (static storage; never NULL). */
const char* mla_status_str(mla_status_t status);

/* Library ABI version (incremented on any signature change; 2 added
 * mla_decode_plan_t.q_len and mla_decode_plan_mq; 3 added mla_cache_t.scales,
 * mla_cache_t.row_format and mla_quantize_rows; 4 added mla_prefill_expand and
 * mla_prefill_attn; 5 added mla_decode_workspace_bytes and the 64-row form of
 * the MFMA kernel, plan->kernel 2; 6 added length-balanced plans and
 * mla_decode_plan_t.partitions). */
int32_t mla_abi_version(void);

/* Absorb W^UK into the query (V2 read-through section 2.3; V3 read-through
 * section 2.3):
 *   q_cat[b, i, c]       = sum_h q_c[b, i, h] * w_uk[i, h, c]   (c < d_latent)
 *   q_cat[b, i, d_c + r] = q_r[b, i, r]                          (r < d_rope)
 * q_c  [batch, n_heads, d_head], q_r [batch, n_heads, d_rope],
 * w_uk [n_heads, d_head, d_latent] (head i's d_h x d_c block of W^UK),
 * q_cat [batch, n_heads, d_latent + d_rope] (output; mirrors the cache row).
 * Accumulates in fp32; the result is rounded once to dims->dtype.
 * batch 0 is a no-op returning MLA_OK. */
mla_status_t mla_absorb_q(const mla_dims_t* dims, int32_t batch, const void* q_c,
                          const void* q_r, const void* w_uk, void* q_cat, void* stream);

/* Choose the split-KV plan for mla_decode_attn on the current device.
 * split_tokens = 0 lets the library choose; otherwise the value is rounded up
 * to the kernel's tile granule (32 tokens for the MFMA kernel, 1 otherwise)
 * and capped at max_len rounded up to that granule.
 * `plan` is a host pointer that receives the result. */
mla_status_t mla_decode_plan(const mla_dims_t* dims, int32_t batch, const mla_cache_t* cache,
                             int32_t split_tokens, mla_decode_plan_t* plan);

/* As mla_decode_plan, for q_len query tokens per request (1 <= q_len <= 1024):
 * the verification pass of speculative decoding, where tokens proposed by the
 * extra prediction depths are checked by the main model in one step (V3
 * read-through section 4.1), or a chunk of a prompt whose rows were just
 * appended (chunked prefill, in the absorbed form).  The last q_len cached rows of request b are the
 * new tokens; query token j (0-based) is the one at position
 * seq_lens[b] - q_len + j and attends causally to rows
 * 0 .. seq_lens[b] - q_len + j (zeeklog MHA equation: attention over
 * positions 1..t).  With such a plan every decode call takes q_cat as
 * [batch, q_len, n_heads, d_latent + d_rope] and writes out_lat
 * [batch, q_len, n_heads, d_latent], lse [batch, q_len, n_heads] and, for
 * mla_decode_combine_out, out [batch, q_len, n_heads, d_head]; a token with
 * no visible row gets out_lat = 0 and lse = -inf.  q_len outside 1..1024 ->
 * MLA_ERR_DIMS; other errors as mla_decode_plan. */
mla_status_t mla_decode_plan_mq(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                                const mla_cache_t* cache, int32_t split_tokens,
                                mla_decode_plan_t* plan);

/* Latent-space decode attention over the cache (V2 read-through section 2.3:
 * scores against the cached latent, weighted sum in latent space; zeeklog MHA
 * equation for the softmax):
 *   s[b,i,j]     = softmax_scale * q_cat[b,i,:] . row_j(b)[:]   (j < seq_lens[b])
 *   out_lat[b,i] = sum_j softmax_j(s[b,i,:]) * row_j(b)[0:d_latent]
 *   lse[b,i]     = ln sum_j exp(s[b,i,j])
 * q_cat [batch, n_heads, d_latent + d_rope]; out_lat [batch, n_heads,
 * d_latent] (dims->dtype); lse [batch, n_heads] fp32, may be NULL.
 * A request with seq_lens[b] == 0 yields out_lat = 0 and lse = -inf.
 * `plan` (host pointer) may be NULL: the library plans with split_tokens = 0
 * and one query token.  A plan passed in must come from mla_decode_plan (or
 * mla_decode_plan_mq, whose q_len then sets the shapes) with the same dims,
 * batch and cache bounds.  workspace: device, >= plan->workspace_bytes, 256-byte
 * aligned, contents need no initialisation; calls that share a workspace
 * must be ordered on one stream.  With a one-split plan on the MFMA kernel
 * (plan->split_tokens > 0, plan->num_splits == 1, plan->kernel 1 or 2) over
 * native rows the decode kernel normalises its rows and writes out_lat and
 * lse itself: nothing is merged and the workspace is not touched; otherwise
 * the call is mla_decode_partials followed by mla_decode_combine. */
mla_status_t mla_decode_attn(const mla_dims_t* dims, int32_t batch, const void* q_cat,
                             const mla_cache_t* cache, float softmax_scale,
                             const mla_decode_plan_t* plan, void* out_lat, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream);

/* mla_decode_attn for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, arguments and errors, with no workspace argument.  The
 * workspace is a static device array in the library, 48 MiB
 * (mla_decode_noalloc_max_bytes()), one copy per device, held from the first
 * call on that device until the process ends; the call allocates nothing.  A
 * plan whose workspace_bytes exceed it -> MLA_ERR_WORKSPACE (nothing is
 * enqueued); MLA_ERR_DEVICE if the array's device address cannot be found.
 * Every call on one device shares its array: calls that may overlap on one
 * device (different streams) race and must not be issued; the array's
 * contents need no initialisation and are left undefined. */
mla_status_t mla_decode_attn_noalloc(const mla_dims_t* dims, int32_t batch, const void* q_cat,
                                     const mla_cache_t* cache, float softmax_scale,
                                     const mla_decode_plan_t* plan, void* out_lat, float* lse,
                                     void* stream);

/* Size in bytes of mla_decode_attn_noalloc's static workspace (48 MiB). */
size_t mla_decode_noalloc_max_bytes(void);

/* The two phases of mla_decode_attn, for callers that merge partial results
 * themselves (for example across devices that each hold a slice of a long
 * cache) or time them separately.  mla_decode_attn(...) is exactly
 * mla_decode_partials(...) followed by mla_decode_combine(...) on the same
 * stream with the same plan and workspace.
 *
 * mla_decode_partials: for every request b, split s and head i with tokens in
 *   [s*c, min((s+1)*c, seq_lens[b])) (c = split_tokens, or in a balanced plan
 *   the length this call picks), writes into the workspace the split's
 *   softmax-weighted latent sum and the fp32 statistics that weight it in
 *   the merge (its natural-log sum-exp among them), and in a balanced plan
 *   the partition table the combine reads.  The workspace layout is private
 *   to the library and depends on the plan.  Splits with no tokens are not
 *   written.
 * mla_decode_combine: merges the used splits of each request, split s
 *   weighted by exp(lse_s - max_s lse_s) relative to its normalised sum, into
 *   out_lat (dims->dtype) and lse (fp32, may be NULL); it reads only seq_lens
 *   from `cache` (data may be NULL).
 * Arguments, errors and the plan rule are those of mla_decode_attn. */
mla_status_t mla_decode_partials(const mla_dims_t* dims, int32_t batch, const void* q_cat,
                                 const mla_cache_t* cache, float softmax_scale,
                                 const mla_decode_plan_t* plan, void* workspace,
                                 size_t workspace_bytes, void* stream);
mla_status_t mla_decode_combine(const mla_dims_t* dims, int32_t batch, const mla_cache_t* cache,
                                const mla_decode_plan_t* plan, const void* workspace,
                                size_t workspace_bytes, void* out_lat, float* lse,
                                void* stream);

/* The tail of a decode step in one pass: mla_decode_combine followed by
 * mla_out_uv on its result, without a separate launch for the projection.
 * The merged latent output is the softmax-weighted latent sum of every cached
 * row; W^UV is applied to it afterwards (V2 read-through section 2.3):
 *   out_lat[b, i, :] = merged partials of mla_decode_partials (as
 *                      mla_decode_combine; required)
 *   lse[b, i]        = merged log-sum-exp (fp32; may be NULL)
 *   out[b, i, h]     = sum_c out_lat[b, i, c] * w_uv[i, c, h]
 * w_uv [n_heads, d_latent, d_head] and out [batch, n_heads, d_head] as in
 * mla_out_uv; dims->d_head must be set.  The projection reads out_lat as
 * rounded to dims->dtype, exactly as the two separate calls would.  Up to
 * 32 requests (MFMA plan) this is one kernel; beyond, where that kernel would
 * re-read W^UV once per 8 requests, it is the two calls in sequence.  Plan,
 * workspace, cache and error rules are those of mla_decode_combine; a NULL
 * w_uv or out returns MLA_ERR_NULL, a misaligned one MLA_ERR_ALIGN. */
mla_status_t mla_decode_combine_out(const mla_dims_t* dims, int32_t batch,
                                    const mla_cache_t* cache, const mla_decode_plan_t* plan,
                                    const void* workspace, size_t workspace_bytes,
                                    const void* w_uv, void* out, void* out_lat, float* lse,
                                    void* stream);

/* Apply W^UV after the latent-space sum (V2 read-through section 2.3):
 *   out[b, i, h] = sum_c out_lat[b, i, c] * w_uv[i, c, h]
 * out_lat [batch, n_heads, d_latent], w_uv [n_heads, d_latent, d_head]
 * (head i's up-projection stored d_c x d_h), out [batch, n_heads, d_head].
 * Accumulates in fp32, rounds once to dims->dtype. */
mla_status_t mla_out_uv(const mla_dims_t* dims, int32_t batch, const void* out_lat,
                        const void* w_uv, void* out, void* stream);

/* Rotary position encoding of the decoupled key k^R.  Pairs (x[2i], x[2i+1])
 * turn by pos * f_i, f_i = base^(-2i/d_rope).  With yarn_scale s != 1 the
 * frequencies follow YaRN's interpolation (Peng et al. 2023), which the
 * DeepSeek-V2 long-context extension applies to k^R only (ai-library
 * "DeepSeek-V2" notes, "Long-Context Extension"; zeeklog notes: s = 40,
 * alpha = 1, beta = 32, from a 4K context): with r_i = L f_i / (2 pi) the
 * number of turns pair i makes over the original context L, f_i is kept for
 * r_i >= beta, divided by s for r_i <= alpha and blended linearly in r
 * between.  YaRN's attention-temperature factor is not applied here: it
 * belongs to the decode step's softmax_scale. */
typedef struct {
  float base;                 /* > 0 (10000 is the usual value)                */
  float yarn_scale;           /* s > 0; 1 = plain RoPE                         */
  float yarn_alpha;           /* ramp start, in turns over the original context */
  float yarn_beta;            /* ramp end, > yarn_alpha (when yarn_scale != 1)  */
  int32_t yarn_original_len;  /* L > 0 (when yarn_scale != 1)                  */
} mla_rope_t;

/* Quantise rows to the low-bit cache format (MLA_ROWS_FP8): for each of the
 * n_rows rows of `width` elements,
 *   scale[r] = max_j |x[r, j]| / 448   (1 for an all-zero row; fp32 division)
 *   dst[r, j] = E4M3(x[r, j] / scale[r])   (fp32 division, round to nearest
 *               with ties to even, |.| <= 448 by construction, sign kept)
 * src [n_rows, width] device, src_dtype (MLA_F32 or MLA_BF16); dst
 * [n_rows, width] device bytes; scales [n_rows] device fp32.  A contiguous or
 * paged cache is quantised as its flat array of rows.  n_rows < 0 or width
 * outside 1..4096 -> MLA_ERR_DIMS; NULL pointer -> MLA_ERR_NULL; src not
 * 16-byte aligned -> MLA_ERR_ALIGN.  Asynchronous on `stream`. */
mla_status_t mla_quantize_rows(int64_t n_rows, int32_t width, int32_t src_dtype, const void* src,
                               void* dst, float* scales, void* stream);

/* Device bytes of workspace mla_cache_append needs for these sizes. */
size_t mla_cache_append_workspace_bytes(const mla_dims_t* dims, int32_t batch, int32_t d_model);

/* Append the new token of each request to the latent cache (V3 read-through
 * section 2.2: the KV-side listing and cache.append((c_kv, k_r)); section
 * 2.3: k_r = RoPE(W_kr h_t); ai-library "DeepSeek-V2" notes, "Model
 * configuration": RMSNorm after the compressed latent):
 *   c     = W^DKV h[b]                       (d_latent values)
 *   c'    = c / sqrt(mean(c^2) + rms_eps) * rms_weight
 *   k     = RoPE(W^KR h[b], positions[b])    (d_rope values, see mla_rope_t)
 *   row positions[b] of request b := [c' | k]
 * h [batch, d_model], w_dkv [d_latent, d_model], w_kr [d_rope, d_model],
 * rms_weight [d_latent], all in dims->dtype; positions device int32 [batch].
 * The row is written through cache->data (contiguous or paged exactly as
 * mla_decode_attn reads it); positions outside [0, max_len) write nothing.
 * Updating seq_lens is the caller's.  Accumulates in fp32 (angles in fp64),
 * rounds once to dims->dtype; into a low-bit cache (MLA_ROWS_FP8) the fp32
 * row is quantised as mla_quantize_rows does and its scale written to
 * cache->scales.  Uses dims->d_latent, d_rope and dtype;
 * d_rope must be even.  Errors: NULL pointers (with batch > 0) ->
 * MLA_ERR_NULL; d_model < 1, odd d_rope, rms_eps < 0 or not finite, a bad
 * rope description -> MLA_ERR_DIMS; h, the weights or cache->data not
 * 16-byte aligned -> MLA_ERR_ALIGN; workspace NULL or smaller than
 * mla_cache_append_workspace_bytes -> MLA_ERR_WORKSPACE. */
mla_status_t mla_cache_append(const mla_dims_t* dims, int32_t batch, int32_t d_model,
                              const void* h, const void* w_dkv, const void* w_kr,
                              const void* rms_weight, float rms_eps, const mla_rope_t* rope,
                              const int32_t* positions, const mla_cache_t* cache,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ---- A chunk of new tokens in the primary (unabsorbed) form ----
 * For a long chunk of new tokens (prefill) the explicit per-head keys and
 * values can cost less than absorption: the up-projection (zeeklog equations
 * 10-11) is paid once per cached row and shared by every query of the chunk,
 * after which each query-key pair costs (d_h + d_h^R) + d_h multiply-adds per
 * head instead of (d_c + d_h^R) + d_c (V2 read-through section 2.3 places the
 * absorption's gain at decode).  Two calls:
 *   mla_prefill_expand  k_c[b,i,t] = W^UK_i c_t,  v[b,i,t,h] = sum_c W^UV[i,c,h] c_t[c]
 *   mla_prefill_attn    causal attention of the chunk over [k_c ; k^R] and v
 * Supported: dims->dtype MLA_BF16, d_head 128, d_rope 64, d_latent 512, any
 * n_heads >= 1; a contiguous cache (page_table NULL) of native rows.  Other
 * dims -> MLA_ERR_DIMS, other storage -> MLA_ERR_DTYPE. */

/* Explicit keys and values of every cached row of each request (rows
 * 0 .. seq_lens[b]-1; the rows past the length are not written):
 *   k_c[b, i, t, :] = W^UK[i] c_t        (w_uk [n_heads, d_head, d_latent])
 *   v  [b, i, t, h] = sum_c w_uv[i, c, h] c_t[c]   (w_uv [n_heads, d_latent, d_head])
 * with c_t = row t of request b [0:d_latent].  k_c and v: device,
 * [batch, n_heads, cache->max_len, d_head] bf16, caller-owned (2 * batch *
 * n_heads * max_len * d_head * 2 bytes together).  fp32 accumulation, one
 * rounding to bf16.  batch 0 is a no-op. */
mla_status_t mla_prefill_expand(const mla_dims_t* dims, int32_t batch, const mla_cache_t* cache,
                                const void* w_uk, const void* w_uv, void* k_c, void* v,
                                void* stream);

/* Causal attention of q_len new tokens per request, unabsorbed (zeeklog MHA
 * equation; keys [k^C ; k^R] with k^R shared by the heads, ai-library
 * "Multi-Head Latent Attention"): token j of request b sits at position
 * seq_lens[b] - q_len + j (its row already in the cache and expanded) and
 *   s[t]         = softmax_scale * (q_c[b,j,i] . k_c[b,i,t] + q_r[b,j,i] . k^R_t)
 *   out[b,j,i,:] = sum_{t <= pos} softmax_t(s) v[b,i,t,:]
 *   lse[b,j,i]   = ln sum_{t <= pos} exp(s[t])
 * q_c [batch, q_len, n_heads, d_head], q_r [batch, q_len, n_heads, d_rope],
 * k_c and v as written by mla_prefill_expand, k^R_t = cache row t [d_latent:];
 * out [batch, q_len, n_heads, d_head] bf16, lse fp32 (may be NULL).  A token
 * with no visible row gets out = 0 and lse = -inf.  q_len outside
 * 1..cache->max_len -> MLA_ERR_DIMS.  fp32 scores, softmax and accumulation;
 * the probabilities enter the value product as bf16. */
mla_status_t mla_prefill_attn(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                              const void* q_c, const void* q_r, const mla_cache_t* cache,
                              const void* k_c, const void* v, float softmax_scale, void* out,
                              float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_ABSORB_H */
