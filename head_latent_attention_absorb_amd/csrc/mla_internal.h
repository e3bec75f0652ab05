// Internal declarations shared by the kernels and the C-ABI layer.
// Nothing here is part of the public ABI (include/mla_absorb.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Split-KV partial results of the decode kernels live in the caller's
// workspace: row-major partial outputs of d_latent elements and
// per (request, split, head) statistics behind them.  The generic kernel
// writes fp32 sums normalised by their own softmax sum and the fp32
// natural-log sum-exp, split-major ([request, split, row]); the MFMA kernel
// writes bf16 sums relative to a reference max m (not normalised) and the
// fp32 pair (log-sum-exp, m), both in base-2 log units, partition-major
// ([partition, row]): partition s of request b is number off_b + s, where
// off_b = b * num_splits in a uniform plan and, in a length-balanced one
// (MFMA only), the number of partitions of the requests before b.  The
// balanced launch sizes its partitions on the device and leaves the
// partition table behind the statistics: [0] the partition length c,
// [1 + b] off_b, [1 + batch] the partition count.

struct CacheView {
  const uint8_t* data;      // cache rows, (d_latent + d_rope) elements each
  const float* scales;      // FP8 rows: one fp32 scale per row, else nullptr
  int32_t fp8;              // 1: rows of OCP E4M3 bytes scaled by `scales`
  const int32_t* seq_lens;  // [batch]
  const int32_t* page_table;  // [batch, max_pages] or nullptr
  int32_t page_size;        // 0 => contiguous
  int32_t max_len;
  int32_t max_pages;        // max_len / page_size when paged
};

// Several query tokens per request (q_len > 1): q_cat, the outputs and the
// partials hold q_len * n_heads rows per request, token-major ([B, q_len,
// n_heads, ...]); query token j of request b is the one at position
// seq_lens[b] - q_len + j and attends to the rows up to its own position,
// seq_lens[b] - (q_len - 1 - j) of them.
struct DecodeArgs {
  int32_t batch, n_heads, d_latent, d_rope, dtype;
  int32_t q_len;        // query tokens per request (1 for plain decode)
  const void* q_cat;
  CacheView cache;
  float softmax_scale;
  int32_t split_tokens, num_splits, head_groups;
  // MFMA kernel: query rows per workgroup, 128 or 64 (head_groups = q_len *
  // n_heads / group_rows).
  int32_t group_rows = 128;
  // Partitions one launch has room for (batch * num_splits in a uniform
  // plan).  Length-balanced plan (split_tokens == 0): the device picks the
  // partition length, for about part_target partitions of at most
  // part_max_tokens tokens, and writes the partition table to part_table.
  int32_t partitions = 0;
  int32_t part_target = 0, part_max_tokens = 0;
  int32_t* part_table = nullptr;
  void* out_lat;
  float* lse;           // may be nullptr
  void* part_o;         // workspace: fp32 (generic kernel) or bf16 (MFMA kernel)
  float* part_lse;      // workspace: lse (generic kernel) or (lse, m) pairs (MFMA kernel)
  hipStream_t stream;
  // MFMA kernel with one split: write out_lat and lse directly (no partials,
  // no combine).
  bool direct = false;
};

// Launchers return the hipError_t of the launch (hipSuccess when nothing
// needed launching).
hipError_t launch_absorb_q(int dtype, int batch, int n_heads, int d_head, int d_rope,
                           int d_latent, const void* q_c, const void* q_r,
                           const void* w_uk, void* q_cat, hipStream_t stream);
hipError_t launch_out_uv(int dtype, int batch, int n_heads, int d_head, int d_latent,
                         const void* out_lat, const void* w_uv, void* out,
                         hipStream_t stream);

// Unabsorbed chunk form (bf16, d_h = 128, d_h^R = 64, d_c = 512, contiguous
// native cache): explicit keys and values of the cached rows, then causal
// attention of q_len new tokens per request over them.
bool prefill_supported(int dtype, int n_heads, int d_head, int d_latent, int d_rope);
hipError_t launch_expand_kv(int batch, int n_heads, const CacheView& cache, const void* w_uk,
                            const void* w_uv, void* k_c, void* v, hipStream_t stream);
hipError_t launch_prefill_attn(int batch, int q_len, int n_heads, const CacheView& cache,
                               const void* q_c, const void* q_r, const void* k_c,
                               const void* v, float softmax_scale, void* out, float* lse,
                               hipStream_t stream);

// Generic split-KV partials (fp32 VALU arithmetic, any dims, fp32 or bf16
// storage), row-major partial layout.
hipError_t launch_partials_generic(const DecodeArgs& a);
// bf16 MFMA split-KV partials for d_latent = 512, d_rope = 64,
// n_heads % 128 == 0.
hipError_t launch_partials_mfma(const DecodeArgs& a);
// Merge the partials of each request into out_lat / lse.  `mfma_partials`
// selects the layout written by the MFMA kernel (else the generic one).
hipError_t launch_combine(const DecodeArgs& a, bool mfma_partials);
// Merge of the MFMA kernel's partials into out_lat / lse and, when w_uv is
// not null, the W^UV product of the merged rows into out in the same kernel
// (requires combine_out_fusable(d_latent, d_head)).
bool combine_out_fusable(int d_latent, int d_head);
// (w_uv is indexed by head, out by row: [B, q_len, n_heads, d_head].)
hipError_t launch_combine_rows(const DecodeArgs& a, const void* w_uv, void* out, int d_head);

// Cache append: projections of the new token's hidden state, RMSNorm of the
// latent, RoPE (optionally YaRN) of the key, row written at `positions[b]`
// of request b through `cache_data` (the layout of `cache`).  The workspace
// holds fp32 partial sums, append_workspace_bytes() of them.
size_t append_workspace_bytes(int dtype, int batch, int d_model, int d_c, int d_r);
hipError_t launch_cache_append(int dtype, int batch, int d_model, int d_c, int d_r,
                               const void* h, const void* w_dkv, const void* w_kr,
                               const void* gamma, float eps, double base, double yarn_scale,
                               double yarn_alpha, double yarn_beta, double yarn_len,
                               const int32_t* positions, const CacheView& cache,
                               void* cache_data, void* workspace, hipStream_t stream);

// Low-bit cache rows: E4M3 codes and one fp32 scale per row (src fp32 or
// bf16 per src_dtype).
hipError_t launch_quantize_rows(int src_dtype, int64_t n_rows, int width, const void* src,
                                void* dst, float* scales, hipStream_t stream);

// Length-balanced plans: the most requests (each lane of a wave keeps four
// lengths in registers while the device sizes the partitions) and the
// longest cache (lengths convert exactly to fp32, and their sum fits int32).
constexpr int kBalancedMaxBatch = 256;
constexpr int kBalancedMaxLen = 1 << 22;

// Constants of the MFMA decode kernel that the planner needs.
constexpr int kMfmaHeadsPerGroup = 128;  // query rows of a workgroup (128-row form)
constexpr int kMfmaHalfGroup = 64;       // query rows of a workgroup (64-row form)
constexpr int kMfmaTokenGranule = 32;    // tokens consumed per workgroup iteration
// The 64-row form is chosen when the 128-row plan would give each
// workgroup at most this many tokens (8 steps): there the partial sums
// written per split weigh most against the steps.
constexpr int kMfmaHalfGroupMaxSplit = 256;

}  // namespace mla
