// C ABI of the MLA absorbed-decode library: argument checks, split-KV
// planning and kernel dispatch.  Declared in include/mla_absorb.h.

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string.h>

#include "mla_absorb.h"
#include "mla_internal.h"

namespace {

using mla::DecodeArgs;

constexpr int kMaxDevices = 64;

// Workspace of mla_decode_attn_noalloc: a static device array, one copy per
// device the library runs on, held until the process ends.  Host code never
// passes `scratch` itself (on the host it is only a stand-in for the symbol):
// the device address comes from hipGetSymbolAddress, once per device, below.
constexpr size_t kScratchBytes = size_t{48} << 20;
__device__ __align__(256) static uint8_t scratch[kScratchBytes];

struct DeviceInfo {
  bool valid = false;
  bool gfx950 = false;
  int cus = 0;
  void* scratch = nullptr;  // device address of `scratch` (null if the lookup failed)
};

std::mutex g_dev_mu;
DeviceInfo g_dev[kMaxDevices];

// Properties of the current device, queried once per device.
mla_status_t current_device(DeviceInfo* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.valid) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MLA_ERR_DEVICE;
    d.cus = prop.multiProcessorCount;
    d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (d.gfx950) {
      void* ptr = nullptr;
      d.scratch = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess ? ptr : nullptr;
      (void)hipGetLastError();
    }
    d.valid = true;
  }
  if (!d.gfx950) return MLA_ERR_DEVICE;
  *out = d;
  return MLA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mla_status_t check_dims(const mla_dims_t* d) {
  if (d == nullptr) return MLA_ERR_NULL;
  if (d->dtype != MLA_F32 && d->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (d->n_heads < 1 || d->n_heads > 1024 || d->d_head < 1 || d->d_head > 1024 ||
      d->d_rope < 0 || d->d_rope > 1024 || d->d_latent < 1 || d->d_latent > 2048)
    return MLA_ERR_DIMS;
  return MLA_OK;
}

bool use_mfma(const mla_dims_t* d, const mla_cache_t* c) {
  // Low-bit rows are loaded a whole 32-token tile at a time, which must lie
  // within one page.
  const int page_align = c->row_format == MLA_ROWS_FP8 ? 32 : 8;
  return d->dtype == MLA_BF16 && d->d_latent == 512 && d->d_rope == 64 &&
         d->n_heads % mla::kMfmaHeadsPerGroup == 0 &&
         (c->page_table == nullptr ||
          (c->page_size % page_align == 0 && c->page_size >= page_align));
}

mla_status_t check_cache(const mla_cache_t* c) {
  if (c == nullptr) return MLA_ERR_NULL;
  if (c->row_format != MLA_ROWS_NATIVE && c->row_format != MLA_ROWS_FP8) return MLA_ERR_DTYPE;
  if (c->max_len < 0) return MLA_ERR_DIMS;
  if (c->page_table != nullptr) {
    if (c->page_size < 1 || c->max_len % c->page_size != 0 || c->num_pages < 1)
      return MLA_ERR_DIMS;
  } else if (c->page_size != 0) {
    return MLA_ERR_DIMS;
  }
  return MLA_OK;
}

size_t round256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Most query tokens per request a plan accepts (a prefill chunk at most).
constexpr int kMaxQueryLen = 1024;

// Bytes of one partial output element: the MFMA kernel stores bf16 partials.
size_t partial_elem_bytes(bool mfma) { return mfma ? 2 : sizeof(float); }

// Per (request, split, head) the generic kernel keeps its log-sum-exp, the
// MFMA kernel the pair (log-sum-exp, reference max) of its unnormalised sum.
size_t partial_stat_bytes(bool mfma) { return mfma ? 2 * sizeof(float) : sizeof(float); }

// Workspace layout: partial rows of `partitions` (request, partition) pairs,
// then their statistics, then (length-balanced plans) the partition table:
// the partition length, each request's first partition and the count.
size_t partials_bytes(const mla_dims_t* d, int q_len, int partitions, bool mfma) {
  const size_t parts = static_cast<size_t>(partitions) * q_len * d->n_heads;
  return round256(parts * d->d_latent * partial_elem_bytes(mfma));
}
size_t stats_bytes(const mla_dims_t* d, int q_len, int partitions, bool mfma) {
  const size_t parts = static_cast<size_t>(partitions) * q_len * d->n_heads;
  return round256(parts * partial_stat_bytes(mfma));
}
size_t table_bytes(int batch, bool balanced) {
  return balanced ? round256((static_cast<size_t>(batch) + 2) * sizeof(int32_t)) : 0;
}
size_t workspace_for(const mla_dims_t* d, int batch, int q_len, int partitions, bool mfma,
                     bool balanced) {
  return partials_bytes(d, q_len, partitions, mfma) + stats_bytes(d, q_len, partitions, mfma) +
         table_bytes(batch, balanced);
}

// Bounds of a length-balanced plan: about `target` partitions (one
// workgroup per compute unit), each at most c_max tokens, and the room the
// launch keeps for them.
struct BalancedBounds {
  int target, c_max, capacity;
};

// Longest partition the kernels take: the cache's length rounded up to the
// kernel's token granule; on the MFMA kernel over a paged cache at most 63
// pages' worth (it keeps a partition's page ids in one register per lane,
// so a partition may touch at most 64 pages).
int partition_cap(const mla_cache_t* c, bool mfma) {
  const int granule = mfma ? mla::kMfmaTokenGranule : 1;
  const int max_len = c->max_len;
  int cap = max_len > 0 ? (max_len + granule - 1) / granule * granule : granule;
  if (mfma && c->page_table != nullptr)
    cap = std::min(cap, (63 * c->page_size) / granule * granule);
  return cap;
}

BalancedBounds balanced_bounds(int batch, int groups, int c_max, int max_len,
                               const DeviceInfo& dev) {
  BalancedBounds bb;
  bb.target = std::max(1, dev.cus / groups);
  bb.c_max = c_max;
  // With c capped at c_max a request takes up to ceil(max_len / c_max)
  // partitions, whatever the target.
  const int per_request = max_len > 0 ? (max_len + c_max - 1) / c_max : 1;
  bb.capacity = std::max(bb.target, batch * per_request);
  return bb;
}

// form: -1 lets the planner choose the kernel form; 0, 1 or 2 asks for that
// plan->kernel (a caller's plan being checked), MLA_ERR_DIMS if these dims
// cannot run it.
mla_status_t make_plan(const mla_dims_t* d, int batch, int q_len, const mla_cache_t* c,
                       int split_req, const DeviceInfo& dev, mla_decode_plan_t* plan,
                       int form = -1) {
  if (q_len < 1 || q_len > kMaxQueryLen) return MLA_ERR_DIMS;
  if (split_req < 0) return MLA_ERR_DIMS;
  const bool mfma = use_mfma(d, c);
  const int granule = mfma ? mla::kMfmaTokenGranule : 1;
  const int max_len = c->max_len;
  const int c_max = partition_cap(c, mfma);
  // Split length for `groups` row groups per request: the caller's, or about
  // one workgroup per compute unit when every request is at max_len.
  auto choose_split = [&](int groups) {
    int split;
    if (split_req > 0) {
      split = (split_req + granule - 1) / granule * granule;
    } else {
      const long long per_split = static_cast<long long>(batch > 0 ? batch : 1) * groups;
      const long long target = mfma ? dev.cus : 2LL * dev.cus;
      const long long splits = (target + per_split - 1) / per_split;
      const long long raw = (max_len + splits - 1) / (splits > 0 ? splits : 1);
      split = static_cast<int>((raw + granule - 1) / granule * granule);
      const int floor_tokens = mfma ? 2 * granule : 64;
      if (split < floor_tokens) split = floor_tokens;
    }
    return std::min(split, c_max);
  };
  auto splits_of = [&](int split) { return max_len > 0 ? (max_len + split - 1) / split : 1; };
  // MFMA: 128 query rows per workgroup, or 64 when the 128-row plan has
  // several splits of at most kMfmaHalfGroupMaxSplit tokens (bf16 rows
  // only): half the query and partial bytes per split for twice the
  // workgroups per request, which pays where each workgroup runs few steps.
  // Head groups count the query rows of all q_len tokens of a request.
  int rows = 1, kernel = 0;
  if (mfma) {
    kernel = 1;
    if (form >= 0) {
      if (form != 1 && (form != 2 || c->row_format != MLA_ROWS_NATIVE)) return MLA_ERR_DIMS;
      kernel = form;
    } else if (c->row_format == MLA_ROWS_NATIVE) {
      const int split128 = choose_split(q_len * d->n_heads / mla::kMfmaHeadsPerGroup);
      if (splits_of(split128) > 1 && split128 <= mla::kMfmaHalfGroupMaxSplit) kernel = 2;
    }
    rows = kernel == 2 ? mla::kMfmaHalfGroup : mla::kMfmaHeadsPerGroup;
  } else if (form > 0) {
    return MLA_ERR_DIMS;
  }
  const int groups = q_len * d->n_heads / rows;
  plan->kernel = kernel;
  plan->head_groups = groups;
  plan->q_len = q_len;
  // Length-balanced partitions when the requests alone leave compute units
  // idle: the device then sizes the partitions from the actual lengths
  // (a uniform cut sized from max_len leaves the units of short requests
  // idle and makes the longest request's partitions the critical path).
  const bool balanced = mfma && split_req == 0 && batch >= 1 &&
                        batch <= mla::kBalancedMaxBatch && max_len <= mla::kBalancedMaxLen &&
                        static_cast<long long>(batch) * groups < dev.cus;
  if (balanced) {
    const BalancedBounds bb = balanced_bounds(batch, groups, c_max, max_len, dev);
    plan->split_tokens = 0;
    plan->num_splits = std::min(bb.capacity, std::max(1, (max_len + granule - 1) / granule));
    plan->partitions = bb.capacity;
  } else {
    const int split = choose_split(groups);
    plan->split_tokens = split;
    plan->num_splits = splits_of(split);
    plan->partitions = batch * plan->num_splits;
  }
  plan->workspace_bytes =
      workspace_for(d, batch, q_len, plan->partitions, mfma, plan->split_tokens == 0);
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_str(mla_status_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_DIMS: return "MLA_ERR_DIMS: size out of range or inconsistent";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: unsupported storage type";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN: device pointer not 16-byte aligned";
    case MLA_ERR_LAUNCH: return "MLA_ERR_LAUNCH: kernel launch failed";
    case MLA_ERR_DEVICE: return "MLA_ERR_DEVICE: no current gfx950 device";
  }
  return "MLA_ERR_UNKNOWN";
}

int32_t mla_abi_version(void) { return 6; }

mla_status_t mla_quantize_rows(int64_t n_rows, int32_t width, int32_t src_dtype, const void* src,
                               void* dst, float* scales, void* stream) {
  if (src_dtype != MLA_F32 && src_dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (n_rows < 0 || width < 1 || width > 4096) return MLA_ERR_DIMS;
  if (n_rows == 0) return MLA_OK;
  if (src == nullptr || dst == nullptr || scales == nullptr) return MLA_ERR_NULL;
  if (!aligned16(src)) return MLA_ERR_ALIGN;
  DeviceInfo dev;
  mla_status_t st = current_device(&dev);
  if (st != MLA_OK) return st;
  (void)hipGetLastError();
  const hipError_t e = mla::launch_quantize_rows(src_dtype, n_rows, width, src, dst, scales,
                                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

mla_status_t mla_absorb_q(const mla_dims_t* dims, int32_t batch, const void* q_c,
                          const void* q_r, const void* w_uk, void* q_cat, void* stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0) return MLA_ERR_DIMS;
  if (batch == 0) return MLA_OK;
  if (q_c == nullptr || w_uk == nullptr || q_cat == nullptr ||
      (dims->d_rope > 0 && q_r == nullptr))
    return MLA_ERR_NULL;
  if (!aligned16(q_c) || !aligned16(w_uk) || !aligned16(q_cat) ||
      (q_r != nullptr && !aligned16(q_r)))
    return MLA_ERR_ALIGN;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != MLA_OK) return st;
  (void)hipGetLastError();
  const hipError_t e = mla::launch_absorb_q(dims->dtype, batch, dims->n_heads, dims->d_head,
                                            dims->d_rope, dims->d_latent, q_c, q_r, w_uk,
                                            q_cat, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

mla_status_t mla_decode_plan(const mla_dims_t* dims, int32_t batch, const mla_cache_t* cache,
                             int32_t split_tokens, mla_decode_plan_t* plan) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (plan == nullptr) return MLA_ERR_NULL;
  if ((st = check_cache(cache)) != MLA_OK) return st;
  if (batch < 0) return MLA_ERR_DIMS;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != MLA_OK) return st;
  return make_plan(dims, batch, 1, cache, split_tokens, dev, plan);
}

mla_status_t mla_decode_plan_mq(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                                const mla_cache_t* cache, int32_t split_tokens,
                                mla_decode_plan_t* plan) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (plan == nullptr) return MLA_ERR_NULL;
  if ((st = check_cache(cache)) != MLA_OK) return st;
  if (batch < 0) return MLA_ERR_DIMS;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != MLA_OK) return st;
  return make_plan(dims, batch, q_len, cache, split_tokens, dev, plan);
}

size_t mla_decode_workspace_bytes(const mla_dims_t* dims, int32_t batch, int32_t max_len) {
  if (check_dims(dims) != MLA_OK || batch < 0 || max_len < 0) return 0;
  DeviceInfo dev;
  if (current_device(&dev) != MLA_OK) return 0;
  mla_cache_t c{};
  c.max_len = max_len;
  mla_decode_plan_t plan;
  if (make_plan(dims, batch, 1, &c, 0, dev, &plan) != MLA_OK) return 0;
  return plan.workspace_bytes;
}

}  // extern "C"

namespace {

enum DecodePart { kPartials = 1, kCombine = 2 };

// Validate a decode call and fill the kernel arguments.  `parts` says which
// of the two phases will run, so only their pointers are required.
mla_status_t prepare_decode(const mla_dims_t* dims, int32_t batch, const void* q_cat,
                            const mla_cache_t* cache, float softmax_scale,
                            const mla_decode_plan_t* plan, void* out_lat, float* lse,
                            const void* workspace, size_t workspace_bytes, void* stream,
                            int parts, mla_decode_plan_t* plan_out, DecodeArgs* a) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_cache(cache)) != MLA_OK) return st;
  if (batch < 0) return MLA_ERR_DIMS;
  if (batch == 0) return MLA_OK;  // nothing to do; callers return before launching
  if (cache->seq_lens == nullptr) return MLA_ERR_NULL;
  if ((parts & kPartials) && (q_cat == nullptr || cache->data == nullptr)) return MLA_ERR_NULL;
  if ((parts & kPartials) && cache->row_format == MLA_ROWS_FP8 && cache->scales == nullptr)
    return MLA_ERR_NULL;
  if ((parts & kCombine) && out_lat == nullptr) return MLA_ERR_NULL;
  if (((parts & kPartials) && (!aligned16(q_cat) || !aligned16(cache->data))) ||
      ((parts & kCombine) && (!aligned16(out_lat) ||
                              (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)))
    return MLA_ERR_ALIGN;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != MLA_OK) return st;

  if (plan == nullptr) {
    if ((st = make_plan(dims, batch, 1, cache, 0, dev, plan_out)) != MLA_OK) return st;
  } else {
    // A caller's plan must be one this library would produce for these sizes.
    if ((st = make_plan(dims, batch, plan->q_len, cache, plan->split_tokens, dev, plan_out,
                        plan->kernel)) != MLA_OK)
      return st;
    if (plan_out->split_tokens != plan->split_tokens ||
        plan_out->num_splits != plan->num_splits || plan_out->kernel != plan->kernel ||
        plan_out->head_groups != plan->head_groups || plan_out->q_len != plan->q_len ||
        plan_out->workspace_bytes != plan->workspace_bytes ||
        plan_out->partitions != plan->partitions)
      return MLA_ERR_DIMS;
  }
  if (workspace == nullptr || workspace_bytes < plan_out->workspace_bytes)
    return MLA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MLA_ERR_ALIGN;

  a->batch = batch;
  a->n_heads = dims->n_heads;
  a->q_len = plan_out->q_len;
  a->d_latent = dims->d_latent;
  a->d_rope = dims->d_rope;
  a->dtype = dims->dtype;
  a->q_cat = q_cat;
  a->cache.data = static_cast<const uint8_t*>(cache->data);
  a->cache.scales = cache->scales;
  a->cache.fp8 = cache->row_format == MLA_ROWS_FP8 ? 1 : 0;
  a->cache.seq_lens = cache->seq_lens;
  a->cache.page_table = cache->page_table;
  a->cache.page_size = cache->page_table ? cache->page_size : 0;
  a->cache.max_len = cache->max_len;
  a->cache.max_pages = cache->page_table ? cache->max_len / cache->page_size : 0;
  a->softmax_scale = softmax_scale;
  a->split_tokens = plan_out->split_tokens;
  a->num_splits = plan_out->num_splits;
  a->head_groups = plan_out->head_groups;
  a->group_rows = plan_out->kernel == 2 ? mla::kMfmaHalfGroup : mla::kMfmaHeadsPerGroup;
  a->out_lat = out_lat;
  a->lse = lse;
  const bool mfma = plan_out->kernel >= 1;
  uint8_t* ws = static_cast<uint8_t*>(const_cast<void*>(workspace));
  const size_t pb = partials_bytes(dims, plan_out->q_len, plan_out->partitions, mfma);
  const size_t sb = stats_bytes(dims, plan_out->q_len, plan_out->partitions, mfma);
  a->part_o = ws;
  a->part_lse = reinterpret_cast<float*>(ws + pb);
  a->partitions = plan_out->partitions;
  if (plan_out->split_tokens == 0) {
    const BalancedBounds bb = balanced_bounds(batch, plan_out->head_groups,
                                              partition_cap(cache, true), cache->max_len, dev);
    a->part_target = bb.target;
    a->part_max_tokens = bb.c_max;
    a->part_table = reinterpret_cast<int32_t*>(ws + pb + sb);
  }
  a->stream = static_cast<hipStream_t>(stream);
  return MLA_OK;
}

mla_status_t run_partials(const DecodeArgs& a, const mla_decode_plan_t& plan) {
  const hipError_t e = plan.kernel >= 1 ? mla::launch_partials_mfma(a)
                                        : mla::launch_partials_generic(a);
  return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

mla_status_t run_combine(const DecodeArgs& a, const mla_decode_plan_t& plan) {
  const hipError_t e = mla::launch_combine(a, plan.kernel >= 1);
  return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

mla_status_t mla_decode_partials(const mla_dims_t* dims, int32_t batch, const void* q_cat,
                                 const mla_cache_t* cache, float softmax_scale,
                                 const mla_decode_plan_t* plan, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  mla_decode_plan_t p;
  DecodeArgs a;
  mla_status_t st = prepare_decode(dims, batch, q_cat, cache, softmax_scale, plan, nullptr,
                                   nullptr, workspace, workspace_bytes, stream, kPartials, &p,
                                   &a);
  if (st != MLA_OK || batch == 0) return st;
  (void)hipGetLastError();
  return run_partials(a, p);
}

mla_status_t mla_decode_combine(const mla_dims_t* dims, int32_t batch, const mla_cache_t* cache,
                                const mla_decode_plan_t* plan, const void* workspace,
                                size_t workspace_bytes, void* out_lat, float* lse,
                                void* stream) {
  mla_decode_plan_t p;
  DecodeArgs a;
  mla_status_t st = prepare_decode(dims, batch, nullptr, cache, 0.f, plan, out_lat, lse,
                                   workspace, workspace_bytes, stream, kCombine, &p, &a);
  if (st != MLA_OK || batch == 0) return st;
  (void)hipGetLastError();
  return run_combine(a, p);
}

mla_status_t mla_decode_attn_noalloc(const mla_dims_t* dims, int32_t batch, const void* q_cat,
                                     const mla_cache_t* cache, float softmax_scale,
                                     const mla_decode_plan_t* plan, void* out_lat, float* lse,
                                     void* stream) {
  DeviceInfo dev;
  mla_status_t st = current_device(&dev);
  if (st != MLA_OK) return st;
  if (dev.scratch == nullptr) return MLA_ERR_DEVICE;
  // The plan's workspace must fit the static array; prepare_decode (through
  // mla_decode_attn) returns MLA_ERR_WORKSPACE otherwise.
  return mla_decode_attn(dims, batch, q_cat, cache, softmax_scale, plan, out_lat, lse,
                         dev.scratch, kScratchBytes, stream);
}

size_t mla_decode_noalloc_max_bytes(void) { return kScratchBytes; }

mla_status_t mla_decode_attn(const mla_dims_t* dims, int32_t batch, const void* q_cat,
                             const mla_cache_t* cache, float softmax_scale,
                             const mla_decode_plan_t* plan, void* out_lat, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream) {
  mla_decode_plan_t p;
  DecodeArgs a;
  mla_status_t st = prepare_decode(dims, batch, q_cat, cache, softmax_scale, plan, out_lat, lse,
                                   workspace, workspace_bytes, stream, kPartials | kCombine,
                                   &p, &a);
  if (st != MLA_OK || batch == 0) return st;
  (void)hipGetLastError();
  // One split per request: the MFMA kernel normalises its rows itself and
  // writes o_lat and lse, so there is nothing to merge.
  a.direct = p.kernel >= 1 && p.split_tokens > 0 && p.num_splits == 1 &&
             cache->row_format == MLA_ROWS_NATIVE;
  if ((st = run_partials(a, p)) != MLA_OK || a.direct) return st;
  return run_combine(a, p);
}

constexpr int32_t kFusedTailMaxBatch = 32;

mla_status_t mla_decode_combine_out(const mla_dims_t* dims, int32_t batch,
                                    const mla_cache_t* cache, const mla_decode_plan_t* plan,
                                    const void* workspace, size_t workspace_bytes,
                                    const void* w_uv, void* out, void* out_lat, float* lse,
                                    void* stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_cache(cache)) != MLA_OK) return st;
  if (batch < 0) return MLA_ERR_DIMS;
  if (batch > 0) {
    if (w_uv == nullptr || out == nullptr) return MLA_ERR_NULL;
    if (!aligned16(w_uv) || !aligned16(out)) return MLA_ERR_ALIGN;
  }
  mla_decode_plan_t p;
  DecodeArgs a;
  st = prepare_decode(dims, batch, nullptr, cache, 0.f, plan, out_lat, lse, workspace,
                      workspace_bytes, stream, kCombine, &p, &a);
  if (st != MLA_OK || batch == 0) return st;
  (void)hipGetLastError();
  // The fused kernel stages W^UV[i] once per group of 8 requests, so it
  // re-reads the weights ceil(batch / 8) times; past 32 requests the separate
  // combine and the weight-streaming projection are faster (measured at
  // n_heads 128, d_latent 512: 18.0 vs 18.9 us at 32 requests, 30.0 vs 21.4
  // at 64).
  if (p.kernel >= 1 && batch * p.q_len <= kFusedTailMaxBatch &&
      mla::combine_out_fusable(dims->d_latent, dims->d_head)) {
    const hipError_t e = mla::launch_combine_rows(a, w_uv, out, dims->d_head);
    return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
  }
  if ((st = run_combine(a, p)) != MLA_OK) return st;
  // o_lat rows are [batch, q_len, n_heads]: the projection sees batch * q_len
  // requests.
  const hipError_t e = mla::launch_out_uv(dims->dtype, batch * p.q_len, dims->n_heads,
                                          dims->d_head, dims->d_latent, out_lat, w_uv, out,
                                          a.stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

mla_status_t mla_out_uv(const mla_dims_t* dims, int32_t batch, const void* out_lat,
                        const void* w_uv, void* out, void* stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0) return MLA_ERR_DIMS;
  if (batch == 0) return MLA_OK;
  if (out_lat == nullptr || w_uv == nullptr || out == nullptr) return MLA_ERR_NULL;
  if (!aligned16(out_lat) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_ALIGN;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != MLA_OK) return st;
  (void)hipGetLastError();
  const hipError_t e = mla::launch_out_uv(dims->dtype, batch, dims->n_heads, dims->d_head,
                                          dims->d_latent, out_lat, w_uv, out,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

}  // extern "C"

// ----------------------------------------------------------------------------
// Cache append
// ----------------------------------------------------------------------------

namespace {

mla_status_t check_append(const mla_dims_t* dims, int32_t batch, int32_t d_model, float eps,
                          const mla_rope_t* rope) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (rope == nullptr) return MLA_ERR_NULL;
  if (batch < 0 || d_model < 1 || d_model > (1 << 20) || (dims->d_rope & 1) != 0 ||
      !(eps >= 0.f) || !std::isfinite(eps))
    return MLA_ERR_DIMS;
  if (!(rope->base > 0.f) || !std::isfinite(rope->base) || !(rope->yarn_scale > 0.f) ||
      !std::isfinite(rope->yarn_scale))
    return MLA_ERR_DIMS;
  if (rope->yarn_scale != 1.f &&
      (rope->yarn_original_len < 1 || !(rope->yarn_beta > rope->yarn_alpha) ||
       !std::isfinite(rope->yarn_alpha) || !std::isfinite(rope->yarn_beta)))
    return MLA_ERR_DIMS;
  return MLA_OK;
}

}  // namespace

size_t mla_cache_append_workspace_bytes(const mla_dims_t* dims, int32_t batch, int32_t d_model) {
  if (check_dims(dims) != MLA_OK || batch < 0 || d_model < 1) return 0;
  return round256(mla::append_workspace_bytes(dims->dtype, batch, d_model, dims->d_latent,
                                              dims->d_rope));
}

mla_status_t mla_cache_append(const mla_dims_t* dims, int32_t batch, int32_t d_model,
                              const void* h, const void* w_dkv, const void* w_kr,
                              const void* rms_weight, float rms_eps, const mla_rope_t* rope,
                              const int32_t* positions, const mla_cache_t* cache,
                              void* workspace, size_t workspace_bytes, void* stream) {
  mla_status_t st = check_append(dims, batch, d_model, rms_eps, rope);
  if (st != MLA_OK) return st;
  if ((st = check_cache(cache)) != MLA_OK) return st;
  if (batch == 0) return MLA_OK;
  if (h == nullptr || w_dkv == nullptr || (dims->d_rope > 0 && w_kr == nullptr) ||
      rms_weight == nullptr || positions == nullptr || cache->data == nullptr ||
      (cache->row_format == MLA_ROWS_FP8 && cache->scales == nullptr))
    return MLA_ERR_NULL;
  if (!aligned16(h) || !aligned16(w_dkv) || (dims->d_rope > 0 && !aligned16(w_kr)) ||
      !aligned16(cache->data))
    return MLA_ERR_ALIGN;
  const size_t need = mla::append_workspace_bytes(dims->dtype, batch, d_model, dims->d_latent,
                                                  dims->d_rope);
  if (workspace == nullptr || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return MLA_ERR_ALIGN;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != MLA_OK) return st;
  mla::CacheView view;
  view.data = static_cast<const uint8_t*>(cache->data);
  view.scales = cache->scales;
  view.fp8 = cache->row_format == MLA_ROWS_FP8 ? 1 : 0;
  view.seq_lens = cache->seq_lens;
  view.page_table = cache->page_table;
  view.page_size = cache->page_table ? cache->page_size : 0;
  view.max_len = cache->max_len;
  view.max_pages = cache->page_table ? cache->max_len / cache->page_size : 0;
  (void)hipGetLastError();
  const hipError_t e = mla::launch_cache_append(
      dims->dtype, batch, d_model, dims->d_latent, dims->d_rope, h, w_dkv, w_kr, rms_weight,
      rms_eps, rope->base, rope->yarn_scale, rope->yarn_alpha, rope->yarn_beta,
      static_cast<double>(rope->yarn_original_len), positions, view,
      const_cast<void*>(cache->data), workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

// ----------------------------------------------------------------------------
// Unabsorbed chunk form (explicit keys and values)
// ----------------------------------------------------------------------------

namespace {

// Shared checks of the two chunk-form calls: bf16 at the DeepSeek-V2 widths,
// a contiguous cache of native rows.
mla_status_t check_prefill(const mla_dims_t* dims, int32_t batch, const mla_cache_t* cache) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if ((st = check_cache(cache)) != MLA_OK) return st;
  if (batch < 0) return MLA_ERR_DIMS;
  if (dims->dtype != MLA_BF16 || cache->row_format != MLA_ROWS_NATIVE) return MLA_ERR_DTYPE;
  if (!mla::prefill_supported(1, dims->n_heads, dims->d_head, dims->d_latent, dims->d_rope) ||
      cache->page_table != nullptr)
    return MLA_ERR_DIMS;
  return MLA_OK;
}

mla::CacheView contiguous_view(const mla_cache_t* cache) {
  mla::CacheView view{};
  view.data = static_cast<const uint8_t*>(cache->data);
  view.seq_lens = cache->seq_lens;
  view.max_len = cache->max_len;
  return view;
}

}  // namespace

extern "C" {

mla_status_t mla_prefill_expand(const mla_dims_t* dims, int32_t batch, const mla_cache_t* cache,
                                const void* w_uk, const void* w_uv, void* k_c, void* v,
                                void* stream) {
  mla_status_t st = check_prefill(dims, batch, cache);
  if (st != MLA_OK || batch == 0) return st;
  if (cache->data == nullptr || cache->seq_lens == nullptr || w_uk == nullptr ||
      w_uv == nullptr || k_c == nullptr || v == nullptr)
    return MLA_ERR_NULL;
  if (!aligned16(cache->data) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(k_c) ||
      !aligned16(v))
    return MLA_ERR_ALIGN;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != MLA_OK) return st;
  (void)hipGetLastError();
  const hipError_t e = mla::launch_expand_kv(batch, dims->n_heads, contiguous_view(cache), w_uk,
                                             w_uv, k_c, v, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

mla_status_t mla_prefill_attn(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                              const void* q_c, const void* q_r, const mla_cache_t* cache,
                              const void* k_c, const void* v, float softmax_scale, void* out,
                              float* lse, void* stream) {
  mla_status_t st = check_prefill(dims, batch, cache);
  if (st != MLA_OK) return st;
  if (q_len < 1 || q_len > cache->max_len) return MLA_ERR_DIMS;
  if (batch == 0) return MLA_OK;
  if (q_c == nullptr || q_r == nullptr || cache->data == nullptr ||
      cache->seq_lens == nullptr || k_c == nullptr || v == nullptr || out == nullptr)
    return MLA_ERR_NULL;
  if (!aligned16(q_c) || !aligned16(q_r) || !aligned16(cache->data) || !aligned16(k_c) ||
      !aligned16(v) || !aligned16(out) || (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return MLA_ERR_ALIGN;
  DeviceInfo dev;
  if ((st = current_device(&dev)) != MLA_OK) return st;
  (void)hipGetLastError();
  const hipError_t e = mla::launch_prefill_attn(batch, q_len, dims->n_heads,
                                                contiguous_view(cache), q_c, q_r, k_c, v,
                                                softmax_scale, out, lse,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

}  // extern "C"
