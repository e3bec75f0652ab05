// K3 (split-KV combine) for the bf16 MFMA partials, alone or fused with K4
// (the W^UV output projection).
//
// Combine: the splits s of request b each hold a latent partial O_s
// normalised by its own softmax sum and its log-sum-exp lse_s; the merged
// latent output is
//   o_lat = sum_s exp(lse_s - L) O_s / sum_s exp(lse_s - L),  L = max_s lse_s,
// and its log-sum-exp is L + ln sum_s exp(lse_s - L) (computed in one pass
// with a running max, rescaling the sums whenever it grows).  This is the softmax of
// the concatenated scores regrouped by partition, so it equals the single-pass
// latent weighted sum of the DeepSeek-V2 read-through (2kiu.com/news/6085339),
// section 2.3.
// Output projection, applied after the latent-space sum (same section):
//   out[b, i, h] = sum_c o_lat[b, i, c] W^UV[i, c, h].
//
// One workgroup = one head i and up to 8 requests (8 waves).  The MFMA
// partials are row-major bf16, part_o[((b * S + s) * n_heads + i) * 512 + c],
// so every (request, split) contributes one contiguous 1 KiB row.  Wave r
// merges request r, 8 latents per lane, with the loads of kBatch splits (rows
// and log-sum-exps) in flight at once.  In the fused form the workgroup first starts W^UV[i]
// (d_latent x d_head bf16, 128 KiB for DeepSeek-V2) streaming into LDS with
// direct-to-LDS loads, merges the partials while it lands, writes o_lat, and
// multiplies the bf16 o_lat rows by W^UV[i] with v_mfma_f32_32x32x16_bf16
// (M = requests, padded to 32; 32 output columns per pair of waves, which
// split the contraction).  o is rounded
// from the same bf16 o_lat that o_lat holds, as the unfused path computes it.

#include "device_common.h"

namespace mla {
namespace {

constexpr int kLat = 512;          // d_latent of the MFMA path
constexpr int kThreads = 512;      // 8 waves
constexpr int kRowsPerGroup = 8;   // requests per workgroup
constexpr int kSegs = kThreads / kRowsPerGroup;  // 64 threads per request, 8 latents each
constexpr int kBatch = 16;         // splits whose loads are in flight together
constexpr int kMaxHead = 128;      // d_head handled by the fused kernel
constexpr int kWBytes = kLat * kMaxHead * 2;
constexpr int kOStride = kLat + 8;  // o_lat rows in LDS, padded against bank conflicts
static_assert(kSegs * 8 == kLat, "");

__device__ __forceinline__ int used_splits(int len, int split_tokens) {
  return len > 0 ? (len + split_tokens - 1) / split_tokens : 0;
}

// 16-byte direct-to-LDS load (see the decode kernel): lands at lds_base +
// 16 * lane.  Issued as inline asm; the kernel waits for it with an explicit
// s_waitcnt vmcnt(0) before the barrier that publishes the LDS contents.
__device__ __forceinline__ void load_to_lds16(const void* src, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}

template <bool kOut>
__global__ __launch_bounds__(kThreads) void combine_rows_kernel(
    const uint16_t* __restrict__ part_o, const float* __restrict__ part_lse,
    const int32_t* __restrict__ seq_lens, int batch, int n_heads, int split_tokens,
    int num_splits, __bf16* __restrict__ out_lat, float* __restrict__ lse_out,
    const __bf16* __restrict__ w_uv, __bf16* __restrict__ out, int d_head) {
  __shared__ __attribute__((aligned(16))) uint8_t w_s[kOut ? kWBytes : 16];
  __shared__ __attribute__((aligned(16))) __bf16 o_s[kOut ? kRowsPerGroup * kOStride : 8];
  __shared__ float red[kOut ? 4 * 16 * 64 : 1];

  // Workgroups (i, g) and (i, g') are n_heads apart in launch order, so with
  // n_heads % 8 == 0 they land on the same XCD and share W^UV[i] through its
  // L2.
  const int i = blockIdx.x;
  const int b0 = blockIdx.y * kRowsPerGroup;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  if constexpr (kOut) {
    // Start W^UV[i] streaming into LDS: a linear copy of its d_latent x d_head
    // bf16 elements, 1 KiB per wave instruction.
    const uint8_t* src = reinterpret_cast<const uint8_t*>(w_uv) +
                         static_cast<size_t>(i) * kLat * d_head * 2 + lane * 16;
    const unsigned base = static_cast<unsigned>(
        reinterpret_cast<uintptr_t>((MLA_LDS uint8_t*)w_s));
    const int chunks = kLat * d_head * 2 / 1024;
    for (int j = wave; j < chunks; j += kThreads / 64)
      load_to_lds16(src + j * 1024, base + j * 1024);
  }

  // Merge: this thread's request (a whole wave per request) and 8 latents.
  const int r = tid / kSegs, seg = tid % kSegs;
  const int b = b0 + r;
  const bool live = b < batch;
  const int len = live ? seq_lens[b] : 0;
  const size_t lbase = static_cast<size_t>(live ? b : 0) * num_splits * n_heads + i;
  // Single pass with a running max over batches of kBatch splits.  The loads
  // of a batch (rows and log-sum-exps) are issued together with the length
  // load, without waiting for it: every split's row lies in the workspace,
  // and the splits past the request's length (never written: any bits) are
  // dropped with selects afterwards.  A merge of S splits costs ceil(S /
  // kBatch) memory round trips.
  float L = -INFINITY, W = 0.f;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  const uint16_t* row = part_o + lbase * kLat + seg * 8;
  const size_t split_stride = static_cast<size_t>(n_heads) * kLat;
  int ns = 0;
  for (int s0 = 0; s0 < num_splits; s0 += kBatch) {
    bf16x8_t v[kBatch];
    float x[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int s = min(s0 + j, num_splits - 1);
      v[j] = *reinterpret_cast<const bf16x8_t*>(row + static_cast<size_t>(s) * split_stride);
      x[j] = part_lse[lbase + static_cast<size_t>(s) * n_heads];
    }
    ns = used_splits(len, split_tokens);
    if (s0 >= ns) break;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) x[j] = s0 + j < ns ? x[j] : -INFINITY;
    float Ln = L;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) Ln = fmaxf(Ln, x[j]);
    const float alpha = expf(L - Ln);  // 0 on the first batch (L = -inf)
    W *= alpha;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] *= alpha;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (s0 + j < ns) {
        const float w = expf(x[j] - Ln);
        W += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, static_cast<float>(v[j][e]), acc[e]);
      }
    }
    L = Ln;
  }
  const float invW = ns > 0 ? 1.f / W : 0.f;
  bf16x8_t ob;
#pragma unroll
  for (int e = 0; e < 8; ++e) ob[e] = static_cast<__bf16>(acc[e] * invW);
  if (live) {
    *reinterpret_cast<bf16x8_t*>(out_lat + (static_cast<size_t>(b) * n_heads + i) * kLat +
                                 seg * 8) = ob;
    if (lse_out != nullptr && seg == 0)
      lse_out[static_cast<size_t>(b) * n_heads + i] = ns > 0 ? L + logf(W) : -INFINITY;
  }
  if constexpr (kOut) {
    // Fused W^UV product.  o_lat rows (zero past the batch) go to LDS; the
    // weight stream must have landed before the barrier publishes w_s.
    *reinterpret_cast<bf16x8_t*>(o_s + r * kOStride + seg * 8) = ob;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // Waves 0-3 and 4-7 take the two halves of the K = 512 contraction for
    // output block nb = wave % 4 (32 columns); the high half's sums reach the
    // low half through LDS.
    const int half = lane >> 5, l32 = lane & 31;
    const int kh = wave >> 2, nb0 = wave & 3;
    // Transposing-read coordinates of the weight (B) operand: within a 16-lane
    // group G, lane (G, q) addresses row k0 + (G/2)*8 + q/4 (+4 for the high
    // half) at column 16*(G%2) + 4*(q%4) of the 32-column block.
    const int G = lane >> 4, q16 = lane & 15;
    const int tr_k = ((G >> 1) << 3) + (q16 >> 2);
    const int tr_n = ((G & 1) << 4) + ((q16 & 3) << 2);
    const __bf16* wl = reinterpret_cast<const __bf16*>(w_s);
    // Every wave runs the same number of iterations (the barriers inside
    // must be reached by all of them); waves past the last block idle.
    const int n_iters = (d_head / 32 + 3) / 4;
    for (int it = 0; it < n_iters; ++it) {
      const int nb = nb0 + it * 4;
      const bool act = nb < d_head / 32;
      f32x16_t acc2;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc2[e] = 0.f;
      if (act) {
#pragma unroll 8
        for (int ks = 0; ks < kLat / 32; ++ks) {
          const int k0 = kh * (kLat / 2) + ks * 16;
          // A operand: o_lat row l32 (rows past the group are zero), K slots
          // k0 + half*8 .. +7.
          bf16x8_t a;
          if (l32 < kRowsPerGroup) {
            a = *reinterpret_cast<const bf16x8_t*>(o_s + l32 * kOStride + k0 + half * 8);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = static_cast<__bf16>(0.f);
          }
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (MLA_LDS i16x4_t*)(wl + (k0 + tr_k) * d_head + nb * 32 + tr_n));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (MLA_LDS i16x4_t*)(wl + (k0 + tr_k + 4) * d_head + nb * 32 + tr_n));
          const bf16x8_t bop = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, acc2, 0, 0, 0);
        }
      }
      // Only accumulator rows 0..7 hold real requests: register e < 4 of lane
      // half h is row h*4 + e.
      if (act && kh == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) red[(nb0 * 4 + e) * 64 + lane] = acc2[e];
      }
      __syncthreads();
      if (act && kh == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = half * 4 + e;
          const float y = acc2[e] + red[(nb0 * 4 + e) * 64 + lane];
          if (b0 + rr < batch)
            out[(static_cast<size_t>(b0 + rr) * n_heads + i) * d_head + nb * 32 + l32] =
                static_cast<__bf16>(y);
        }
      }
      __syncthreads();
    }
  }
}

}  // namespace

bool combine_out_fusable(int d_latent, int d_head) {
  return d_latent == kLat && d_head % 32 == 0 && d_head <= kMaxHead;
}

hipError_t launch_combine_rows(const DecodeArgs& a, const void* w_uv, void* out, int d_head) {
  if (a.batch == 0) return hipSuccess;
  const dim3 grid(a.n_heads, (a.batch + kRowsPerGroup - 1) / kRowsPerGroup);
  if (w_uv != nullptr) {
    combine_rows_kernel<true><<<grid, kThreads, 0, a.stream>>>(
        static_cast<const uint16_t*>(a.part_o), a.part_lse, a.cache.seq_lens, a.batch,
        a.n_heads, a.split_tokens, a.num_splits, static_cast<__bf16*>(a.out_lat), a.lse,
        static_cast<const __bf16*>(w_uv), static_cast<__bf16*>(out), d_head);
  } else {
    combine_rows_kernel<false><<<grid, kThreads, 0, a.stream>>>(
        static_cast<const uint16_t*>(a.part_o), a.part_lse, a.cache.seq_lens, a.batch,
        a.n_heads, a.split_tokens, a.num_splits, static_cast<__bf16*>(a.out_lat), a.lse,
        nullptr, nullptr, 0);
  }
  return hipGetLastError();
}

}  // namespace mla
