// K3 (split-KV combine) for the bf16 MFMA partials, alone or fused with K4
// (the W^UV output projection).
//
// Combine: split s of request b holds the latent sum U_s = sum_j 2^(x_j - m_s)
// row_j over its tokens (x_j the scores scaled to log2 units, m_s a reference
// value of the split, U_s not divided by its softmax sum), its base-2
// log-sum-exp lse_s = log2 sum_j 2^(x_j) and m_s.  The merged latent output is
//   o_lat = sum_s 2^(m_s - L) U_s / sum_s 2^(lse_s - L),  L = max_s lse_s
// (2^(m_s - L) U_s = 2^(lse_s - L) times the split's normalised sum), and its
// natural-log sum-exp is ln 2 * (L + log2 sum_s 2^(lse_s - L)) (computed in one
// pass with a running max, rescaling the sums whenever it grows).  This is the softmax of
// the concatenated scores regrouped by partition, so it equals the single-pass
// latent weighted sum of the DeepSeek-V2 read-through (2kiu.com/news/6085339),
// section 2.3.
// Output projection, applied after the latent-space sum (same section):
//   out[b, i, h] = sum_c o_lat[b, i, c] W^UV[i, c, h].
//
// One workgroup = one head i and R = 8 / P requests (8 waves, P waves per
// request).  The MFMA partials are row-major bf16, partition-major,
// part_o[((off_b + s) * n_rows + i) * 512 + c], so every (request, split)
// contributes one contiguous 1 KiB row; (lse_s, m_s) are an fp32 pair per
// (partition, head).  off_b is b * S in a uniform plan; in a length-balanced
// one the decode kernel leaves the partition length and every off_b in a
// table behind the statistics.  Wave p of a request merges splits p, p + P,
// p + 2P, ..., 8 latents per lane, with the loads of up to kBatch splits
// (rows and statistics) in flight at once; with P > 1 the waves of a request
// then merge their results through LDS.  P grows with the split count, so
// that a request with many splits (few long requests) is not merged by one
// wave in many dependent memory round trips.  In the fused form the workgroup first starts W^UV[i]
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
constexpr int kWaves = kThreads / 64;
constexpr int kRowsPerGroup = 8;   // o_lat rows of the fused product (requests, zero-padded)
constexpr int kSegs = 64;          // lanes per wave, 8 latents each
constexpr int kBatch = 16;         // most splits a wave has in flight at once
constexpr int kMaxHead = 128;      // d_head handled by the fused kernel
constexpr int kWBytes = kLat * kMaxHead * 2;
constexpr int kOStride = kLat + 8;  // o_lat rows in LDS, padded against bank conflicts
static_assert(kSegs * 8 == kLat, "");

__device__ __forceinline__ int used_splits(int len, int split_tokens) {
  return len > 0 ? (len + split_tokens - 1) / split_tokens : 0;
}


// kB: splits per batch of loads (at most kBatch), sized on the host to the
// splits a wave merges.
template <bool kOut, int kB>
__global__ __launch_bounds__(kThreads) void combine_rows_kernel(
    const uint16_t* __restrict__ part_o, const float2* __restrict__ part_ml,
    const int32_t* __restrict__ seq_lens, int batch, int n_rows, int heads_per_token, int q_len,
    int split_tokens, int num_splits, const int32_t* __restrict__ part_table, int partitions,
    int p_log2,
    __bf16* __restrict__ out_lat, float* __restrict__ lse_out,
    const __bf16* __restrict__ w_uv, __bf16* __restrict__ out, int d_head) {
  __shared__ __attribute__((aligned(16))) uint8_t w_s[kOut ? kWBytes : 16];
  __shared__ __attribute__((aligned(16))) __bf16 o_s[kOut ? kRowsPerGroup * kOStride : 8];
  // Per-wave partial sums of the cross-wave merge, later (fused form) the
  // reduction buffer of the two contraction halves.
  __shared__ __attribute__((aligned(16))) float red[kWaves * kLat];
  __shared__ float2 stat_s[kWaves];
  static_assert(4 * 16 * 64 <= kWaves * kLat, "");

  // Row i of a request: query token i / heads_per_token, head i % heads_per_token
  // (one token per request unless several are verified at once).
  // Workgroups (i, g) and (i, g') are n_rows apart in launch order, so with
  // n_rows % 8 == 0 they land on the same XCD and share W^UV[i] through its
  // L2.
  const int i = blockIdx.x;
  const int P = 1 << p_log2;                 // waves per request
  const int R = kWaves >> p_log2;            // requests per workgroup
  const int b0 = blockIdx.y * R;
  // The wave index is made uniform so that the per-request values (length,
  // partition table) come through scalar loads: those are waited for apart
  // from the vector loads, which queue behind the W^UV stream issued first.
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // W^UV rows of 128 elements (256 bytes, the width of the 64 banks) are
  // stored with their 16-byte chunk c in slot c ^ 4 (row % 4): the
  // transposing reads of the product below address four consecutive rows at
  // once, which would otherwise fall in the same banks.
  const int w_swz = d_head == kMaxHead ? 4 : 0;
  if constexpr (kOut) {
    // Start W^UV[i] streaming into LDS, 1 KiB (four 256-byte rows at d_head
    // 128) per wave instruction.
    const uint8_t* src = reinterpret_cast<const uint8_t*>(w_uv) +
                         static_cast<size_t>(i % heads_per_token) * kLat * d_head * 2;
    const unsigned base = static_cast<unsigned>(
        reinterpret_cast<uintptr_t>((MLA_LDS uint8_t*)w_s));
    const int chunks = kLat * d_head * 2 / 1024;
    const int lane_src = (lane & ~15) | ((lane & 15) ^ (w_swz * ((lane >> 4) & 3)));
    for (int j = wave; j < chunks; j += kThreads / 64)
      load_to_lds16(src + j * 1024 + lane_src * 16, base + j * 1024);
  }

  // Merge: this wave's request r and split subset p, 8 latents per lane.
  const int r = wave >> p_log2, p = wave & (P - 1), seg = lane;
  const int b = b0 + r;
  const bool live = b < batch;
  // The rows this query token sees: up to its own position.
  const int len = live ? seq_lens[b] - (q_len - 1 - i / heads_per_token) : 0;
  // Partition length and the request's first partition.  A uniform plan
  // knows both on the host; a length-balanced one reads them from the
  // table, and then also its split count (one memory round trip in front of
  // the partial loads, which therefore cover the used splits only).
  int c = split_tokens, nk;
  size_t pbase;
  if (part_table != nullptr) {
    // (clamped, so that a table the decode kernel did not write cannot
    // send the loads outside the workspace)
    c = max(part_table[0], 32);
    const int first = min(max(part_table[1 + (live ? b : 0)], 0), partitions);
    pbase = static_cast<size_t>(first);
    const int used = min(used_splits(len, c), partitions - first);
    nk = max(0, (used - p + P - 1) >> p_log2);
  } else {
    pbase = static_cast<size_t>(live ? b : 0) * num_splits;
    nk = (num_splits - p + P - 1) >> p_log2;
  }
  const size_t lbase = pbase * n_rows + i;  // partition pbase's row i
  // This wave's splits are p + k * P, k < nk.  Single pass with a running max
  // over batches of kB of them.  The loads of a batch (rows and statistics)
  // are issued together with the length load, without waiting for it and
  // without branches (a branch around a load makes the compiler wait for it
  // before the branches join): every split's row lies in the workspace,
  // indexes past the wave's last split are clamped to it, and the splits past
  // the request's length (never written: any bits) are dropped with selects
  // afterwards.  A wave's merge of its splits costs ceil(nk / kB) memory round
  // trips.
  float L = -INFINITY, W = 0.f;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  const uint16_t* row = part_o + lbase * kLat + seg * 8;
  const size_t split_stride = static_cast<size_t>(n_rows) * kLat;
  int ns = 0;
  // One batch: returns false once the batch starts past the used splits.
  auto merge_batch = [&](int k0) {
    bf16x8_t v[kB];
    float x[kB], y[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const size_t sidx = static_cast<size_t>(p + (min(k0 + j, nk - 1) << p_log2));
      v[j] = *reinterpret_cast<const bf16x8_t*>(row + sidx * split_stride);
      const float2 ml = part_ml[lbase + sidx * n_rows];
      x[j] = ml.x;
      y[j] = ml.y;
    }
    // The length is used only here, behind the loads (laundered so that the
    // compiler does not hoist its wait in front of them).
    int len_k = len;
    asm volatile("" : "+v"(len_k));
    ns = used_splits(len_k, c);
    if (p + (k0 << p_log2) >= ns) return false;
    bool use[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      use[j] = k0 + j < nk && p + ((k0 + j) << p_log2) < ns;
      x[j] = use[j] ? x[j] : -INFINITY;
    }
    float Ln = L;
#pragma unroll
    for (int j = 0; j < kB; ++j) Ln = fmaxf(Ln, x[j]);
    const float alpha = __builtin_amdgcn_exp2f(L - Ln);  // 0 on the first batch (L = -inf)
    W *= alpha;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] *= alpha;
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      if (use[j]) {
        W += __builtin_amdgcn_exp2f(x[j] - Ln);
        const float w = __builtin_amdgcn_exp2f(y[j] - Ln);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, static_cast<float>(v[j][e]), acc[e]);
      }
    }
    L = Ln;
    return true;
  };
  // The first batch is peeled off the loop: at a loop header the compiler
  // waits for every outstanding load, the length load included, which would
  // add a memory round trip in front of the row loads.
  if (nk > 0 && merge_batch(0))
    for (int k0 = kB; k0 < nk; k0 += kB)
      if (!merge_batch(k0)) break;
  if (P > 1) {
    // The P waves of a request publish (L, W) and their sums; the first of
    // them rescales all of them to the common max and adds them up.  A wave
    // whose splits were all unused has L = -inf and weight 0.
    *reinterpret_cast<f32x4_t*>(red + wave * kLat + seg * 8) = {acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4_t*>(red + wave * kLat + seg * 8 + 4) = {acc[4], acc[5], acc[6], acc[7]};
    if (seg == 0) stat_s[wave] = make_float2(L, W);
    __syncthreads();
    if (p == 0) {
      float Lm = -INFINITY;
      for (int q = 0; q < P; ++q) Lm = fmaxf(Lm, stat_s[wave + q].x);
      W = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = 0.f;
      for (int q = 0; q < P; ++q) {
        const float2 st = stat_s[wave + q];
        const float w = st.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.x - Lm);
        W += w * st.y;
        const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(red + (wave + q) * kLat + seg * 8);
        const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(red + (wave + q) * kLat + seg * 8 + 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[k] = fmaf(w, a0[k], acc[k]);
          acc[k + 4] = fmaf(w, a1[k], acc[k + 4]);
        }
      }
      L = Lm;
    }
    // red is reused by the fused product below.
    __syncthreads();
  }
  const float invW = ns > 0 ? 1.f / W : 0.f;
  bf16x8_t ob;
#pragma unroll
  for (int e = 0; e < 8; ++e) ob[e] = static_cast<__bf16>(acc[e] * invW);
  if (live && p == 0) {
    *reinterpret_cast<bf16x8_t*>(out_lat + (static_cast<size_t>(b) * n_rows + i) * kLat +
                                 seg * 8) = ob;
    if (lse_out != nullptr && seg == 0)
      lse_out[static_cast<size_t>(b) * n_rows + i] =
          ns > 0 ? (L + __log2f(W)) * kLn2 : -INFINITY;
  }
  if constexpr (kOut) {
    // Fused W^UV product.  o_lat rows (zero past the batch and past the
    // workgroup's R requests) go to LDS; the weight stream must have landed
    // before the barrier publishes w_s.
    if (p == 0) *reinterpret_cast<bf16x8_t*>(o_s + r * kOStride + seg * 8) = ob;
    if (wave >= R) {
      bf16x8_t z;
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = static_cast<__bf16>(0.f);
      *reinterpret_cast<bf16x8_t*>(o_s + wave * kOStride + seg * 8) = z;
    }
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
          // (row k0 + tr_k and row k0 + tr_k + 4 have the same swizzle)
          const int col = ((((nb * 32 + tr_n) >> 3) ^ (w_swz * (tr_k & 3))) << 3) | (tr_n & 7);
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (MLA_LDS i16x4_t*)(wl + (k0 + tr_k) * d_head + col));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (MLA_LDS i16x4_t*)(wl + (k0 + tr_k + 4) * d_head + col));
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
          if (rr < R && b0 + rr < batch)
            out[(static_cast<size_t>(b0 + rr) * n_rows + i) * d_head + nb * 32 + l32] =
                static_cast<__bf16>(y);
        }
      }
      __syncthreads();
    }
  }
}

template <bool kOut, int kB>
void launch_rows(const DecodeArgs& a, int p_log2, const dim3& grid, const void* w_uv, void* out,
                 int d_head) {
  combine_rows_kernel<kOut, kB><<<grid, kThreads, 0, a.stream>>>(
      static_cast<const uint16_t*>(a.part_o), reinterpret_cast<const float2*>(a.part_lse),
      a.cache.seq_lens, a.batch, a.q_len * a.n_heads, a.n_heads, a.q_len, a.split_tokens,
      a.num_splits, a.split_tokens == 0 ? a.part_table : nullptr, a.partitions, p_log2,
      static_cast<__bf16*>(a.out_lat), a.lse, static_cast<const __bf16*>(w_uv),
      static_cast<__bf16*>(out), d_head);
}

// Splits per request the launch shape is sized for: all of them in a
// uniform plan; in a length-balanced one the mean over the requests (a
// request with more takes more batches of loads).
int sizing_splits(const DecodeArgs& a) {
  return a.split_tokens == 0 ? (a.partitions + a.batch - 1) / a.batch : a.num_splits;
}

template <bool kOut>
void launch_rows_sized(const DecodeArgs& a, int p_log2, const dim3& grid, const void* w_uv,
                       void* out, int d_head) {
  const int nk = (sizing_splits(a) + (1 << p_log2) - 1) >> p_log2;  // splits of wave 0
  // (A mean of two splits per wave takes batches of four: in a length-balanced
  // plan the longer requests hold more than the mean, and a second batch is a
  // second memory round trip.)
  if (nk <= 1)
    launch_rows<kOut, 2>(a, p_log2, grid, w_uv, out, d_head);
  else if (nk <= 4)
    launch_rows<kOut, 4>(a, p_log2, grid, w_uv, out, d_head);
  else if (nk <= 8)
    launch_rows<kOut, 8>(a, p_log2, grid, w_uv, out, d_head);
  else
    launch_rows<kOut, kBatch>(a, p_log2, grid, w_uv, out, d_head);
}

}  // namespace

bool combine_out_fusable(int d_latent, int d_head) {
  return d_latent == kLat && d_head % 32 == 0 && d_head <= kMaxHead;
}

hipError_t launch_combine_rows(const DecodeArgs& a, const void* w_uv, void* out, int d_head) {
  if (a.batch == 0) return hipSuccess;
  // Waves per request: the fewest (a power of two up to 8) that leave every
  // wave at most kBatch splits, so each wave's merge is one memory round
  // trip.  The fused form stops earlier, at no more than four workgroups per
  // head (counting every query token's rows): each of them streams its own
  // copy of W^UV[i] into LDS.
  int p_log2 = 0;
  const int splits = sizing_splits(a);
  while (p_log2 < 3 && (splits + (1 << p_log2) - 1) >> p_log2 > kBatch) ++p_log2;
  if (w_uv != nullptr)
    while (p_log2 > 0 &&
           a.q_len * ((a.batch + (kWaves >> p_log2) - 1) / (kWaves >> p_log2)) > 4)
      --p_log2;
  const int rows = kWaves >> p_log2;
  const dim3 grid(a.q_len * a.n_heads, (a.batch + rows - 1) / rows);
  if (w_uv != nullptr)
    launch_rows_sized<true>(a, p_log2, grid, w_uv, out, d_head);
  else
    launch_rows_sized<false>(a, p_log2, grid, nullptr, nullptr, 0);
  return hipGetLastError();
}

}  // namespace mla
