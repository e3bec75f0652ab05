// Generic split-KV latent decode and the split combines.
//
// The generic decode serves fp32 storage and any (n_heads, d_latent, d_rope):
// one workgroup owns one (request, head, split) and walks the split in tiles
// of 256 tokens.  Scores are the full-row dot product
//   s_j = scale * q_cat . [c_j | k^R_j]
// (the absorbed content score plus the decoupled RoPE score, DeepSeek-V2
// read-through, 2kiu.com/news/6085339, sections 2.3-2.4), the softmax is kept
// online (running max and sum), and the weighted sum is taken over the latent
// part of the row only (section 2.3: the weighted sum happens in latent space).
//
// Partials are normalised by their own softmax sum and stored with their
// natural-log sum-exp; the combine merges splits s with weights
// exp(lse_s - max_s lse_s).
//
// Rows: n_rows = q_len * heads_per_token query rows per request, token-major;
// row i belongs to query token j = i / heads_per_token, which sees the
// request's first seq_len - (q_len - 1 - j) cached rows (the rows up to its
// own position).

#include "device_common.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxLatentPerThread = 8;  // d_latent <= 2048

// Number of splits that hold tokens of a request of length len.
__device__ __forceinline__ int used_splits(int len, int split_tokens) {
  return len > 0 ? (len + split_tokens - 1) / split_tokens : 0;
}

// Rows visible to query row i of a request holding `len` rows.
__device__ __forceinline__ int visible_rows(int len, int i, int heads_per_token, int q_len) {
  return len - (q_len - 1 - i / heads_per_token);
}

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// grid: x = split, y = query row, z = request.  Partials row-major:
// part_o[((b * S + s) * n_rows + i) * d_latent + c], part_lse[(b * S + s) * n_rows + i].
template <typename T>
__global__ __launch_bounds__(kThreads) void decode_generic_kernel(
    const T* __restrict__ q_cat, CacheView cache, int n_rows, int heads_per_token, int q_len,
    int d_latent, int d_rope, float scale, int split_tokens, int num_splits,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  extern __shared__ float sm[];
  const int row = d_latent + d_rope;
  float* q_s = sm;                 // [row]
  float* p_s = sm + row;           // [kThreads]
  float* red = p_s + kThreads;     // [4]
  const int s = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
  const int len = visible_rows(cache.seq_lens[b], i, heads_per_token, q_len);
  const int t0 = s * split_tokens;
  const int t1 = min(t0 + split_tokens, len);
  if (t0 >= t1) return;  // the combine never reads splits past the length

  const T* q = q_cat + (static_cast<size_t>(b) * n_rows + i) * row;
  for (int k = threadIdx.x; k < row; k += kThreads) q_s[k] = ld(q + k);
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  float o[kMaxLatentPerThread];
#pragma unroll
  for (int r = 0; r < kMaxLatentPerThread; ++r) o[r] = 0.f;
  // Low-bit rows: one E4M3 byte per element times the row's scale; the scale
  // multiplies the dot product, and the probability in the weighted sum.
  const bool fp8 = cache.fp8 != 0;
  const int row_bytes = row * (fp8 ? 1 : static_cast<int>(sizeof(T)));

  for (int tile = t0; tile < t1; tile += kThreads) {
    const int j = tile + threadIdx.x;
    float sj = -INFINITY, row_scale = 1.f;
    if (j < t1) {
      float dot = 0.f;
      if (fp8) {
        const size_t idx = cache_row_index(cache, b, j);
        const uint8_t* rp = cache.data + idx * row_bytes;
        for (int k = 0; k < row; ++k) dot = fmaf(q_s[k], ld_e4m3(rp + k), dot);
        row_scale = cache.scales[idx];
        dot *= row_scale;
      } else {
        const T* rp = reinterpret_cast<const T*>(cache_row(cache, b, j, row_bytes));
        for (int k = 0; k < row; ++k) dot = fmaf(q_s[k], ld(rp + k), dot);
      }
      sj = dot * scale;
    }
    const float tmax = block_max(sj, red);
    const float m_new = fmaxf(m, tmax);
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
    const float pj = (j < t1) ? expf(sj - m_new) : 0.f;
    p_s[threadIdx.x] = pj * row_scale;
    const float psum = block_sum(pj, red);  // its barriers also publish p_s
    l = l * alpha + psum;
    m = m_new;
    const int nt = min(kThreads, t1 - tile);
#pragma unroll
    for (int r = 0; r < kMaxLatentPerThread; ++r) {
      const int c = threadIdx.x + r * kThreads;
      if (c < d_latent) {
        float acc = o[r] * alpha;
        if (fp8) {
          for (int jj = 0; jj < nt; ++jj)
            acc = fmaf(p_s[jj], ld_e4m3(cache_row(cache, b, tile + jj, row_bytes) + c), acc);
        } else {
          for (int jj = 0; jj < nt; ++jj) {
            const T* rp = reinterpret_cast<const T*>(cache_row(cache, b, tile + jj, row_bytes));
            acc = fmaf(p_s[jj], ld(rp + c), acc);
          }
        }
        o[r] = acc;
      }
    }
    __syncthreads();  // p_s is rewritten by the next tile
  }

  const float inv = 1.f / l;
  const size_t base = (static_cast<size_t>(b) * num_splits + s) * n_rows + i;
#pragma unroll
  for (int r = 0; r < kMaxLatentPerThread; ++r) {
    const int c = threadIdx.x + r * kThreads;
    if (c < d_latent) part_o[base * d_latent + c] = o[r] * inv;
  }
  if (threadIdx.x == 0) part_lse[base] = m + logf(l);
}


// Combine for row-major partials.  grid: x = query row, y = request.
template <typename T>
__global__ __launch_bounds__(kThreads) void combine_rowmajor_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse,
    const int32_t* __restrict__ seq_lens, int n_rows, int heads_per_token, int q_len,
    int d_latent, int split_tokens, int num_splits, T* __restrict__ out_lat,
    float* __restrict__ lse_out) {
  const int i = blockIdx.x, b = blockIdx.y;
  const int ns =
      used_splits(visible_rows(seq_lens[b], i, heads_per_token, q_len), split_tokens);
  const int n_heads = n_rows;  // strides below are per query row
  const size_t obase = (static_cast<size_t>(b) * n_heads + i) * d_latent;
  const size_t pbase = static_cast<size_t>(b) * num_splits * n_heads + i;
  float L = -INFINITY;
  for (int s = 0; s < ns; ++s) L = fmaxf(L, part_lse[pbase + static_cast<size_t>(s) * n_heads]);
  float W = 0.f;
  for (int s = 0; s < ns; ++s) W += expf(part_lse[pbase + static_cast<size_t>(s) * n_heads] - L);
  const float invW = ns > 0 ? 1.f / W : 0.f;
  for (int c = threadIdx.x; c < d_latent; c += kThreads) {
    float acc = 0.f;
    for (int s = 0; s < ns; ++s) {
      const size_t ps = pbase + static_cast<size_t>(s) * n_heads;
      acc = fmaf(expf(part_lse[ps] - L), part_o[ps * d_latent + c], acc);
    }
    st(out_lat + obase + c, acc * invW);
  }
  if (lse_out != nullptr && threadIdx.x == 0)
    lse_out[static_cast<size_t>(b) * n_heads + i] = ns > 0 ? L + logf(W) : -INFINITY;
}

}  // namespace

hipError_t launch_partials_generic(const DecodeArgs& a) {
  if (a.batch == 0) return hipSuccess;
  const int row = a.d_latent + a.d_rope;
  const int n_rows = a.q_len * a.n_heads;
  const size_t lds = sizeof(float) * (row + kThreads + 4);
  const dim3 grid(a.num_splits, n_rows, a.batch);
  if (a.dtype == 0) {
    decode_generic_kernel<float><<<grid, kThreads, lds, a.stream>>>(
        static_cast<const float*>(a.q_cat), a.cache, n_rows, a.n_heads, a.q_len, a.d_latent,
        a.d_rope, a.softmax_scale, a.split_tokens, a.num_splits, static_cast<float*>(a.part_o),
        a.part_lse);
  } else {
    decode_generic_kernel<__bf16><<<grid, kThreads, lds, a.stream>>>(
        static_cast<const __bf16*>(a.q_cat), a.cache, n_rows, a.n_heads, a.q_len, a.d_latent,
        a.d_rope, a.softmax_scale, a.split_tokens, a.num_splits, static_cast<float*>(a.part_o),
        a.part_lse);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeArgs& a, bool mfma_partials) {
  if (a.batch == 0) return hipSuccess;
  if (mfma_partials) return launch_combine_rows(a, nullptr, nullptr, 0);
  const int n_rows = a.q_len * a.n_heads;
  const dim3 cgrid(n_rows, a.batch);
  if (a.dtype == 0) {
    combine_rowmajor_kernel<float><<<cgrid, kThreads, 0, a.stream>>>(
        static_cast<const float*>(a.part_o), a.part_lse, a.cache.seq_lens, n_rows, a.n_heads,
        a.q_len, a.d_latent, a.split_tokens, a.num_splits, static_cast<float*>(a.out_lat),
        a.lse);
  } else {
    combine_rowmajor_kernel<__bf16><<<cgrid, kThreads, 0, a.stream>>>(
        static_cast<const float*>(a.part_o), a.part_lse, a.cache.seq_lens, n_rows, a.n_heads,
        a.q_len, a.d_latent, a.split_tokens, a.num_splits, static_cast<__bf16*>(a.out_lat),
        a.lse);
  }
  return hipGetLastError();
}

}  // namespace mla
