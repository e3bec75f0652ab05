// K1 (query absorption) and K4 (W^UV output projection): per-head batched
// products that stream one weight matrix per head.
//
// Absorption: q_lat,i = W^UK_i^T q^C_i (DeepSeek-V2 read-through,
// 2kiu.com/news/6085339, section 2.3; DeepSeek-V3 read-through,
// 2kiu.com/news/6340724, section 2.3).  Output: o_i = W^UV_i o_lat,i applied
// after the latent-space sum (V2 read-through section 2.3).
//
// Both are HBM-bound at decode batch sizes: every weight element is read once
// per call and used for `batch` multiply-adds.  One workgroup owns one head
// and a 256-wide slice of output columns; the batch rows it serves are staged
// in LDS as fp32 and each thread keeps kRows accumulators, so a weight element
// loaded once feeds kRows FMAs.

#include "device_common.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 8;  // batch rows per workgroup

// q_cat[b, i, c] = sum_h q_c[b, i, h] w_uk[i, h, c]   (c < d_latent)
// q_cat[b, i, d_latent + r] = q_r[b, i, r]
// grid: x = column tiles over d_latent + d_rope, y = head, z = batch chunks
template <typename T>
__global__ __launch_bounds__(kThreads) void absorb_q_kernel(
    const T* __restrict__ q_c, const T* __restrict__ q_r, const T* __restrict__ w_uk,
    T* __restrict__ q_cat, int batch, int n_heads, int d_head, int d_rope, int d_latent) {
  extern __shared__ float q_s[];  // [kRows][d_head]
  const int i = blockIdx.y;
  const int b0 = blockIdx.z * kRows;
  const int nb = min(kRows, batch - b0);
  const int row = d_latent + d_rope;
  const int col = blockIdx.x * kThreads + threadIdx.x;

  for (int e = threadIdx.x; e < kRows * d_head; e += kThreads) {
    const int bb = e / d_head, h = e - bb * d_head;
    q_s[e] = bb < nb ? ld(q_c + (static_cast<size_t>(b0 + bb) * n_heads + i) * d_head + h) : 0.f;
  }
  __syncthreads();
  if (col >= row) return;

  if (col >= d_latent) {  // the RoPE part of the query is copied unchanged
    for (int bb = 0; bb < nb; ++bb) {
      const size_t bi = static_cast<size_t>(b0 + bb) * n_heads + i;
      st(q_cat + bi * row + col, ld(q_r + bi * d_rope + (col - d_latent)));
    }
    return;
  }

  float acc[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) acc[r] = 0.f;
  const T* w = w_uk + static_cast<size_t>(i) * d_head * d_latent + col;
  for (int h = 0; h < d_head; ++h) {
    const float wv = ld(w + static_cast<size_t>(h) * d_latent);
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[r] = fmaf(q_s[r * d_head + h], wv, acc[r]);
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    if (r < nb) st(q_cat + (static_cast<size_t>(b0 + r) * n_heads + i) * row + col, acc[r]);
  }
}

// out[b, i, h] = sum_c out_lat[b, i, c] w_uv[i, c, h]
// grid: x = column tiles over d_head, y = head, z = batch chunks
template <typename T>
__global__ __launch_bounds__(kThreads) void out_uv_kernel(
    const T* __restrict__ out_lat, const T* __restrict__ w_uv, T* __restrict__ out,
    int batch, int n_heads, int d_head, int d_latent) {
  extern __shared__ float o_s[];  // [kRows][d_latent]
  const int i = blockIdx.y;
  const int b0 = blockIdx.z * kRows;
  const int nb = min(kRows, batch - b0);
  const int col = blockIdx.x * kThreads + threadIdx.x;

  for (int e = threadIdx.x; e < kRows * d_latent; e += kThreads) {
    const int bb = e / d_latent, c = e - bb * d_latent;
    o_s[e] = bb < nb ? ld(out_lat + (static_cast<size_t>(b0 + bb) * n_heads + i) * d_latent + c)
                     : 0.f;
  }
  __syncthreads();
  if (col >= d_head) return;

  float acc[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) acc[r] = 0.f;
  const T* w = w_uv + static_cast<size_t>(i) * d_latent * d_head + col;
  for (int c = 0; c < d_latent; ++c) {
    const float wv = ld(w + static_cast<size_t>(c) * d_head);
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[r] = fmaf(o_s[r * d_latent + c], wv, acc[r]);
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    if (r < nb) st(out + (static_cast<size_t>(b0 + r) * n_heads + i) * d_head + col, acc[r]);
  }
}

}  // namespace

hipError_t launch_absorb_q(int dtype, int batch, int n_heads, int d_head, int d_rope,
                           int d_latent, const void* q_c, const void* q_r,
                           const void* w_uk, void* q_cat, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  const dim3 grid((d_latent + d_rope + kThreads - 1) / kThreads, n_heads,
                  (batch + kRows - 1) / kRows);
  const size_t lds = sizeof(float) * kRows * d_head;
  if (dtype == 0) {
    absorb_q_kernel<float><<<grid, kThreads, lds, stream>>>(
        static_cast<const float*>(q_c), static_cast<const float*>(q_r),
        static_cast<const float*>(w_uk), static_cast<float*>(q_cat), batch, n_heads, d_head,
        d_rope, d_latent);
  } else {
    absorb_q_kernel<__bf16><<<grid, kThreads, lds, stream>>>(
        static_cast<const __bf16*>(q_c), static_cast<const __bf16*>(q_r),
        static_cast<const __bf16*>(w_uk), static_cast<__bf16*>(q_cat), batch, n_heads, d_head,
        d_rope, d_latent);
  }
  return hipGetLastError();
}

hipError_t launch_out_uv(int dtype, int batch, int n_heads, int d_head, int d_latent,
                         const void* out_lat, const void* w_uv, void* out,
                         hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  const dim3 grid((d_head + kThreads - 1) / kThreads, n_heads, (batch + kRows - 1) / kRows);
  const size_t lds = sizeof(float) * kRows * d_latent;
  if (dtype == 0) {
    out_uv_kernel<float><<<grid, kThreads, lds, stream>>>(
        static_cast<const float*>(out_lat), static_cast<const float*>(w_uv),
        static_cast<float*>(out), batch, n_heads, d_head, d_latent);
  } else {
    out_uv_kernel<__bf16><<<grid, kThreads, lds, stream>>>(
        static_cast<const __bf16*>(out_lat), static_cast<const __bf16*>(w_uv),
        static_cast<__bf16*>(out), batch, n_heads, d_head, d_latent);
  }
  return hipGetLastError();
}

}  // namespace mla
