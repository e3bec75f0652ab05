// K1 (query absorption) and K4 (W^UV output projection): per-head batched
// products that stream one weight matrix per head.
//
// Absorption: q_lat,i = W^UK_i^T q^C_i (DeepSeek-V2 read-through,
// 2kiu.com/news/6085339, section 2.3; DeepSeek-V3 read-through,
// 2kiu.com/news/6340724, section 2.3).  Output: o_i = W^UV_i o_lat,i applied
// after the latent-space sum (V2 read-through section 2.3).
//
// Both are HBM-bound at decode batch sizes: every weight element is read once
// per call and used for `batch` multiply-adds.  Two forms:
//  * head_proj_mfma_kernel, bf16 at the DeepSeek-V2 widths: a workgroup stages
//    one [K x NB] weight block in LDS and multiplies it on MFMA (see below).
//  * absorb_q_kernel / out_uv_kernel, any widths and fp32: one workgroup owns
//    one head and a 256-wide slice of output columns; the batch rows it serves
//    are staged in LDS as fp32 and each thread keeps kRows accumulators, so a
//    weight element loaded once feeds kRows FMAs.

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

// bf16 MFMA form of both products, for the DeepSeek-V2 widths:
//   Y[b, i, n] = sum_{k < K} X[b, i, k] W[i, k, n]      (n < N, per head i)
// absorption: X = q^C (K = d_head = 128), W = W^UK (N = d_latent = 512)
// output:     X = o_lat (K = d_latent = 512), W = W^UV (N = d_head = 128)
// One workgroup owns head i and an NB-column block of W, stages that
// [K x NB] block in LDS (the only HBM stream: every weight element is read
// once), and computes all batch rows with v_mfma_f32_32x32x16_bf16.  The
// 4 waves split the block into NS column sub-blocks of 32 and 4/NS K parts;
// K parts are summed through LDS.  Batch rows are the A operand (M tiles of
// 32, loaded straight from global memory, zero past `batch`); the weight is
// the B operand, read with the transposing LDS read (within a 16-lane group,
// lane i receives element i%4 of the 8-byte chunk addressed by lane 4j + i/4,
// for j = 0..3).
template <int K, int NB, int NS>
__global__ __launch_bounds__(256) void head_proj_mfma_kernel(
    const __bf16* __restrict__ X, const __bf16* __restrict__ W, __bf16* __restrict__ Y,
    int batch, int n_heads, int N, int y_row, const __bf16* __restrict__ tail_src,
    int tail_w) {
  constexpr int KP = 4 / NS;          // K parts
  constexpr int KW = K / KP;          // K range of one wave
  constexpr int KSTEPS = KW / 16;
  static_assert(NS * KP == 4 && KW % 16 == 0 && NB == NS * 32, "");
  __shared__ __attribute__((aligned(16))) __bf16 w_s[K * NB];
  __shared__ __attribute__((aligned(16))) float red[(KP > 1 ? KP - 1 : 1) * NS * 16 * 64];

  const int i = blockIdx.y;
  const int n0 = blockIdx.x * NB;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int ns = wave % NS, kp = wave / NS;

  // Transposing-read source coordinates of this lane (see above).
  const int G = lane >> 4, r16 = lane & 15;
  const int tr_k = ((G >> 1) << 3) + (r16 >> 2);
  const int tr_n = ns * 32 + ((G & 1) << 4) + ((r16 & 3) << 2);

  // A operand fragments of one 32-row M tile: row m0 + l32, K elements
  // kp*KW + ks*16 + half*8 .. +7.  Rows past `batch` are zero.
  bf16x8_t a[KSTEPS], a_next[KSTEPS];
  auto load_a = [&](int m0, bf16x8_t(&dst)[KSTEPS]) {
    const int b = m0 + l32;
    const __bf16* xrow = X + (static_cast<size_t>(b) * n_heads + i) * K + kp * KW + half * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if (b < batch) {
        dst[ks] = *reinterpret_cast<const bf16x8_t*>(xrow + ks * 16);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[ks][j] = static_cast<__bf16>(0.f);
      }
    }
  };
  // The first tile's rows are requested before the weight block so that both
  // HBM round trips overlap.
  load_a(0, a);

  // The RoPE tail of the absorbed query is copied unchanged (absorption only),
  // in 4-element vectors spread over the gridDim.x workgroups of this head.
  // The first round is loaded here so that it overlaps the weight stream.
  const int tail_q = tail_w / 4;
  const int tail_vecs = tail_src != nullptr ? batch * tail_q : 0;
  const int tv0 = blockIdx.x * 256 + tid, tv_step = gridDim.x * 256;
  auto tail_at = [&](int e) {
    const int b = e / tail_q, r4 = e - b * tail_q;
    return reinterpret_cast<const bf16x4_t*>(
        tail_src + (static_cast<size_t>(b) * n_heads + i) * tail_w + r4 * 4);
  };
  auto tail_dst = [&](int e) {
    const int b = e / tail_q, r4 = e - b * tail_q;
    return reinterpret_cast<bf16x4_t*>(Y + (static_cast<size_t>(b) * n_heads + i) * y_row + N +
                                       r4 * 4);
  };
  bf16x4_t tv;
  if (tv0 < tail_vecs) tv = tail_at(tv0)[0];

  // Stage W[i][0:K][n0:n0+NB] (row-major, NB contiguous): all loads first,
  // then the LDS stores.
  constexpr int kChunksPerRow = NB / 8;
  constexpr int kLoads = K * kChunksPerRow / 256;
  static_assert(K * kChunksPerRow % 256 == 0, "");
  const __bf16* wsrc = W + static_cast<size_t>(i) * K * N + n0;
  bf16x8_t wv[kLoads];
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int ch = tid + u * 256;
    const int k = ch / kChunksPerRow, cc = ch - k * kChunksPerRow;
    wv[u] = *reinterpret_cast<const bf16x8_t*>(wsrc + static_cast<size_t>(k) * N + cc * 8);
  }
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int ch = tid + u * 256;
    const int k = ch / kChunksPerRow, cc = ch - k * kChunksPerRow;
    *reinterpret_cast<bf16x8_t*>(w_s + k * NB + cc * 8) = wv[u];
  }
  // Second half of the RoPE tail copy: store what was loaded above, then the
  // further rounds needed when the tail has more vectors than the head's
  // workgroups have threads.
  if (tv0 < tail_vecs) {
    tail_dst(tv0)[0] = tv;
    for (int e = tv0 + tv_step; e < tail_vecs; e += tv_step) tail_dst(e)[0] = tail_at(e)[0];
  }
  __syncthreads();

  for (int m0 = 0; m0 < batch; m0 += 32) {
    // The next M tile's rows are requested before this tile's products.
    if (m0 + 32 < batch) load_a(m0 + 32, a_next);
    f32x16_t acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int k0 = kp * KW + ks * 16;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (MLA_LDS i16x4_t*)(w_s + (k0 + tr_k) * NB + tr_n));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (MLA_LDS i16x4_t*)(w_s + (k0 + tr_k + 4) * NB + tr_n));
      const bf16x8_t bop =
          __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], bop, acc, 0, 0, 0);
    }
    if constexpr (KP > 1) {
      if (kp > 0) {
#pragma unroll
        for (int v = 0; v < 16; ++v) red[(((kp - 1) * NS + ns) * 16 + v) * 64 + lane] = acc[v];
      }
      __syncthreads();
      if (kp == 0) {
#pragma unroll
        for (int q = 0; q < KP - 1; ++q)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[v] += red[((q * NS + ns) * 16 + v) * 64 + lane];
      }
      __syncthreads();
    }
    if (kp == 0) {
      // Accumulator register v of this lane: row (v/4)*8 + half*4 + v%4, column l32.
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int bb = m0 + (v >> 2) * 8 + half * 4 + (v & 3);
        if (bb < batch)
          Y[(static_cast<size_t>(bb) * n_heads + i) * y_row + n0 + ns * 32 + l32] =
              static_cast<__bf16>(acc[v]);
      }
    }
    if (m0 + 32 < batch) {
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) a[ks] = a_next[ks];
    }
  }
}

}  // namespace

hipError_t launch_absorb_q(int dtype, int batch, int n_heads, int d_head, int d_rope,
                           int d_latent, const void* q_c, const void* q_r,
                           const void* w_uk, void* q_cat, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  if (dtype == 1 && d_head == 128 && d_latent % 128 == 0 && d_rope % 4 == 0) {
    head_proj_mfma_kernel<128, 128, 4><<<dim3(d_latent / 128, n_heads), 256, 0, stream>>>(
        static_cast<const __bf16*>(q_c), static_cast<const __bf16*>(w_uk),
        static_cast<__bf16*>(q_cat), batch, n_heads, d_latent, d_latent + d_rope,
        d_rope > 0 ? static_cast<const __bf16*>(q_r) : nullptr, d_rope);
    return hipGetLastError();
  }
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
  if (dtype == 1 && d_latent == 512 && d_head % 64 == 0) {
    head_proj_mfma_kernel<512, 64, 2><<<dim3(d_head / 64, n_heads), 256, 0, stream>>>(
        static_cast<const __bf16*>(out_lat), static_cast<const __bf16*>(w_uv),
        static_cast<__bf16*>(out), batch, n_heads, d_head, d_head, nullptr, 0);
    return hipGetLastError();
  }
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
