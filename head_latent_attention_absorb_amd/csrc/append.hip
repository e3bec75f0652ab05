// Cache append: the row a decode step adds to a layer's latent cache for the
// new token of each request.
//
//   c^KV = RMSNorm(W^DKV h) (gamma, eps)                       [d_c]
//   k^R  = RoPE(W^KR h) at the token's position                [d_h^R]
//   row  = [c^KV | k^R]  written at that position of the cache
//
// (V3 read-through, 2kiu.com/news/6340724, section 2.2: the KV-side listing
// and cache.append; section 2.3: k_r = RoPE(W_kr h); ai-library "DeepSeek-V2"
// notes, "Model configuration": RMSNorm after the compressed latent, and
// "Long-Context Extension": YaRN on k^R only.)  RoPE turns consecutive pairs
// (x[2i], x[2i+1]) by pos * f_i, f_i = base^(-2i/d_h^R); with a YaRN scale
// s != 1 the frequencies follow YaRN's interpolation (Peng et al. 2023): a
// pair completing r_i = L f_i / (2 pi) turns over the original context L keeps
// f_i above r = beta, is slowed to f_i / s below r = alpha, and is blended
// linearly in between.
//
// Two kernels.  (1) The projections, Y[b, n] = sum_k h[b, k] W[n, k] over the
// stacked rows of W^DKV and W^KR, as fp32 partial sums over P slices of k:
// on bf16 MFMA (both operands are k-contiguous, so each lane loads its
// operand fragment straight from global memory) when the widths allow, else
// on VALU.  Every weight element is read once: the step is HBM-bound on the
// (d_c + d_h^R) x d weights.  (2) One workgroup per request sums the slices,
// normalises the latent, rotates the key pairs and writes the row.  The pair
// frequencies are computed on the host in fp64 and each angle pos * f_i is
// reduced modulo 2 pi in fp64 before an fp32 sine and cosine: at 128K
// positions an fp32 angle would be off by ~0.01 rad.

#include <math.h>

#include "device_common.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxParts = 16;   // k slices of the projection
constexpr int kMaxPairs = 64;   // key pairs (d_h^R <= 128)
constexpr int kChunk = 8;       // k steps whose operand loads are issued together

struct AppendParams {
  const void* h;         // [B, d]
  const void* w_dkv;     // [d_c, d]
  const void* w_kr;      // [d_r, d]
  const void* gamma;     // [d_c]
  const int32_t* pos;    // [B]
  float* part;           // workspace: [P, B, d_c + d_r] fp32
  CacheView cache;       // rows written through cache.data
  void* cache_data;
  int batch, d_model, d_c, d_r, parts;
  float eps;
  double freq[kMaxPairs];  // rotation frequency of each key pair
};

// Row n of the stacked projection [W^DKV; W^KR].
template <typename T>
__device__ __forceinline__ const T* w_row(const AppendParams& p, int n) {
  return n < p.d_c ? static_cast<const T*>(p.w_dkv) + static_cast<size_t>(n) * p.d_model
                   : static_cast<const T*>(p.w_kr) + static_cast<size_t>(n - p.d_c) * p.d_model;
}

// bf16 MFMA projection.  Workgroup (column block nb of 32 rows of W, k slice
// s) has 4 waves, each over a quarter of the slice; lane (l32, half) loads
// W[nb*32 + l32][k + half*8 .. +7] (B operand) and h[m0 + l32][k + half*8 ..]
// (A operand, zero past the batch) with one 16-byte load each.  The waves'
// sums meet in LDS; wave 0 writes the slice's partial.
__global__ __launch_bounds__(kThreads) void project_mfma_kernel(AppendParams p) {
  __shared__ float red[3][16][64];
  const int nb = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int n_total = p.d_c + p.d_r;
  const int kw = p.d_model / (p.parts * 4);  // k per wave, a multiple of 16
  const int k0 = (s * 4 + wave) * kw;
  const __bf16* wrow = w_row<__bf16>(p, nb * 32 + l32) + k0 + half * 8;
  const __bf16* h = static_cast<const __bf16*>(p.h);

  for (int m0 = 0; m0 < p.batch; m0 += 32) {
    const int b = m0 + l32;
    const __bf16* hrow = h + static_cast<size_t>(min(b, p.batch - 1)) * p.d_model + k0 + half * 8;
    f32x16_t acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    // Up to kChunk k steps at a time: all their operand loads first, so that
    // they share one memory round trip, then the products.
    const int steps = kw / 16;
    for (int c0 = 0; c0 < steps; c0 += kChunk) {
      bf16x8_t bop[kChunk], aop[kChunk];
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        if (c0 + j < steps) {
          bop[j] = *reinterpret_cast<const bf16x8_t*>(wrow + (c0 + j) * 16);
          aop[j] = *reinterpret_cast<const bf16x8_t*>(hrow + (c0 + j) * 16);
        }
      }
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        if (c0 + j < steps) {
          if (b >= p.batch) {
#pragma unroll
            for (int e = 0; e < 8; ++e) aop[j][e] = static_cast<__bf16>(0.f);
          }
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[j], bop[j], acc, 0, 0, 0);
        }
      }
    }
    // Accumulator register v of this lane: row (batch) m0 + (v/4)*8 +
    // half*4 + v%4, column (n) nb*32 + l32.
    if (wave > 0) {
#pragma unroll
      for (int v = 0; v < 16; ++v) red[wave - 1][v][lane] = acc[v];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float y = acc[v] + red[0][v][lane] + red[1][v][lane] + red[2][v][lane];
        const int bb = m0 + (v >> 2) * 8 + half * 4 + (v & 3);
        if (bb < p.batch)
          p.part[(static_cast<size_t>(s) * p.batch + bb) * n_total + nb * 32 + l32] = y;
      }
    }
    __syncthreads();
  }
}

// VALU projection for any widths and fp32 or bf16 storage: workgroup (n, b
// chunk of 8) sums over the whole of k (one slice).
template <typename T>
__global__ __launch_bounds__(kThreads) void project_valu_kernel(AppendParams p) {
  __shared__ float red[8][kThreads / 64];
  const int n = blockIdx.x, b0 = blockIdx.y * 8;
  const int nb = min(8, p.batch - b0);
  const T* w = w_row<T>(p, n);
  const T* h = static_cast<const T*>(p.h);
  float acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = 0.f;
  for (int k = threadIdx.x; k < p.d_model; k += kThreads) {
    const float wv = ld(w + k);
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (r < nb) acc[r] = fmaf(wv, ld(h + static_cast<size_t>(b0 + r) * p.d_model + k), acc[r]);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const float v = wave_sum(acc[r]);
    if (lane == 0) red[r][wave] = v;
  }
  __syncthreads();
  if (threadIdx.x < nb) {
    float y = 0.f;
    for (int w2 = 0; w2 < kThreads / 64; ++w2) y += red[threadIdx.x][w2];
    p.part[static_cast<size_t>(b0 + threadIdx.x) * (p.d_c + p.d_r) + n] = y;
  }
}

// Rotation frequency of key pair i (computed on the host, in fp64).
double rope_frequency(int i, int d_r, double base, double yarn_scale, double yarn_alpha,
                      double yarn_beta, double yarn_len) {
  const double f = pow(base, -2.0 * i / d_r);
  if (yarn_scale == 1.0) return f;
  const double r = yarn_len * f / (2.0 * M_PI);
  double g = (r - yarn_alpha) / (yarn_beta - yarn_alpha);
  g = g < 0.0 ? 0.0 : (g > 1.0 ? 1.0 : g);
  return (1.0 - g) * f / yarn_scale + g * f;
}

// One workgroup per request: sum the slices, RMSNorm the latent, rotate the
// key pairs, write the row at the request's position (rows at positions
// outside [0, max_len) are not written).
template <typename T>
__global__ __launch_bounds__(kThreads) void finalize_kernel(AppendParams p) {
  extern __shared__ float y[];  // [d_c + d_r]
  __shared__ float red[kThreads / 64];
  static_assert(kThreads == 256, "the block reductions below read four waves");
  const int b = blockIdx.x;
  const int n_total = p.d_c + p.d_r;
  // What does not depend on the slices is requested first, so that its
  // memory round trips overlap theirs: the position, then the page it falls
  // in (clamped into the table; positions outside the cache write nothing),
  // and the RMSNorm weights of the first kGam * kThreads latents.
  const int pos = p.pos[b];
  const T* gamma = static_cast<const T*>(p.gamma);
  constexpr int kGam = 4;
  // (Loads are unconditional, at clamped indexes, and unused values are
  // dropped afterwards: a branch around a load makes the compiler wait for
  // it where the branches join, one memory round trip per load.)
  // The weights stay in their storage type until used (converting them
  // here would make the compiler wait for them before the slices' loads).
  T gam[kGam];
#pragma unroll
  for (int j = 0; j < kGam; ++j)
    gam[j] = gamma[min(static_cast<int>(threadIdx.x) + j * kThreads, p.d_c - 1)];
  const int pos_c = min(max(pos, 0), p.cache.max_len - 1);
  int page = 0;
  if (p.cache.page_table != nullptr)
    page = p.cache.page_table[static_cast<size_t>(b) * p.cache.max_pages +
                              pos_c / p.cache.page_size];
  // The slices' loads of kCols columns per thread are all issued before they
  // are summed (one memory round trip for up to kCols * kThreads columns).
  // The first chunk is peeled off the loop: at a loop header the compiler
  // waits for the loads issued above.
  constexpr int kCols = 3;
  auto sum_chunk = [&](int n0) {
    float v[kCols][kMaxParts];
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
      const int n = min(n0 + c * kThreads, n_total - 1);
#pragma unroll
      for (int s = 0; s < kMaxParts; ++s)
        v[c][s] = p.part[(static_cast<size_t>(min(s, p.parts - 1)) * p.batch + b) * n_total + n];
    }
    // (Pinned here, so that the compiler cannot sink loads into the
    // conditional stores below, behind the first ones' wait.)
#pragma unroll
    for (int c = 0; c < kCols; ++c)
#pragma unroll
      for (int s = 0; s < kMaxParts; ++s) {
        asm volatile("" : "+v"(v[c][s]));
        if (s >= p.parts) v[c][s] = 0.f;
      }
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
      float t = 0.f;
#pragma unroll
      for (int s = 0; s < kMaxParts; ++s) t += v[c][s];
      if (n0 + c * kThreads < n_total) y[n0 + c * kThreads] = t;
    }
  };
  sum_chunk(threadIdx.x);
  for (int n0 = threadIdx.x + kCols * kThreads; n0 < n_total; n0 += kCols * kThreads)
    sum_chunk(n0);
  __syncthreads();
  float ss = 0.f;
  for (int n = threadIdx.x; n < p.d_c; n += kThreads) ss += y[n] * y[n];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < kThreads / 64; ++w) tot += red[w];
  const float inv = 1.f / sqrtf(tot / p.d_c + p.eps);

  if (pos < 0 || pos >= p.cache.max_len) return;
  const size_t phys =
      p.cache.page_table == nullptr
          ? static_cast<size_t>(b) * p.cache.max_len + pos
          : static_cast<size_t>(page) * p.cache.page_size + pos % p.cache.page_size;
  // The finished row, in place in y: the normalised latent, then the rotated
  // key pairs.
#pragma unroll
  for (int j = 0; j < kGam; ++j) {
    const int n = threadIdx.x + j * kThreads;
    if (n < p.d_c) y[n] = y[n] * inv * static_cast<float>(gam[j]);
  }
  for (int n = threadIdx.x + kGam * kThreads; n < p.d_c; n += kThreads)
    y[n] = y[n] * inv * ld(gamma + n);
  for (int i = threadIdx.x; i < p.d_r / 2; i += kThreads) {
    // The angle is reduced modulo 2 pi in fp64; the reduced angle's sine and
    // cosine are fp32-accurate.
    const double ang = static_cast<double>(pos) * p.freq[i];
    const float ra = static_cast<float>(ang - 2.0 * M_PI * rint(ang / (2.0 * M_PI)));
    float sn, cs;
    sincosf(ra, &sn, &cs);
    const float x0 = y[p.d_c + 2 * i], x1 = y[p.d_c + 2 * i + 1];
    y[p.d_c + 2 * i] = x0 * cs - x1 * sn;
    y[p.d_c + 2 * i + 1] = x0 * sn + x1 * cs;
  }
  __syncthreads();
  if (!p.cache.fp8) {
    T* row = static_cast<T*>(p.cache_data) + phys * n_total;
    for (int n = threadIdx.x; n < n_total; n += kThreads) st(row + n, y[n]);
    return;
  }
  // Low-bit cache: E4M3 codes with the row's scale max|y| / 448, as
  // mla_quantize_rows computes them (fp32 divisions, round to nearest even).
  float amax = 0.f;
  for (int n = threadIdx.x; n < n_total; n += kThreads) amax = fmaxf(amax, fabsf(y[n]));
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = amax > 0.f ? amax / 448.f : 1.f;
  uint8_t* codes = static_cast<uint8_t*>(p.cache_data) + phys * n_total;
  for (int n = 2 * threadIdx.x; n < n_total; n += 2 * kThreads) {
    const float a = fminf(fmaxf(y[n] / sc, -448.f), 448.f);
    const float c = n + 1 < n_total ? fminf(fmaxf(y[n + 1] / sc, -448.f), 448.f) : 0.f;
    const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(a, c, 0, false);
    codes[n] = static_cast<uint8_t>(packed & 0xFF);
    if (n + 1 < n_total) codes[n + 1] = static_cast<uint8_t>((packed >> 8) & 0xFF);
  }
  if (threadIdx.x == 0) const_cast<float*>(p.cache.scales)[phys] = sc;
}

// k slices of the MFMA projection: the most of 16, 8, 4, 2, 1 that divides
// d_model into 4 * 16-element steps per wave; 0 when none does.
int mfma_parts(int d_model) {
  for (int parts = kMaxParts; parts >= 1; parts /= 2)
    if (d_model % (parts * 4 * 16) == 0) return parts;
  return 0;
}

bool use_mfma_projection(int dtype, int d_model, int d_c, int d_r) {
  return dtype == 1 && (d_c + d_r) % 32 == 0 && d_c % 32 == 0 && mfma_parts(d_model) > 0;
}

}  // namespace

size_t append_workspace_bytes(int dtype, int batch, int d_model, int d_c, int d_r) {
  const int parts = use_mfma_projection(dtype, d_model, d_c, d_r) ? mfma_parts(d_model) : 1;
  return static_cast<size_t>(parts) * batch * (d_c + d_r) * sizeof(float);
}

hipError_t launch_cache_append(int dtype, int batch, int d_model, int d_c, int d_r,
                               const void* h, const void* w_dkv, const void* w_kr,
                               const void* gamma, float eps, double base, double yarn_scale,
                               double yarn_alpha, double yarn_beta, double yarn_len,
                               const int32_t* positions, const CacheView& cache,
                               void* cache_data, void* workspace, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  AppendParams p;
  p.h = h;
  p.w_dkv = w_dkv;
  p.w_kr = w_kr;
  p.gamma = gamma;
  p.pos = positions;
  p.part = static_cast<float*>(workspace);
  p.cache = cache;
  p.cache_data = cache_data;
  p.batch = batch;
  p.d_model = d_model;
  p.d_c = d_c;
  p.d_r = d_r;
  p.eps = eps;
  if (d_r / 2 > kMaxPairs) return hipErrorInvalidValue;
  for (int i = 0; i < d_r / 2; ++i)
    p.freq[i] = rope_frequency(i, d_r, base, yarn_scale, yarn_alpha, yarn_beta, yarn_len);
  const int n_total = d_c + d_r;
  if (use_mfma_projection(dtype, d_model, d_c, d_r)) {
    p.parts = mfma_parts(d_model);
    project_mfma_kernel<<<dim3(n_total / 32, p.parts), kThreads, 0, stream>>>(p);
  } else {
    p.parts = 1;
    const dim3 grid(n_total, (batch + 7) / 8);
    if (dtype == 1)
      project_valu_kernel<__bf16><<<grid, kThreads, 0, stream>>>(p);
    else
      project_valu_kernel<float><<<grid, kThreads, 0, stream>>>(p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = sizeof(float) * n_total;
  if (dtype == 1)
    finalize_kernel<__bf16><<<batch, kThreads, lds, stream>>>(p);
  else
    finalize_kernel<float><<<batch, kThreads, lds, stream>>>(p);
  return hipGetLastError();
}

}  // namespace mla
