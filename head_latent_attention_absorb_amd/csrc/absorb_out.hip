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


// The same products for many rows (a prefill chunk: batch = requests x query
// tokens): a workgroup owns head i and a run of rows_per_wg rows, stages the
// whole [K x N] weight of the head in LDS once (128 KiB at both DeepSeek-V2
// shapes) and streams its rows through it.  Each wave takes 64 rows (two M
// tiles that share every B operand read) per pass of 256 rows; K is walked in
// chunks of 128 whose A operands are loaded a chunk ahead.  The weight lands
// in LDS with direct loads, its rows XOR-swizzled in 8-byte units so that the
// transposing reads of four consecutive k rows hit distinct banks: logical
// unit u of row k sits at u ^ ((k & 3) << 3).  Workgroups of one head are 8
// apart in launch order, so they share one XCD and the weight's trip through
// its L2.
template <int K, int N>
__global__ __launch_bounds__(256) void head_proj_wide_kernel(
    const __bf16* __restrict__ X, const __bf16* __restrict__ W, __bf16* __restrict__ Y,
    int batch, int n_heads, int y_row, int rows_per_wg, int chunks,
    const __bf16* __restrict__ tail_src, int tail_w) {
  constexpr int KC = 128, NKC = K / KC, NG = N / 128;
  static_assert(K % KC == 0 && N % 128 == 0 && (NKC == 1 || NG == 1), "");
  static_assert(K * N * 2 + 4 * 32 * 256 <= 160 * 1024, "the weight must fit in LDS");
  __shared__ __attribute__((aligned(16))) __bf16 w_s[K * N];
  // Per wave: one 32-row x 128-column output block on its way to global
  // memory (256-byte rows, 16-byte chunks XOR-swizzled by row & 15).
  __shared__ __attribute__((aligned(16))) uint8_t y_s[4][32 * 256];

  // Head and row run of this workgroup (see above for the XCD grouping).
  const int id = blockIdx.x;
  int i, chunk;
  if (n_heads % 8 == 0) {
    i = (id / (8 * chunks)) * 8 + id % 8;
    chunk = (id / 8) % chunks;
  } else {
    i = id / chunks;
    chunk = id % chunks;
  }
  const int r0 = chunk * rows_per_wg;
  const int r1 = min(batch, r0 + rows_per_wg);
  if (r0 >= r1) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;

  // A operand fragments of the wave's two M tiles for one K chunk: row
  // m + t*32 + l32, K elements kc*128 + ks*16 + half*8 .. +7 (zero past r1).
  bf16x8_t a[2][8], an[2][8];
  const int passes = (r1 - r0 + 255) / 256;
  const int n_chunks = passes * NKC;
  auto load_a = [&](int u, bf16x8_t(&dst)[2][8]) {
    const int pass = u / NKC, kc = u - pass * NKC;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = r0 + pass * 256 + wave * 64 + t * 32 + l32;
      const __bf16* xr = X + (static_cast<size_t>(min(row, r1 - 1)) * n_heads + i) * K +
                         kc * KC + half * 8;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) dst[t][ks] = *reinterpret_cast<const bf16x8_t*>(xr + ks * 16);
    }
  };
  load_a(0, a);

  // The whole weight of head i into LDS: wave instruction j fills 1 KiB, lane
  // l its 16-byte unit (k, v) with v the physical 16-byte column; the source is
  // the logical unit v ^ ((k & 3) << 2).
  {
    constexpr int kUnitsPerRow = N / 8;
    const __bf16* src = W + static_cast<size_t>(i) * K * N;
    const unsigned base = static_cast<unsigned>(reinterpret_cast<uintptr_t>((MLA_LDS __bf16*)w_s));
    for (int j = wave; j < K * N * 2 / 1024; j += 4) {
      const int unit = j * 64 + lane;
      const int k = unit / kUnitsPerRow, v = unit - k * kUnitsPerRow;
      load_to_lds16(src + static_cast<size_t>(k) * N + ((v ^ ((k & 3) << 2)) * 8), base + j * 1024);
    }
  }
  // The RoPE tail of the absorbed query rows is copied unchanged, 8 vectors
  // per thread per round: all their loads, then all their stores (one memory
  // round trip per round).
  if (tail_src != nullptr) {
    const int tq = tail_w / 4, n_tail = (r1 - r0) * tq;
    for (int e0 = tid; e0 < n_tail; e0 += 8 * 256) {
      bf16x4_t v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = min(e0 + j * 256, n_tail - 1);
        const int row = r0 + e / tq, c4 = e - (e / tq) * tq;
        v[j] = *reinterpret_cast<const bf16x4_t*>(
            tail_src + (static_cast<size_t>(row) * n_heads + i) * tail_w + c4 * 4);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = e0 + j * 256;
        if (e < n_tail) {
          const int row = r0 + e / tq, c4 = e - (e / tq) * tq;
          *reinterpret_cast<bf16x4_t*>(Y + (static_cast<size_t>(row) * n_heads + i) * y_row + N +
                                       c4 * 4) = v[j];
        }
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // Transposing-read coordinates (see head_proj_mfma_kernel): lane (G, q)
  // reads k row k0 + (G/2)*8 + q/4 (+4 for the high half), 8-byte unit
  // 4*(G%2) + q%4 of the 32-column block; k & 3 = q / 4 for both halves.
  const int G = lane >> 4, q16 = lane & 15;
  const int tr_k = ((G >> 1) << 3) + (q16 >> 2);
  const int tr_u = ((G & 1) << 2) + (q16 & 3);
  const int swz = (q16 >> 2) << 3;
  const i16x4_t* wl = reinterpret_cast<const i16x4_t*>(w_s);  // 8-byte units
  constexpr int kU = N / 4;                                     // units per k row

  f32x16_t acc[2][4];
  for (int u = 0; u < n_chunks; ++u) {
    const int pass = u / NKC, kc = u - pass * NKC;
    if (u + 1 < n_chunks) load_a(u + 1, an);
#pragma unroll
    for (int ng = 0; ng < NG; ++ng) {
      if (kc == 0) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[t][nb][e] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int k0 = kc * KC + ks * 16 + tr_k;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int un = ((ng * 4 + nb) * 8 + tr_u) ^ swz;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (MLA_LDS i16x4_t*)(wl + k0 * kU + un));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (MLA_LDS i16x4_t*)(wl + (k0 + 4) * kU + un));
          const bf16x8_t bop = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          // Transposed product (weight as the A operand): the accumulator holds
          // Y^T, so each lane owns one row and runs of 4 columns.
          acc[0][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bop, a[0][ks], acc[0][nb], 0, 0, 0);
          acc[1][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bop, a[1][ks], acc[1][nb], 0, 0, 0);
        }
      }
      if (kc == NKC - 1) {
        // Accumulator register e of this lane: row l32 of the tile, column
        // (e/4)*8 + half*4 + e%4 of the block, i.e. 16-byte chunk nb*4 + e/4,
        // half `half` of it.  Each 32 x 128 block goes through the wave's
        // LDS area so that the global stores write whole 256-byte row runs
        // (16 lanes per row, 4 rows per store).
        uint8_t* ys = y_s[wave];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              bf16x4_t v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = static_cast<__bf16>(acc[t][nb][g * 4 + e]);
              *reinterpret_cast<bf16x4_t*>(ys + l32 * 256 + (((nb * 4 + g) ^ (l32 & 15)) << 4) +
                                           half * 8) = v;
            }
          const int c16 = lane & 15;
#pragma unroll
          for (int r4 = 0; r4 < 8; ++r4) {
            const int rr = r4 * 4 + (lane >> 4);
            const bf16x8_t v =
                *reinterpret_cast<const bf16x8_t*>(ys + rr * 256 + ((c16 ^ (rr & 15)) << 4));
            const int row = r0 + pass * 256 + wave * 64 + t * 32 + rr;
            if (row < r1)
              *reinterpret_cast<bf16x8_t*>(Y + (static_cast<size_t>(row) * n_heads + i) * y_row +
                                           ng * 128 + c16 * 8) = v;
          }
        }
      }
    }
    if (u + 1 < n_chunks) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) a[t][ks] = an[t][ks];
    }
  }
}

// Workgroups per head of head_proj_wide_kernel and rows per workgroup (a
// multiple of 256): about 512 workgroups in all, fewer when the rows run out.
void wide_split(int batch, int n_heads, int* rows_per_wg, int* chunks) {
  const int tiles = (batch + 255) / 256;
  int c = 512 / n_heads;
  c = c < 1 ? 1 : (c > tiles ? tiles : c);
  const int per = (tiles + c - 1) / c;
  *rows_per_wg = per * 256;
  *chunks = (batch + *rows_per_wg - 1) / *rows_per_wg;
}

// Row count from which the wide form replaces head_proj_mfma_kernel.
constexpr int kWideRows = 256;
}  // namespace

hipError_t launch_absorb_q(int dtype, int batch, int n_heads, int d_head, int d_rope,
                           int d_latent, const void* q_c, const void* q_r,
                           const void* w_uk, void* q_cat, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  if (dtype == 1 && d_head == 128 && d_latent == 512 && d_rope % 4 == 0 &&
      batch >= kWideRows) {
    int rows, chunks;
    wide_split(batch, n_heads, &rows, &chunks);
    head_proj_wide_kernel<128, 512><<<n_heads * chunks, 256, 0, stream>>>(
        static_cast<const __bf16*>(q_c), static_cast<const __bf16*>(w_uk),
        static_cast<__bf16*>(q_cat), batch, n_heads, d_latent + d_rope, rows, chunks,
        d_rope > 0 ? static_cast<const __bf16*>(q_r) : nullptr, d_rope);
    return hipGetLastError();
  }
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
  if (dtype == 1 && d_latent == 512 && d_head == 128 && batch >= kWideRows) {
    int rows, chunks;
    wide_split(batch, n_heads, &rows, &chunks);
    head_proj_wide_kernel<512, 128><<<n_heads * chunks, 256, 0, stream>>>(
        static_cast<const __bf16*>(out_lat), static_cast<const __bf16*>(w_uv),
        static_cast<__bf16*>(out), batch, n_heads, d_head, rows, chunks, nullptr, 0);
    return hipGetLastError();
  }
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
