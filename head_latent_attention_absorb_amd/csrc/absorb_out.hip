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

// The transposing reads of a weight block address four consecutive rows at
// once (the same columns of each), which would fall in the same banks where
// the rows are a multiple of 256 bytes (the width of the 64 LDS banks)
// apart.  The 16-byte chunk c of row r is therefore staged in slot
//   c ^ 4 (r % 4)          for 128-column blocks (256-byte rows),
//   c ^ 4 ((r / 2) % 2)    for 64-column blocks (two 128-byte rows per 256 bytes),
// which puts the four rows' chunks in different banks.
template <int NB>
__device__ __forceinline__ int w_slot_of(int chunk, int row) {
  static_assert(NB == 128 || NB == 64, "");
  return NB == 128 ? chunk ^ ((row & 3) << 2) : chunk ^ (((row >> 1) & 1) << 2);
}
// bf16 MFMA form of both products, for the DeepSeek-V2 widths:
//   Y[b, i, n] = sum_{k < K} X[b, i, k] W[i, k, n]      (n < N, per head i)
// absorption: X = q^C (K = d_head = 128), W = W^UK (N = d_latent = 512)
// output:     X = o_lat (K = d_latent = 512), W = W^UV (N = d_head = 128)
// One workgroup owns head i and an NB-column block of W, stages that
// [K x NB] block in LDS with direct-to-LDS loads, all issued at once (the
// only HBM stream: every weight element is read once), and computes the
// batch's rows (at most 32: one M tile; larger batches run on
// head_proj_rows_kernel) with v_mfma_f32_32x32x16_bf16.  The N / NB blocks of a head are
// consecutive work ids, and consecutive work ids run on one XCD (workgroup x
// runs on XCD x % 8): the blocks of a weight row are read from one L2 at
// about the same time.  The 4 waves split the block into NS column
// sub-blocks of 32 and 4/NS K parts; K parts are summed through LDS.  Batch
// rows are the A operand (loaded straight from global memory, zero past
// `batch`); the weight is the B operand, read with the transposing LDS read
// (within a 16-lane group, lane i receives element i%4 of the 8-byte chunk
// addressed by lane 4j + i/4, for j = 0..3).  The results pass through LDS
// so that every output row is written in 16-byte pieces.
template <int K, int NB, int NS>
__global__ __launch_bounds__(256) void head_proj_mfma_kernel(
    const __bf16* __restrict__ X, const __bf16* __restrict__ W, __bf16* __restrict__ Y,
    int batch, int n_heads, int N, int y_row, const __bf16* __restrict__ tail_src,
    int tail_w) {
  constexpr int KP = 4 / NS;          // K parts
  constexpr int KW = K / KP;          // K range of one wave
  constexpr int KSTEPS = KW / 16;
  static_assert(NS * KP == 4 && KW % 16 == 0 && NB == NS * 32, "");
  __shared__ __attribute__((aligned(1024))) __bf16 w_s[K * NB];
  __shared__ __attribute__((aligned(16))) float red[KP > 1 ? (KP - 1) * NS * 16 * 64 : 1];
  __shared__ __attribute__((aligned(16))) __bf16 y_s[32 * NB];

  const int nblk = N / NB;
  const int nwg = gridDim.x;  // a multiple of 8
  const int work = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  if (work >= n_heads * nblk) return;
  const int i = work / nblk, blk = work - i * nblk;
  const int n0 = blk * NB;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int ns = wave % NS, kp = wave / NS;

  // Transposing-read source coordinates of this lane (see above).
  const int G = lane >> 4, r16 = lane & 15;
  const int tr_k = ((G >> 1) << 3) + (r16 >> 2);
  const int tr_n = ns * 32 + ((G & 1) << 4) + ((r16 & 3) << 2);
  // (its slot in the swizzled weight block: rows k0 + tr_k and k0 + tr_k + 4,
  // k0 a multiple of 16, share the row's swizzle)
  const int tr_col = (w_slot_of<NB>(tr_n >> 3, tr_k) << 3) | (tr_n & 7);

  // A operand fragments of the M tile (batch <= 32 rows; more rows run on
  // head_proj_rows_kernel): row l32, K elements kp*KW + ks*16 + half*8 .. +7.
  // Rows past `batch` are zero.  They are requested before the weight block
  // so that both HBM round trips overlap.
  bf16x8_t a[KSTEPS];
  {
    const __bf16* xrow = X + (static_cast<size_t>(l32) * n_heads + i) * K + kp * KW + half * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if (l32 < batch) {
        a[ks] = *reinterpret_cast<const bf16x8_t*>(xrow + ks * 16);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) a[ks][j] = static_cast<__bf16>(0.f);
      }
    }
  }

  // Stage W[i][0:K][n0:n0+NB] (row-major, NB contiguous) in LDS, in the same
  // layout: one wave instruction copies 1 KiB, rows of NB elements.
  {
    constexpr int kLanesPerRow = NB / 8;  // 16-byte chunks per row
    constexpr int kRowsPerCopy = 64 / kLanesPerRow;
    constexpr int kCopies = K / kRowsPerCopy;
    static_assert(K % kRowsPerCopy == 0 && kCopies % 4 == 0, "");
    const __bf16* src = W + (static_cast<size_t>(i) * K + lane / kLanesPerRow) * N + n0 +
                        w_slot_of<NB>(lane % kLanesPerRow, lane / kLanesPerRow) * 8;
    const unsigned base =
        static_cast<unsigned>(reinterpret_cast<uintptr_t>((MLA_LDS __bf16*)w_s));
#pragma unroll
    for (int jj = 0; jj < kCopies / 4; ++jj) {
      const int j = jj * 4 + wave;
      load_to_lds16(src + static_cast<size_t>(j) * kRowsPerCopy * N, base + j * 1024);
    }
  }

  // The RoPE tail of the absorbed query is copied unchanged (absorption
  // only), in 4-element vectors spread over the nblk workgroups of this head.
  const int tail_q = tail_w / 4;
  const int tail_vecs = tail_src != nullptr ? batch * tail_q : 0;
  for (int e = blk * 256 + tid; e < tail_vecs; e += nblk * 256) {
    const int b = e / tail_q, r4 = e - b * tail_q;
    *reinterpret_cast<bf16x4_t*>(Y + (static_cast<size_t>(b) * n_heads + i) * y_row + N +
                                 r4 * 4) =
        *reinterpret_cast<const bf16x4_t*>(
            tail_src + (static_cast<size_t>(b) * n_heads + i) * tail_w + r4 * 4);
  }
  // The weight block must have landed before the barrier publishes it.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  {
    f32x16_t acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int k0 = kp * KW + ks * 16;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (MLA_LDS i16x4_t*)(w_s + (k0 + tr_k) * NB + tr_col));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (MLA_LDS i16x4_t*)(w_s + (k0 + tr_k + 4) * NB + tr_col));
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
    }
    if (kp == 0) {
      // Accumulator register v of this lane: row (v/4)*8 + half*4 + v%4, column l32.
#pragma unroll
      for (int v = 0; v < 16; ++v)
        y_s[((v >> 2) * 8 + half * 4 + (v & 3)) * NB + ns * 32 + l32] =
            static_cast<__bf16>(acc[v]);
    }
    __syncthreads();
    constexpr int kRowChunks = NB / 8;
    for (int c = tid; c < 32 * kRowChunks; c += 256) {
      const int r = c / kRowChunks, ch = c - r * kRowChunks;
      if (r < batch)
        *reinterpret_cast<bf16x8_t*>(Y + (static_cast<size_t>(r) * n_heads + i) * y_row +
                                     n0 + ch * 8) =
            *reinterpret_cast<const bf16x8_t*>(y_s + r * NB + ch * 8);
    }
  }
}

// Launch shape of head_proj_mfma_kernel: one workgroup per (head, column
// block), a multiple of the 8 XCDs.
int head_proj_grid(int n_heads, int N, int NB) {
  return (n_heads * (N / NB) + 7) / 8 * 8;
}

// The same product for more than one M tile of rows.  One workgroup owns head
// i, an NB-column block of W and a chunk of MR rows; the weight block and the
// chunk's rows are staged in LDS in one burst of direct-to-LDS loads (a
// single memory round trip, where loading each tile's rows in turn would
// expose one round trip per tile), each wave reads its weight fragments once
// into registers, and the chunk's M tiles are multiplied from LDS.  LDS row r
// holds X row r0 + r with its 16-byte chunk c in slot c ^ (r % 16), so that
// the A-operand reads of 16 consecutive rows fall in 16 different bank
// groups.  Rows past the batch are neither loaded nor stored.  The chunks
// and column blocks of a head are consecutive work ids (one XCD: they share
// the weight block through its L2).
template <int K, int NB, int NS, int MR>
__global__ __launch_bounds__(256) void head_proj_rows_kernel(
    const __bf16* __restrict__ X, const __bf16* __restrict__ W, __bf16* __restrict__ Y,
    int batch, int n_heads, int N, int y_row, const __bf16* __restrict__ tail_src,
    int tail_w) {
  constexpr int KP = 4 / NS;          // K parts
  constexpr int KW = K / KP;          // K range of one wave
  constexpr int KSTEPS = KW / 16;
  constexpr int kXChunks = K / 8;     // 16-byte chunks per row
  constexpr int kXRowsPerCopy = 64 / kXChunks;
  static_assert(NS * KP == 4 && KW % 16 == 0 && NB == NS * 32 && MR % 32 == 0, "");
  static_assert(kXChunks % 16 == 0 && 64 % kXChunks == 0, "rows of 128, 256 or 512 elements");
  __shared__ __attribute__((aligned(1024))) __bf16 w_s[K * NB];
  __shared__ __attribute__((aligned(1024))) __bf16 x_s[MR * K];
  __shared__ __attribute__((aligned(16))) float red[KP > 1 ? (KP - 1) * NS * 16 * 64 : 1];
  __shared__ __attribute__((aligned(16))) __bf16 y_s[32 * NB];

  const int nblk = N / NB;
  const int nchunk = (batch + MR - 1) / MR;
  const int nwg = gridDim.x;  // a multiple of 8
  const int work = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  if (work >= n_heads * nblk * nchunk) return;
  const int rc = work % nchunk;
  const int hbk = work / nchunk;
  const int i = hbk / nblk, blk = hbk - i * nblk;
  const int n0 = blk * NB, r0 = rc * MR;
  const int rows = min(MR, batch - r0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int ns = wave % NS, kp = wave / NS;

  // Weight block W[i][0:K][n0:n0+NB], row-major as in global memory.
  {
    constexpr int kLanesPerRow = NB / 8;
    constexpr int kRowsPerCopy = 64 / kLanesPerRow;
    constexpr int kCopies = K / kRowsPerCopy;
    static_assert(K % kRowsPerCopy == 0 && kCopies % 4 == 0, "");
    const __bf16* src = W + (static_cast<size_t>(i) * K + lane / kLanesPerRow) * N + n0 +
                        w_slot_of<NB>(lane % kLanesPerRow, lane / kLanesPerRow) * 8;
    const unsigned base =
        static_cast<unsigned>(reinterpret_cast<uintptr_t>((MLA_LDS __bf16*)w_s));
#pragma unroll
    for (int jj = 0; jj < kCopies / 4; ++jj) {
      const int j = jj * 4 + wave;
      load_to_lds16(src + static_cast<size_t>(j) * kRowsPerCopy * N, base + j * 1024);
    }
  }
  // The chunk's rows, swizzled (see above); one instruction fills 1 KiB.
  {
    const int xr = lane / kXChunks, slot = lane % kXChunks;
    const unsigned base =
        static_cast<unsigned>(reinterpret_cast<uintptr_t>((MLA_LDS __bf16*)x_s));
    const int copies = (rows + kXRowsPerCopy - 1) / kXRowsPerCopy;
    for (int j = wave; j < copies; j += 4) {
      const int r = j * kXRowsPerCopy + xr;
      const int b = r0 + min(r, rows - 1);
      load_to_lds16(X + (static_cast<size_t>(b) * n_heads + i) * K + (slot ^ (r & 15)) * 8,
                    base + j * 1024);
    }
  }

  // The RoPE tail of the absorbed query is copied unchanged (absorption
  // only), spread over the workgroups of this head.
  const int tail_q = tail_w / 4;
  const int tail_vecs = tail_src != nullptr ? batch * tail_q : 0;
  for (int e = (blk * nchunk + rc) * 256 + tid; e < tail_vecs; e += nblk * nchunk * 256) {
    const int b = e / tail_q, r4 = e - b * tail_q;
    *reinterpret_cast<bf16x4_t*>(Y + (static_cast<size_t>(b) * n_heads + i) * y_row + N +
                                 r4 * 4) =
        *reinterpret_cast<const bf16x4_t*>(
            tail_src + (static_cast<size_t>(b) * n_heads + i) * tail_w + r4 * 4);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // Weight fragments of this wave (transposing reads, as head_proj_mfma_kernel).
  const int G = lane >> 4, r16 = lane & 15;
  const int tr_k = ((G >> 1) << 3) + (r16 >> 2);
  const int tr_n = ns * 32 + ((G & 1) << 4) + ((r16 & 3) << 2);
  // (its slot in the swizzled weight block: rows k0 + tr_k and k0 + tr_k + 4,
  // k0 a multiple of 16, share the row's swizzle)
  const int tr_col = (w_slot_of<NB>(tr_n >> 3, tr_k) << 3) | (tr_n & 7);
  bf16x8_t bfr[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const int k0 = kp * KW + ks * 16;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MLA_LDS i16x4_t*)(w_s + (k0 + tr_k) * NB + tr_col));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MLA_LDS i16x4_t*)(w_s + (k0 + tr_k + 4) * NB + tr_col));
    bfr[ks] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }

  const int ntiles = (rows + 31) / 32;
  for (int t = 0; t < ntiles; ++t) {
    const int m0 = t * 32;
    // A operand: row m0 + l32 (its swizzle key is l32 % 16), K slots
    // kp*KW + ks*16 + half*8 .. +7.
    const __bf16* xrow = x_s + (m0 + l32) * K;
    f32x16_t acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int c = (kp * KW + ks * 16) / 8 + half;
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(xrow + (c ^ (l32 & 15)) * 8);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bfr[ks], acc, 0, 0, 0);
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
    }
    if (kp == 0) {
      // Accumulator register v of this lane: row (v/4)*8 + half*4 + v%4, column l32.
#pragma unroll
      for (int v = 0; v < 16; ++v)
        y_s[((v >> 2) * 8 + half * 4 + (v & 3)) * NB + ns * 32 + l32] =
            static_cast<__bf16>(acc[v]);
    }
    __syncthreads();
    constexpr int kRowChunks = NB / 8;
    for (int c = tid; c < 32 * kRowChunks; c += 256) {
      const int r = c / kRowChunks, ch = c - r * kRowChunks;
      if (m0 + r < rows)
        *reinterpret_cast<bf16x8_t*>(
            Y + (static_cast<size_t>(r0 + m0 + r) * n_heads + i) * y_row + n0 + ch * 8) =
            *reinterpret_cast<const bf16x8_t*>(y_s + r * NB + ch * 8);
    }
    // y_s and red are rewritten by the next tile.
    __syncthreads();
  }
}

// Launch shape of head_proj_rows_kernel: one workgroup per (head, column
// block, chunk of MR rows), a multiple of the 8 XCDs.
int head_proj_rows_grid(int n_heads, int N, int NB, int batch, int MR) {
  return (n_heads * (N / NB) * ((batch + MR - 1) / MR) + 7) / 8 * 8;
}


// The same products for many rows: a workgroup owns head i and a run of
// rows_per_wg rows of one request, stages the whole weight of the head in LDS
// once (128 KiB at the DeepSeek-V2 shapes) and streams its rows through it.
// Rows are (request b, row t < len_b) with element offsets
//   X: b * x_req + t * x_row + i * x_head,  Y: b * y_req + t * y_row + i * y_head,
// which covers the absorbed query and W^UV product of a prefill chunk (one
// "request" of batch rows) and the explicit key / value expansion of cached
// latents (rows of each request's cache, shared by all heads).
// Each wave takes 64 rows (two M tiles that share every weight read) per pass
// of 256 rows; K is walked in chunks of 128 whose row operands are loaded a
// chunk ahead.  The weight is the MFMA A operand (the product is computed
// transposed, so that each lane ends up owning one output row), read from LDS
// either with the transposing read (kWT false: W[i] stored [K][N], as W^UK in
// the absorption and W^UV) or plainly (kWT true: stored [N][K], as W^UK in the
// key expansion).  The weight lands in LDS with direct loads, XOR-swizzled
// against bank conflicts: [K][N] rows in 8-byte units, unit u of row k at
// u ^ ((k & 3) << 3); [N][K] rows in 16-byte units, unit c of row n at
// c ^ (n & 15).  Output blocks go through LDS so that stores write whole
// 256-byte row runs.
struct WideArgs {
  const __bf16* X;
  const __bf16* W;
  __bf16* Y;
  const int32_t* seq_lens;  // rows of request b: seq_lens[b] (NULL: rows_per_req)
  int n_req, rows_per_req, n_heads;
  long long x_req, x_row, x_head, y_req, y_row, y_head;
  int rows_per_wg, chunks;  // row runs per request
  const __bf16* tail_src;   // RoPE tail copied after the N product columns:
  int tail_w;               // row t of head i (one request) at
  long long tail_row;       // tail_src + t * tail_row + i * tail_w
};

template <int K, int N, bool kWT>
__global__ __launch_bounds__(256) void head_proj_wide_kernel(WideArgs p) {
  constexpr int KC = 128, NKC = K / KC, NG = N / 128;
  static_assert(K % KC == 0 && N % 128 == 0 && (NKC == 1 || NG == 1), "");
  static_assert(K * N * 2 + 4 * 32 * 256 <= 160 * 1024, "the weight must fit in LDS");
  __shared__ __attribute__((aligned(16))) __bf16 w_s[K * N];
  // Per wave: one 32-row x 128-column output block on its way to global
  // memory (256-byte rows, 16-byte chunks XOR-swizzled by row & 15).
  __shared__ __attribute__((aligned(16))) uint8_t y_s[4][32 * 256];

  // (head, work) of this workgroup; work = request * chunks + run.  When the
  // works split evenly over the 8 XCDs, every XCD takes whole works and runs
  // all heads of each (its rows, shared by the heads, stay in its L2);
  // otherwise workgroups of one head are n_heads apart (same XCD when
  // n_heads % 8 == 0) and share the head's weight through L2.
  const int id = blockIdx.x;
  const int n_works = p.n_req * p.chunks;
  int i, work;
  if (n_works % 8 == 0) {
    i = (id >> 3) % p.n_heads;
    work = ((id >> 3) / p.n_heads) * 8 + (id & 7);
  } else {
    i = id % p.n_heads;
    work = id / p.n_heads;
  }
  const int b = work / p.chunks, chunk = work - b * p.chunks;
  const int len = p.seq_lens != nullptr ? min(p.seq_lens[b], p.rows_per_req) : p.rows_per_req;
  const int r0 = chunk * p.rows_per_wg;
  const int r1 = min(len, r0 + p.rows_per_wg);
  if (r0 >= r1) return;
  const __bf16* X = p.X + b * p.x_req + i * p.x_head;
  __bf16* Y = p.Y + b * p.y_req + i * p.y_head;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;

  // Row operand fragments of the wave's two M tiles for one K chunk: row
  // m + t*32 + l32, K elements kc*128 + ks*16 + half*8 .. +7 (rows past r1
  // repeat the last row and are not stored).
  bf16x8_t a[2][8], an[2][8];
  const int passes = (r1 - r0 + 255) / 256;
  const int n_chunks = passes * NKC;
  auto load_a = [&](int u, bf16x8_t(&dst)[2][8]) {
    const int pass = u / NKC, kc = u - pass * NKC;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = r0 + pass * 256 + wave * 64 + t * 32 + l32;
      const __bf16* xr = X + min(row, r1 - 1) * p.x_row + kc * KC + half * 8;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) dst[t][ks] = *reinterpret_cast<const bf16x8_t*>(xr + ks * 16);
    }
  };
  load_a(0, a);

  // The whole weight of head i into LDS: wave instruction j fills 1 KiB, lane
  // l its physical 16-byte unit; the source is the logical unit it holds.
  {
    const __bf16* src = p.W + static_cast<size_t>(i) * K * N;
    const unsigned base = static_cast<unsigned>(reinterpret_cast<uintptr_t>((MLA_LDS __bf16*)w_s));
    for (int j = wave; j < K * N * 2 / 1024; j += 4) {
      const int unit = j * 64 + lane;
      if constexpr (kWT) {
        constexpr int kUnitsPerRow = K / 8;
        const int n = unit / kUnitsPerRow, c = unit - n * kUnitsPerRow;
        load_to_lds16(src + static_cast<size_t>(n) * K + ((c ^ (n & 15)) * 8), base + j * 1024);
      } else {
        constexpr int kUnitsPerRow = N / 8;
        const int k = unit / kUnitsPerRow, v = unit - k * kUnitsPerRow;
        load_to_lds16(src + static_cast<size_t>(k) * N + ((v ^ ((k & 3) << 2)) * 8),
                      base + j * 1024);
      }
    }
  }
  // The RoPE tail of the absorbed query rows is copied unchanged, 8 vectors
  // per thread per round: all their loads, then all their stores (one memory
  // round trip per round).
  if (p.tail_src != nullptr) {
    const __bf16* tsrc = p.tail_src + i * p.tail_w;
    const long long t_row = p.tail_row;
    const int tq = p.tail_w / 4, n_tail = (r1 - r0) * tq;
    for (int e0 = tid; e0 < n_tail; e0 += 8 * 256) {
      bf16x4_t v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = min(e0 + j * 256, n_tail - 1);
        const int row = r0 + e / tq, c4 = e - (e / tq) * tq;
        v[j] = *reinterpret_cast<const bf16x4_t*>(tsrc + row * t_row + c4 * 4);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = e0 + j * 256;
        if (e < n_tail) {
          const int row = r0 + e / tq, c4 = e - (e / tq) * tq;
          *reinterpret_cast<bf16x4_t*>(Y + row * p.y_row + N + c4 * 4) = v[j];
        }
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // Weight fragment for k rows k0 .. k0+15 (this lane: k0 + half*8 .. +7) and
  // output column n0 + l32.  [K][N]: transposing reads, lane (G, q) reading k
  // row k0 + (G/2)*8 + q/4 (+4 for the high half) at 8-byte unit 4*(G%2) +
  // q%4 of the 32-column block (k & 3 = q / 4 for both halves).
  const int G = lane >> 4, q16 = lane & 15;
  const int tr_k = ((G >> 1) << 3) + (q16 >> 2);
  const int tr_u = ((G & 1) << 2) + (q16 & 3);
  const int swz = (q16 >> 2) << 3;
  auto wfrag = [&](int k0, int n0) -> bf16x8_t {
    if constexpr (kWT) {
      const int n = n0 + l32;
      const int c = ((k0 >> 3) + half) ^ (n & 15);
      return *reinterpret_cast<const bf16x8_t*>(w_s + n * K + c * 8);
    } else {
      const i16x4_t* wl = reinterpret_cast<const i16x4_t*>(w_s);  // 8-byte units
      constexpr int kU = N / 4;
      const int un = ((n0 >> 2) + tr_u) ^ swz;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (MLA_LDS i16x4_t*)(wl + (k0 + tr_k) * kU + un));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (MLA_LDS i16x4_t*)(wl + (k0 + tr_k + 4) * kU + un));
      return __builtin_bit_cast(bf16x8_t,
                                __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  f32x16_t acc[2][4];
  for (int u = 0; u < n_chunks; ++u) {
    const int pass = u / NKC, kc = u - pass * NKC;
    // Several K chunks: the next chunk's rows are loaded while this one is
    // multiplied.  One chunk (the NG column groups share it): the next pass's
    // rows are loaded after this pass, which saves the registers of a second
    // buffer.
    if constexpr (NKC > 1) {
      if (u + 1 < n_chunks) load_a(u + 1, an);
    }
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
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const bf16x8_t wop = wfrag(kc * KC + ks * 16, (ng * 4 + nb) * 32);
          // Transposed product (weight as the A operand): the accumulator
          // holds Y^T, so each lane owns one row and runs of 4 columns.
          acc[0][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wop, a[0][ks], acc[0][nb], 0, 0, 0);
          acc[1][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wop, a[1][ks], acc[1][nb], 0, 0, 0);
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
              *reinterpret_cast<bf16x8_t*>(Y + row * p.y_row + ng * 128 + c16 * 8) = v;
          }
        }
      }
    }
    if (u + 1 < n_chunks) {
      if constexpr (NKC > 1) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) a[t][ks] = an[t][ks];
      } else {
        load_a(u + 1, a);
      }
    }
  }
}

// Runs per request of head_proj_wide_kernel and rows per run (a multiple of
// 256): about 512 workgroups in all, fewer when the rows run out.  When the
// heads share their rows (x_head == 0), the run count is raised so that the
// runs fill the 8 XCDs evenly: each XCD then takes whole runs for all heads
// and reads their rows from its own L2 (a run of 2048 cached rows is 2.4 MB).
void wide_split(int n_req, int rows, int n_heads, bool shared_rows, int* rows_per_wg,
                int* chunks) {
  const int tiles = (rows + 255) / 256;
  int c = 512 / (n_heads * n_req);
  c = c < 1 ? 1 : c;
  if (shared_rows) {
    int g = n_req, h = 8;  // runs per request that make n_req * runs a multiple of 8
    while (h != 0) {
      const int r = g % h;
      g = h;
      h = r;
    }
    const int unit = 8 / g;
    c = (c + unit - 1) / unit * unit;
  }
  c = c > tiles ? tiles : c;
  const int per = (tiles + c - 1) / c;
  *rows_per_wg = per * 256;
  *chunks = (rows + *rows_per_wg - 1) / *rows_per_wg;
}

// Launch over n_req requests of up to rows_per_req rows.
template <int K, int N, bool kWT>
hipError_t launch_wide(WideArgs p, hipStream_t stream) {
  wide_split(p.n_req, p.rows_per_req, p.n_heads, p.x_head == 0, &p.rows_per_wg, &p.chunks);
  head_proj_wide_kernel<K, N, kWT><<<p.n_heads * p.n_req * p.chunks, 256, 0, stream>>>(p);
  return hipGetLastError();
}

// Row count from which the wide form replaces head_proj_mfma_kernel (and,
// above one M tile, head_proj_rows_kernel).
constexpr int kWideRows = 256;
// Rows per workgroup of head_proj_rows_kernel: absorption (128-wide rows,
// 32 KiB beside a 32 KiB weight block) and output (512-wide rows, 64 KiB
// beside a 64 KiB weight block).
constexpr int kChunkRowsQ = 128;
constexpr int kChunkRowsO = 64;
}  // namespace

hipError_t launch_absorb_q(int dtype, int batch, int n_heads, int d_head, int d_rope,
                           int d_latent, const void* q_c, const void* q_r,
                           const void* w_uk, void* q_cat, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  if (dtype == 1 && d_head == 128 && d_latent == 512 && d_rope % 4 == 0 &&
      batch >= kWideRows) {
    WideArgs p{};
    p.X = static_cast<const __bf16*>(q_c);
    p.W = static_cast<const __bf16*>(w_uk);
    p.Y = static_cast<__bf16*>(q_cat);
    p.n_req = 1;
    p.rows_per_req = batch;
    p.n_heads = n_heads;
    p.x_row = static_cast<long long>(n_heads) * d_head;
    p.x_head = d_head;
    p.y_row = static_cast<long long>(n_heads) * (d_latent + d_rope);
    p.y_head = d_latent + d_rope;
    p.tail_src = d_rope > 0 ? static_cast<const __bf16*>(q_r) : nullptr;
    p.tail_w = d_rope;
    p.tail_row = static_cast<long long>(n_heads) * d_rope;
    return launch_wide<128, 512, false>(p, stream);
  }
  if (dtype == 1 && d_head == 128 && d_latent % 128 == 0 && d_rope % 4 == 0 && batch > 32) {
    head_proj_rows_kernel<128, 128, 4, kChunkRowsQ>
        <<<head_proj_rows_grid(n_heads, d_latent, 128, batch, kChunkRowsQ), 256, 0, stream>>>(
            static_cast<const __bf16*>(q_c), static_cast<const __bf16*>(w_uk),
            static_cast<__bf16*>(q_cat), batch, n_heads, d_latent, d_latent + d_rope,
            d_rope > 0 ? static_cast<const __bf16*>(q_r) : nullptr, d_rope);
    return hipGetLastError();
  }
  if (dtype == 1 && d_head == 128 && d_latent % 128 == 0 && d_rope % 4 == 0) {
    head_proj_mfma_kernel<128, 128, 4><<<head_proj_grid(n_heads, d_latent, 128), 256, 0, stream>>>(
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

// Explicit keys and values of every cached latent row of each request (rows
// 0 .. seq_lens[b]-1 of a contiguous bf16 cache): k_c[b, i, t] = W^UK[i] c_t
// and v[b, i, t, h] = sum_c W^UV[i, c, h] c_t[c], both [B, n_h, max_len, d_h].
hipError_t launch_expand_kv(int batch, int n_heads, const CacheView& cache, const void* w_uk,
                            const void* w_uv, void* k_c, void* v, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  constexpr int kDc = 512, kDh = 128, kRowElems = 576;
  WideArgs p{};
  p.X = reinterpret_cast<const __bf16*>(cache.data);
  p.seq_lens = cache.seq_lens;
  p.n_req = batch;
  p.rows_per_req = cache.max_len;
  p.n_heads = n_heads;
  p.x_req = static_cast<long long>(cache.max_len) * kRowElems;
  p.x_row = kRowElems;
  p.x_head = 0;
  p.y_req = static_cast<long long>(n_heads) * cache.max_len * kDh;
  p.y_row = kDh;
  p.y_head = static_cast<long long>(cache.max_len) * kDh;
  p.W = static_cast<const __bf16*>(w_uk);  // [n_h][d_h][d_c]: N rows of K
  p.Y = static_cast<__bf16*>(k_c);
  hipError_t e = launch_wide<kDc, kDh, true>(p, stream);
  if (e != hipSuccess) return e;
  p.W = static_cast<const __bf16*>(w_uv);  // [n_h][d_c][d_h]: K rows of N
  p.Y = static_cast<__bf16*>(v);
  return launch_wide<kDc, kDh, false>(p, stream);
}

hipError_t launch_out_uv(int dtype, int batch, int n_heads, int d_head, int d_latent,
                         const void* out_lat, const void* w_uv, void* out,
                         hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  if (dtype == 1 && d_latent == 512 && d_head == 128 && batch >= kWideRows) {
    WideArgs p{};
    p.X = static_cast<const __bf16*>(out_lat);
    p.W = static_cast<const __bf16*>(w_uv);
    p.Y = static_cast<__bf16*>(out);
    p.n_req = 1;
    p.rows_per_req = batch;
    p.n_heads = n_heads;
    p.x_row = static_cast<long long>(n_heads) * d_latent;
    p.x_head = d_latent;
    p.y_row = static_cast<long long>(n_heads) * d_head;
    p.y_head = d_head;
    return launch_wide<512, 128, false>(p, stream);
  }
  if (dtype == 1 && d_latent == 512 && d_head % 64 == 0 && batch > 32) {
    head_proj_rows_kernel<512, 64, 2, kChunkRowsO>
        <<<head_proj_rows_grid(n_heads, d_head, 64, batch, kChunkRowsO), 256, 0, stream>>>(
            static_cast<const __bf16*>(out_lat), static_cast<const __bf16*>(w_uv),
            static_cast<__bf16*>(out), batch, n_heads, d_head, d_head, nullptr, 0);
    return hipGetLastError();
  }
  if (dtype == 1 && d_latent == 512 && d_head % 64 == 0) {
    head_proj_mfma_kernel<512, 64, 2><<<head_proj_grid(n_heads, d_head, 64), 256, 0, stream>>>(
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
