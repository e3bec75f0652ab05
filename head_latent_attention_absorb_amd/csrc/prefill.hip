// A chunk of new tokens per request in the primary (unabsorbed) form: the
// cached latents of each request are up-projected once to per-head keys and
// values (zeeklog, equations 10-11; the explicit products run in
// head_proj_wide_kernel, see launch_expand_kv), every key carries the shared
// RoPE part k^R straight from the cache row (ai-library "Multi-Head Latent
// Attention"; V3 read-through section 2.3, k = [k_c; k_r]), and the chunk's
// queries attend causally (zeeklog MHA equation, positions 1..t):
//
//   s[j, t] = scale * ([q^C_j ; q^R_j] . [k^C_t ; k^R_t]),   t <= pos(j)
//   o_j     = sum_t softmax_t(s[j, :]) v_t                   [d_h]
//
// With a long chunk this costs (d_h + d_h^R) + d_h multiply-adds per query,
// key and head plus the expansion shared by all queries, against
// (d_c + d_h^R) + d_c in the absorbed form (V2 read-through, section 2.3:
// absorption pays at decode).
//
// Kernel: one workgroup per (request, head, block of 256 queries), 8 waves
// of 32 queries (two per SIMD: one's softmax overlaps the other's products).
// Keys and values stream through a three-stage LDS ring in tiles of 64 tokens
// (k^C 16 KiB, k^R 8 KiB, v 16 KiB), loaded with direct loads two tiles
// ahead: the tiles in flight, not the products, bound the kernel at two
// stages, and 256 queries per tile halve the bytes per product of 128.  Both products are computed transposed so that a lane owns one query
// throughout:
//   S^T = K Q^T   (A: key rows from LDS, B: the wave's queries in registers)
//   O^T += V^T P^T (A: value columns through the transposing LDS read, B: the
//                   probabilities straight from the S^T accumulator)
// which keeps the online softmax's max, sum and rescale per lane.  The
// tokens of a 32-token block appear in the PV contraction in the order the
// S^T accumulator holds them (for lane half h: 4h..4h+3, 8+4h..8+4h+3, then
// the same +16), and the value read addresses rows in that order.

#include <math.h>

#include "device_common.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kDh = 128;        // d_h (content and value width)
constexpr int kDr = 64;         // d_h^R
constexpr int kDc = 512;        // d_c
constexpr int kRow = kDc + kDr; // cache row (elements)
constexpr int kQT = 1;          // 32-query tiles per wave
constexpr float kLazy = 8.f;    // log2 headroom before the running max moves
constexpr int kWaves = 8;
constexpr int kQBlock = kWaves * 32 * kQT;  // queries per workgroup
constexpr int kStages = 3;
constexpr int kTile = 64;       // keys per tile
constexpr int kKcBytes = kTile * kDh * 2;   // 16 KiB
constexpr int kKrBytes = kTile * kDr * 2;   // 8 KiB
constexpr int kVBytes = kTile * kDh * 2;    // 16 KiB
constexpr int kStageBytes = kKcBytes + kKrBytes + kVBytes;
constexpr int kLoadsPerWave = kStageBytes / 1024 / kWaves;  // 1 KiB per wave instruction
static_assert(kStageBytes % (1024 * kWaves) == 0, "");

struct PrefillParams {
  const __bf16* q_c;     // [B, C, n_h, d_h]
  const __bf16* q_r;     // [B, C, n_h, d_h^R]
  const __bf16* k_c;     // [B, n_h, max_len, d_h]
  const __bf16* v;       // [B, n_h, max_len, d_h]
  const __bf16* cache;   // [B, max_len, d_c + d_h^R] (k^R = row[d_c:])
  const int32_t* seq_lens;
  __bf16* out;           // [B, C, n_h, d_h]
  float* lse;            // [B, C, n_h] or nullptr
  int q_len, n_heads, max_len, q_blocks;
  float scale_log2;
};

template <int kN>
__device__ __forceinline__ void wait_vm() {
  static_assert(kN >= 0 && kN < 64, "");
  __builtin_amdgcn_s_waitcnt((kN & 15) | ((kN >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// kPosScale (softmax scale > 0): the max is taken over the raw scores and the
// scale is folded into the exponent's fused multiply-add, saving a multiply
// per score.
template <bool kPosScale>
__global__ __launch_bounds__(kWaves * 64) void prefill_attn_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kStages * kStageBytes];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  // Workgroup -> (request, head, query block).  Workgroup x runs on XCD
  // x % 8: with (requests x heads) % 8 == 0 the query blocks of one (request,
  // head) go to one XCD, adjacent in its order, so they share the head's key
  // and value tiles through that XCD's L2 (and its neighbours there, heads of
  // the same request, share the k^R tiles).
  const int n_bh = gridDim.x / p.q_blocks;
  int qb, bh;
  if (n_bh % 8 == 0) {
    bh = (blockIdx.x / (8 * p.q_blocks)) * 8 + (blockIdx.x & 7);
    qb = (blockIdx.x >> 3) % p.q_blocks;
  } else {
    qb = blockIdx.x % p.q_blocks;
    bh = blockIdx.x / p.q_blocks;
  }
  const int i = bh % p.n_heads;
  const int b = bh / p.n_heads;
  const int len = p.seq_lens[b];
  const int C = p.q_len;
  // Position of query j: len - C + j.  Queries of this workgroup and wave.
  const int q_first = qb * kQBlock;
  const int q_last = min(C, q_first + kQBlock) - 1;
  const int pos_max = len - C + q_last;                 // workgroup's last position
  const int nt = pos_max < 0 ? 0 : pos_max / kTile + 1;
  const int qw0 = q_first + wave * 32 * kQT;
  // This wave's last position (-1: no query of the chunk in this wave).
  const int pos_w = qw0 > q_last ? -1 : len - C + min(q_last, qw0 + 32 * kQT - 1);

  // Queries as B operands: lane (query qw0 + qt*32 + l32, half) holds d =
  // ks*16 + half*8 .. +7 of [q^C | q^R] for ks < 12.
  bf16x8_t qf[kQT][12];
  int my_pos[kQT];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int q_idx = qw0 + qt * 32 + l32;
    my_pos[qt] = q_idx <= q_last ? len - C + q_idx : -1;
    const size_t qrow = (static_cast<size_t>(b) * C + min(q_idx, q_last)) * p.n_heads + i;
    const __bf16* qc = p.q_c + qrow * kDh + half * 8;
    const __bf16* qr = p.q_r + qrow * kDr + half * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[qt][ks] = *reinterpret_cast<const bf16x8_t*>(qc + ks * 16);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[qt][8 + ks] = *reinterpret_cast<const bf16x8_t*>(qr + ks * 16);
  }
  // Wait for the queries here, before any tile load is in flight: the
  // compiler cannot see the direct loads, and a query load it still counts
  // as pending inside the loop would make it wait for every outstanding load
  // (the ring's prefetches included) at each tile.
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));  // vmcnt(0)
  // A tile needs no mask when all its keys precede the first position of a
  // query tile whose queries all lie in the chunk.
  int pos_unmasked[kQT];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int q0 = qw0 + qt * 32;
    pos_unmasked[qt] = q0 + 31 <= q_last ? len - C + q0 : -1;
  }

  // Tile loads: instruction j of the stage (wave j % kWaves issues it) fills
  // 1 KiB: j < 16 the k^C rows (16 units of 16 bytes per 256-byte row, unit
  // c at c ^ (row & 15)), j < 24 the k^R rows (8 units per 128-byte row, two
  // rows per 256 bytes of banks, unit c at c ^ ((row >> 1) & 7)), else the
  // value rows (16 units per row, unit v at
  // v ^ ((row & 3) << 2), i.e. 8-byte unit u at u ^ ((row & 3) << 3)).  Rows
  // past the length repeat row len - 1 (finite values, masked to weight 0).
  const __bf16* kc_base = p.k_c + (static_cast<size_t>(b) * p.n_heads + i) * p.max_len * kDh;
  const __bf16* v_base = p.v + (static_cast<size_t>(b) * p.n_heads + i) * p.max_len * kDh;
  const __bf16* cr_base = p.cache + static_cast<size_t>(b) * p.max_len * kRow + kDc;
  const unsigned ring_base =
      static_cast<unsigned>(reinterpret_cast<uintptr_t>((MLA_LDS uint8_t*)ring));
  auto issue_tile = [&](int t, int stage) {
    const unsigned sbase = ring_base + stage * kStageBytes;
#pragma unroll
    for (int n = 0; n < kLoadsPerWave; ++n) {
      const int j = wave + n * kWaves;
      const void* src;
      if (j < 16) {
        const int unit = j * 64 + lane, r = unit >> 4, c = unit & 15;
        const int row = min(t * kTile + r, len - 1);
        src = kc_base + static_cast<size_t>(row) * kDh + ((c ^ (r & 15)) << 3);
      } else if (j < 24) {
        const int unit = (j - 16) * 64 + lane, r = unit >> 3, c = unit & 7;
        const int row = min(t * kTile + r, len - 1);
        src = cr_base + static_cast<size_t>(row) * kRow + ((c ^ ((r >> 1) & 7)) << 3);
      } else {
        const int unit = (j - 24) * 64 + lane, r = unit >> 4, c = unit & 15;
        const int row = min(t * kTile + r, len - 1);
        src = v_base + static_cast<size_t>(row) * kDh + ((c ^ ((r & 3) << 2)) << 3);
      }
      load_to_lds16(src, sbase + j * 1024);
    }
  };

  f32x16_t o[kQT][4];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[qt][db][e] = 0.f;
  float m[kQT], l[kQT];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    m[qt] = -INFINITY;
    l[qt] = 0.f;
  }

  // Value read coordinates (transposing read): lane (G, q) addresses token
  // row k0 + (G/2)*4 + q/4 (+8 for the second half of the fragment) at 8-byte
  // unit 4*(G%2) + q%4 of the 32-column block; row & 3 = q / 4.
  const int G = lane >> 4, q16 = lane & 15;
  const int tr_k = ((G >> 1) << 2) + (q16 >> 2);
  const int tr_u = ((G & 1) << 2) + (q16 & 3);
  const int swz = (q16 >> 2) << 3;

  // Ring: tile t in stage t % 3.  Iteration t waits for tile t, and after
  // the barrier (every wave is past tile t - 1) refills tile t - 1's stage
  // with tile t + 2.
  if (nt > 0) issue_tile(0, 0);
  if (nt > 1) issue_tile(1, 1);
  for (int t = 0; t < nt; ++t) {
    const int stage = t % kStages;
    if (t + 1 < nt)
      wait_vm<kLoadsPerWave>();
    else
      wait_vm<0>();
    __syncthreads();
    if (t + 2 < nt) issue_tile(t + 2, (t + 2) % kStages);
    const uint8_t* st = ring + stage * kStageBytes;
    if (t * kTile <= pos_w) {
      const i16x4_t* vl = reinterpret_cast<const i16x4_t*>(st + kKcBytes + kKrBytes);
      // The tile's two 32-token blocks, one online-softmax update each.
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        if (t * kTile + tb * 32 > pos_w) break;
        // S^T for the block and each query tile: lane (query l32, half) gets
        // token tb*32 + (e/4)*8 + half*4 + e%4 in register e.  Each key
        // fragment feeds every query tile.
        f32x16_t s[kQT];
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt)
#pragma unroll
          for (int e = 0; e < 16; ++e) s[qt][e] = 0.f;
        const int r = tb * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < 12; ++ks) {
          bf16x8_t kf;
          if (ks < 8)
            kf = *reinterpret_cast<const bf16x8_t*>(st + r * 256 + (((ks * 2 + half) ^ (r & 15)) << 4));
          else
            kf = *reinterpret_cast<const bf16x8_t*>(st + kKcBytes + r * 128 +
                                                    ((((ks - 8) * 2 + half) ^ ((r >> 1) & 7)) << 4));
#pragma unroll
          for (int qt = 0; qt < kQT; ++qt)
            s[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qt][ks], s[qt], 0, 0, 0);
        }
        // Causal mask (blocks that reach the diagonal), running max and the
        // probabilities (base 2).
        bf16x8_t pf[kQT][2];
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt) {
          const int tok0 = t * kTile + tb * 32;
          const bool masked = tok0 + 31 > pos_unmasked[qt];
          float mx = -INFINITY;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int tok = tok0 + (e >> 2) * 8 + half * 4 + (e & 3);
            float x = kPosScale ? s[qt][e] : s[qt][e] * p.scale_log2;
            if (masked) x = tok <= my_pos[qt] ? x : -INFINITY;
            s[qt][e] = x;
            mx = fmaxf(mx, x);
          }
          mx = halves_max(mx);
          if constexpr (kPosScale) mx *= p.scale_log2;  // -inf stays -inf
          // Lazy rescale: the reference max m (exponent base of l and o)
          // moves only when a score exceeds it by more than kLazy (so every
          // probability stays below 2^kLazy), and the accumulators are
          // rescaled only when some lane's reference moved.
          const bool move = mx > m[qt] + kLazy;
          if (__builtin_amdgcn_ballot_w64(move) != 0) {
            const float m_new = move ? mx : m[qt];
            const float alpha = move ? __builtin_amdgcn_exp2f(m[qt] - m_new) : 1.f;  // 0 from -inf
            m[qt] = m_new;
            l[qt] *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
              for (int e = 0; e < 16; ++e) o[qt][db][e] *= alpha;
          }
          const float m_use = m[qt] == -INFINITY ? 0.f : m[qt];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float pe = __builtin_amdgcn_exp2f(
                  kPosScale ? fmaf(s[qt][kk * 8 + e], p.scale_log2, -m_use)
                            : s[qt][kk * 8 + e] - m_use);
              l[qt] += pe;
              pf[qt][kk][e] = static_cast<__bf16>(pe);
            }
        }
        // O^T += V^T P^T over the block's two 16-token steps; each value
        // fragment feeds every query tile.
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int k0 = tb * 32 + kk * 16;
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const int un = ((db * 8) + tr_u) ^ swz;
            const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (MLA_LDS i16x4_t*)(vl + (k0 + tr_k) * 32 + un));
            const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (MLA_LDS i16x4_t*)(vl + (k0 + 8 + tr_k) * 32 + un));
            const bf16x8_t vf = __builtin_bit_cast(
                bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int qt = 0; qt < kQT; ++qt)
              o[qt][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qt][kk], o[qt][db], 0, 0, 0);
          }
        }
      }
    }
  }

  // Both halves saw half of every tile's tokens.
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const float lt = halves_sum(l[qt]);
    const int q_idx = qw0 + qt * 32 + l32;
    if (q_idx > q_last) continue;
    const float inv_l = lt > 0.f ? 1.f / lt : 0.f;
    const size_t orow = (static_cast<size_t>(b) * C + q_idx) * p.n_heads + i;
    // Register e of block db: d = db*32 + (e/4)*8 + half*4 + e%4.
    __bf16* dst = p.out + orow * kDh + half * 4;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4_t v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = static_cast<__bf16>(o[qt][db][g * 4 + e] * inv_l);
        *reinterpret_cast<bf16x4_t*>(dst + db * 32 + g * 8) = v4;
      }
    if (p.lse != nullptr && half == 0)
      p.lse[orow] = lt > 0.f ? (m[qt] + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

}  // namespace

bool prefill_supported(int dtype, int n_heads, int d_head, int d_latent, int d_rope) {
  return dtype == 1 && n_heads > 0 && d_head == kDh && d_latent == kDc && d_rope == kDr;
}

hipError_t launch_prefill_attn(int batch, int q_len, int n_heads, const CacheView& cache,
                               const void* q_c, const void* q_r, const void* k_c,
                               const void* v, float softmax_scale, void* out, float* lse,
                               hipStream_t stream) {
  if (batch == 0 || q_len == 0) return hipSuccess;
  PrefillParams p;
  p.q_c = static_cast<const __bf16*>(q_c);
  p.q_r = static_cast<const __bf16*>(q_r);
  p.k_c = static_cast<const __bf16*>(k_c);
  p.v = static_cast<const __bf16*>(v);
  p.cache = reinterpret_cast<const __bf16*>(cache.data);
  p.seq_lens = cache.seq_lens;
  p.out = static_cast<__bf16*>(out);
  p.lse = lse;
  p.q_len = q_len;
  p.n_heads = n_heads;
  p.max_len = cache.max_len;
  p.q_blocks = (q_len + kQBlock - 1) / kQBlock;
  p.scale_log2 = softmax_scale * kLog2e;
  const long long grid = static_cast<long long>(batch) * n_heads * p.q_blocks;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (p.scale_log2 > 0.f)
    prefill_attn_kernel<true><<<static_cast<unsigned>(grid), kWaves * 64, 0, stream>>>(p);
  else
    prefill_attn_kernel<false><<<static_cast<unsigned>(grid), kWaves * 64, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace mla
