// K2: bf16 MFMA split-KV latent decode for gfx950 (d_latent 512, d_rope 64).
//
// What it computes, per request b, head i and split-KV partition [t0, t1):
//   s_j   = scale * q_cat[b,i,:] . row_j[0:576]        (absorbed content score
//           plus the decoupled RoPE score against the one cached row,
//           DeepSeek-V2 read-through, 2kiu.com/news/6085339, sections 2.3-2.4)
//   O_i   = sum_j softmax_j(s) * row_j[0:512]           (weighted sum in latent
//           space, section 2.3; the cached latent serves as both K and V)
// written as a partial normalised by its own softmax sum plus its log-sum-exp.
//
// Mapping onto CDNA4:
//  * One workgroup = 4 waves (one per SIMD) = (request, 64 heads, partition).
//    Wave (hb, hf): hb picks a 32-head block; hf picks half of the score
//    contraction (K = 288 of 576) and half of the latent output (256 of 512).
//    All four waves consume the same 32-token tile per step.
//  * Tiles move HBM -> LDS with 16-byte direct-to-LDS loads (no VGPR
//    staging) through a 3-stage ring, two tiles in flight.  A 32-token tile is
//    stored column-group major: the 576-element row is cut into 9 groups of 64
//    elements (128 B); group g of token n sits at ((g * 32 + n) * 128), its
//    eight 16-byte chunks XOR-swizzled by (n & 7) so MFMA operand reads are
//    conflict free.  A load instruction fills 8 tokens x one group: each lane
//    owns one token row per tile and every global access is a whole 128-byte
//    segment.
//  * Scores are computed transposed, S^T[token, head] = tile . Q^T, with
//    v_mfma_f32_32x32x16_bf16: the tile is the A operand (LDS), the query the
//    B operand (registers for the whole kernel).  The two half-K partial
//    scores of a head block are summed through LDS (same order in both waves,
//    so both hold bitwise identical scores and softmax state).  In the
//    accumulator layout each lane owns one head, so the softmax max and sum
//    need one cross-lane step (lane l <-> l^32).
//  * The probabilities stay in registers: the S^T accumulator converted to
//    bf16 is exactly the B operand of O^T[latent, head] += V^T . P^T, with the
//    token (K) index permuted identically on both operands.  O^T is 8
//    accumulator tiles (128 registers per lane).
//  * The running max only moves when a tile's max exceeds it by more than 8
//    (exp2 units), so the accumulator rescale runs rarely and p <= 256.

#include "device_common.h"

namespace mla {
namespace {

constexpr int kRow = 576;             // d_latent + d_rope
constexpr int kRowBytes = kRow * 2;
constexpr int kTile = 32;             // tokens per step
constexpr int kTileBytes = kTile * kRowBytes;        // 36864
constexpr int kStages = 4;            // LDS ring depth; kStages - 1 tiles in flight
constexpr int kGroups = kRow / 64;    // 9 column groups of 128 bytes
constexpr int kHalfKSteps = kRow / 16 / 2;           // 18 score K-steps per wave
constexpr int kHalfCBlocks = 512 / 32 / 2;           // 8 latent blocks per wave
constexpr int kXchBytes = 2 * 2 * 64 * 16 * 4;       // pair x wave x fragment
constexpr int kLdsBytes = kStages * kTileBytes + kXchBytes;
static_assert(kStages == 4, "the main loop is unrolled over exactly four stage arrays");
constexpr float kRescaleThreshold = 8.f;             // log2 units

static_assert(kTileBytes == 4 * kGroups * 1024, "each wave issues kGroups loads per tile");
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
static_assert(kMfmaHeadsPerGroup == 64 && kMfmaTokenGranule == kTile, "");

// s_waitcnt immediate: wait until at most `n` vector-memory loads are
// outstanding; expcnt and lgkmcnt are left at their maxima (no wait).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

struct MfmaParams {
  const uint16_t* q_cat;  // [B, n_heads, 576] bf16
  CacheView cache;
  int n_heads, split_tokens, num_splits, head_groups, work_items;
  float scale_log2;       // softmax scale * log2(e)
  float* part_o;
  float* part_lse;
};

// 16-byte direct-to-LDS load: every lane reads 16 bytes at `src` and writes
// them at LDS byte address lds_base + 16 * lane (lds_base wave-uniform, in M0).
// Issued as inline asm so the compiler's wait insertion does not see it: it
// cannot tell the ring stages apart and would otherwise drain every
// outstanding load before each LDS read.  The kernel waits for these loads
// itself (s_waitcnt vmcnt) before the barrier that publishes a stage.  The
// instruction has no result registers; its address is read at issue.  No
// other instruction in this kernel uses M0.
__device__ __forceinline__ void load_to_lds16(const void* src, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}

__device__ __forceinline__ unsigned lds_address(const void* p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>((MLA_LDS const void*)p));
}

// LDS byte offset (within a tile) of 16-byte chunk `chunk` (0..71) of token `n`.
__device__ __forceinline__ int swz(int n, int chunk) {
  return (((chunk >> 3) * kTile + n) << 7) + (((chunk & 7) ^ (n & 7)) << 4);
}

template <bool kPaged>
__global__ __launch_bounds__(256, 1) void decode_mfma_kernel(MfmaParams p) {
  // Four ring stages (3 tiles in flight) plus the score exchange fill the
  // 160 KiB of LDS exactly.  The stages are distinct arrays and the loop is
  // unrolled over them, so every stage offset is a compile-time constant.
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage2[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t stage3[kTileBytes];
  __shared__ __attribute__((aligned(1024))) float xch[kXchBytes / 4];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hb = wave >> 1, hf = wave & 1;
  const int half = lane >> 5, l32 = lane & 31;

  // XCD-aware work mapping: workgroup x runs on XCD x % 8; give every XCD a
  // contiguous range of work ids so the head groups of one partition
  // (adjacent ids) share that XCD's L2.
  const int nwg = gridDim.x;
  const int work = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  if (work >= p.work_items) return;
  const int g = work % p.head_groups;
  const int rest = work / p.head_groups;
  const int s = rest % p.num_splits;
  const int b = rest / p.num_splits;

  const int len = p.cache.seq_lens[b];
  const int t0 = s * p.split_tokens;
  const int t1 = min(t0 + p.split_tokens, len);
  if (t0 >= t1) return;  // the combine never reads partitions past the length

  const int hblock = g * 2 + hb;
  const int head = hblock * 32 + l32;

  // Query as the B operand: lane holds head `head`, K slots half*8..+7 of
  // each of this wave's 18 K-steps.
  bf16x8_t qf[kHalfKSteps];
  {
    const uint16_t* qrow = p.q_cat + (static_cast<size_t>(b) * p.n_heads + head) * kRow +
                           hf * (kRow / 2) + half * 8;
#pragma unroll
    for (int ks = 0; ks < kHalfKSteps; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16);
  }

  f32x16_t acc[kHalfCBlocks];
#pragma unroll
  for (int cb = 0; cb < kHalfCBlocks; ++cb)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[cb][v] = 0.f;
  float m = -INFINITY, l = 0.f;

  // Loader: wave w fills token octet w of every column group.  This lane's
  // token is w*8 + lane/8 and it fills LDS position lane%8 of that token's
  // group, which holds logical chunk (lane%8) ^ (token & 7).  Rows past the
  // partition are clamped to t1 - 1: never read past the request, and their
  // probabilities are forced to 0.
  const int n_load = wave * 8 + (lane >> 3);
  const int chunk_off = ((lane & 7) ^ (n_load & 7)) * 16;
  const uint8_t* req_base =
      kPaged ? p.cache.data
             : p.cache.data + static_cast<size_t>(b) * p.cache.max_len * kRowBytes;
  // Paged cache: lane j holds the physical id of the partition's j-th page
  // (at most 64 pages, which the planner guarantees), fetched once here.  A
  // wave's 8 tokens of a tile are 8-aligned, so with page_size % 8 == 0 they
  // share one page, picked per tile with readlane: no memory access, and no
  // load the compiler would have to wait for inside the loop.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  int page_of_lane = 0, first_page = 0;
  if constexpr (kPaged) {
    first_page = t0 / p.cache.page_size;
    const int npages = (t1 - 1) / p.cache.page_size - first_page + 1;
    if (lane < npages)
      page_of_lane = p.cache.page_table[static_cast<size_t>(b) * p.cache.max_pages +
                                        first_page + lane];
  }
  auto issue_tile = [&](uint8_t* stage, int tile_t0) {
    const int t = min(tile_t0 + n_load, t1 - 1);
    const uint8_t* src;
    if constexpr (kPaged) {
      const int t_first = min(tile_t0 + wave_u * 8, t1 - 1);
      const int page =
          __builtin_amdgcn_readlane(page_of_lane, t_first / p.cache.page_size - first_page);
      src = req_base + (static_cast<size_t>(page) * p.cache.page_size + t % p.cache.page_size) *
                           kRowBytes;
    } else {
      src = req_base + static_cast<size_t>(t) * kRowBytes;
    }
    src += chunk_off;
    const unsigned dst = lds_address(stage) + wave * 1024;
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) load_to_lds16(src + gi * 128, dst + gi * 4096);
  };

  // Per-lane coordinates of the transposing reads of the PV operand.
  const int tr_tok = (half << 2) + ((lane >> 2) & 3);
  const int tr_col = (((lane >> 4) & 1) << 4) + ((lane & 3) << 2);
  const int ntiles = (t1 - t0 + kTile - 1) / kTile;
  // Prologue: tiles 0..2 in flight, then one wait (visible to the compiler)
  // for them and for the query fragments, which every step needs at once.
  // From here on the compiler sees no outstanding loads, and the tile loads
  // are governed only by the waits below.  Every step issues exactly one
  // tile (past the last tile they re-read the partition's last row into a
  // stage that is never read again), so "this wave's loads of tile it have
  // landed" is always vmcnt(18): the two younger tiles may stay in flight.
  issue_tile(stage0, t0);
  issue_tile(stage1, t0 + kTile);
  issue_tile(stage2, t0 + 2 * kTile);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // One step: tile `it` is in `tile`; tile it+3 is loaded into `next3`.
  auto step = [&](int it, const uint8_t* tile, uint8_t* next3) {
    // Wait for this wave's loads of tile `it` (those of tile it+1 may stay in
    // flight), then for everyone's.  A raw s_barrier, not __syncthreads(): the
    // latter also waits for every outstanding global load and would drain the
    // prefetch at each barrier.  The compiler fence keeps LDS accesses on
    // their side of the barrier.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kGroups));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // Everyone is past step it-1, whose stage is `next3`: refill it.
    issue_tile(next3, t0 + (it + 3) * kTile);

    const int nvalid = t1 - (t0 + it * kTile);

    // Per-lane LDS offsets.  Score operand of K-step ks: swz(l32, chunk) with
    // chunk = 36 hf + 2 ks + half, which equals qoff[ks % 4] + (ks / 4) * 4096.
    // PV operand of latent block cb, K-step kk, read lo/hi:
    // voff[cb % 2] + (cb / 2) * 4096 + kk * 2048 + hi * 1024.  The empty asm
    // keeps these few offsets from being hoisted out of the loop per stage
    // (three stages x 50 addresses would not fit in registers).
    int qoff[4], voff[2];
#pragma unroll
    for (int q = 0; q < 4; ++q) qoff[q] = swz(l32, (hf * kHalfKSteps + q) * 2 + half);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = (hf * kHalfCBlocks + q) * 32 + tr_col;
      voff[q] = swz(tr_tok, c >> 3) + (c & 7) * 2;
    }
    asm volatile("" : "+v"(qoff[0]), "+v"(qoff[1]), "+v"(qoff[2]), "+v"(qoff[3]),
                 "+v"(voff[0]), "+v"(voff[1]));

    // Partial S^T[token, head] over this wave's half of K.  All 18 operand
    // reads are issued before the MFMA chain so LDS latency overlaps it.
    bf16x8_t ta[kHalfKSteps];
#pragma unroll
    for (int ks = 0; ks < kHalfKSteps; ++ks)
      ta[ks] = *reinterpret_cast<const bf16x8_t*>(tile + qoff[ks & 3] + (ks >> 2) * 4096);
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMA chain
    f32x16_t sacc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kHalfKSteps; ++ks)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[ks], qf[ks], sacc, 0, 0, 0);

    // Sum the two half-K partials of this head block through LDS.  Both waves
    // add (K-half 0) + (K-half 1) in that order, so their scores match bitwise.
    // One buffer serves every step: each wave consumes its partner's values
    // (softmax below) before it reaches the next step's barrier, and nobody
    // rewrites the buffer before passing that barrier.
    float* xw = xch + hb * 2 * 1024;  // [wave of pair][reg][lane]
#pragma unroll
    for (int v = 0; v < 16; v += 4)
      *reinterpret_cast<f32x4_t*>(xw + hf * 1024 + v * 64 + lane * 4) =
          f32x4_t{sacc[v], sacc[v + 1], sacc[v + 2], sacc[v + 3]};
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the exchange writes are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // O^T[latent, head] += V^T[latent, token] . P^T[token, head] over this
    // wave's 256 latent columns.  K slot j of lane half `half` in K-step kk is
    // token kk*16 + (j/4)*8 + half*4 + j%4, matching the P^T registers below.
    // The A operand (lane: one latent column, 8 tokens) comes from two
    // transposing LDS reads: within each 16-lane group, ds_read_b64_tr_b16
    // gives lane i the (i%4)-th element of the 8-byte chunk addressed by lane
    // 4j + i/4, for j = 0..3.  So lane (group G, index r) addresses token
    // kk*16 + {0,8} + (G/2)*4 + r/4 at latent column 16*(G%2) + 4*(r%4).
    // The first half of these reads is issued before the softmax math, which
    // then runs while they are in flight.
    bf16x8_t va[kHalfCBlocks][2];
    auto read_v = [&](int cb) {
      const uint8_t* vb = tile + voff[cb & 1] + (cb >> 1) * 4096;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const i16x4_t lo =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4_t*)(vb + kk * 2048));
        const i16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS i16x4_t*)(vb + kk * 2048 + 1024));
        va[cb][kk] =
            __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
#pragma unroll
    for (int cb = 0; cb < kHalfCBlocks / 2; ++cb) read_v(cb);
    __builtin_amdgcn_sched_barrier(0);

    float sv[16];
#pragma unroll
    for (int v = 0; v < 16; v += 4) {
      const f32x4_t o =
          *reinterpret_cast<const f32x4_t*>(xw + (hf ^ 1) * 1024 + v * 64 + lane * 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[v + r] = hf == 0 ? sacc[v + r] + o[r] : o[r] + sacc[v + r];
    }

    // Accumulator row of register v in this lane: token (v/4)*8 + half*4 + v%4.
    float tmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int n = (v >> 2) * 8 + half * 4 + (v & 3);
      sv[v] = n < nvalid ? sv[v] * p.scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, sv[v]);
    }
    tmax = halves_max(tmax);

    if (__builtin_amdgcn_ballot_w64(tmax > m + kRescaleThreshold) != 0) {
      const float m_new = fmaxf(m, tmax);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 on the first tile
      // Scale the accumulators in place in the accumulation registers: going
      // through inline asm keeps the compiler from giving all accumulator
      // values a second home in ordinary VGPRs.  The MFMAs that last wrote
      // them retired a whole score pass ago; the s_nops cover the
      // MFMA-to-read wait states regardless.
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory");
#pragma unroll
      for (int cb = 0; cb < kHalfCBlocks; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = acc[cb][v], tmp;
          asm volatile(
              "v_accvgpr_read_b32 %1, %0\n\t"
              "v_mul_f32 %1, %1, %2\n\t"
              "v_accvgpr_write_b32 %0, %1"
              : "+a"(x), "=&v"(tmp)
              : "v"(alpha));
          acc[cb][v] = x;
        }
      l *= alpha;
      m = m_new;
    }

    bf16x8_t pb[2];
    float psum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float pv = __builtin_amdgcn_exp2f(sv[v] - m);
      psum += pv;
      pb[v >> 3][v & 7] = static_cast<__bf16>(pv);
    }
    l += psum;

#pragma unroll
    for (int cb = kHalfCBlocks / 2; cb < kHalfCBlocks; ++cb) read_v(cb);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int cb = 0; cb < kHalfCBlocks; ++cb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[cb][kk], pb[kk], acc[cb], 0, 0, 0);
  };

  for (int it = 0; it < ntiles; it += kStages) {
    step(it, stage0, stage3);
    if (it + 1 < ntiles) step(it + 1, stage1, stage0);
    if (it + 2 < ntiles) step(it + 2, stage2, stage1);
    if (it + 3 < ntiles) step(it + 3, stage3, stage2);
  }
  // The trailing loads must land before the workgroup's LDS is released.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // Softmax sum over both lane halves (each half saw half of the tokens).
  l = halves_sum(l);
  const float inv = 1.f / l;
  float* dst = p.part_o +
               ((static_cast<size_t>(b) * p.num_splits + s) * (p.n_heads / 32) + hblock) * 16384 +
               hf * kHalfCBlocks * 1024 + lane;
#pragma unroll
  for (int cb = 0; cb < kHalfCBlocks; ++cb)
#pragma unroll
    for (int v = 0; v < 16; ++v) dst[(cb * 16 + v) * 64] = acc[cb][v] * inv;
  if (hf == 0 && half == 0)
    p.part_lse[(static_cast<size_t>(b) * p.num_splits + s) * p.n_heads + head] =
        (m + __log2f(l)) * kLn2;
}

}  // namespace

hipError_t launch_partials_mfma(const DecodeArgs& a) {
  if (a.batch == 0) return hipSuccess;
  MfmaParams p;
  p.q_cat = static_cast<const uint16_t*>(a.q_cat);
  p.cache = a.cache;
  p.n_heads = a.n_heads;
  p.split_tokens = a.split_tokens;
  p.num_splits = a.num_splits;
  p.head_groups = a.head_groups;
  p.work_items = a.batch * a.num_splits * a.head_groups;
  p.scale_log2 = a.softmax_scale * kLog2e;
  p.part_o = a.part_o;
  p.part_lse = a.part_lse;
  const int grid = (p.work_items + 7) / 8 * 8;  // multiple of the 8 XCDs
  if (a.cache.page_table != nullptr)
    decode_mfma_kernel<true><<<grid, 256, 0, a.stream>>>(p);
  else
    decode_mfma_kernel<false><<<grid, 256, 0, a.stream>>>(p);
  return hipGetLastError();
}

}  // namespace mla
