// K2: bf16 MFMA split-KV latent decode for gfx950 (d_latent 512, d_rope 64).
//
// What it computes, per request b, head i and split-KV partition [t0, t1):
//   s_j   = scale * q_cat[b,i,:] . row_j[0:576]        (absorbed content score
//           plus the decoupled RoPE score against the one cached row,
//           DeepSeek-V2 read-through, 2kiu.com/news/6085339, sections 2.3-2.4)
//   O_i   = sum_j softmax_j(s) * row_j[0:512]           (weighted sum in latent
//           space, section 2.3; the cached latent serves as both K and V)
// written as a bf16 partial sum_j 2^(scale*log2(e)*s_j - m) row_j (not divided by
// its softmax sum: the combine folds both factors into one weight) with the
// fp32 pair (log2 sum_j 2^(scale*log2(e)*s_j), m).
//
// Mapping onto CDNA4:
//  * One workgroup = 4 waves (one per SIMD) = (request, 128 heads, partition).
//    Wave w owns 32 heads over the whole score contraction (K = 576) and the
//    whole latent output (512): 144 registers of query fragments and 256
//    accumulator registers per lane.  Every cached token is read from HBM by
//    exactly one workgroup.
//  * Tiles move HBM -> LDS with 16-byte direct-to-LDS loads (no VGPR
//    staging) through a 4-stage ring.  A 32-token tile is stored column-group
//    major: the 576-element row is cut into 9 groups of 64 elements (128 B);
//    group g of token n sits at ((g * 32 + n) * 128), its eight 16-byte chunks
//    XOR-swizzled by a key of n (swz_key) so that both MFMA operand reads are
//    free of bank conflicts on the 64-bank LDS.  A load
//    instruction fills 8 tokens x one group: each lane owns one token row per
//    tile and every global access is a whole 128-byte segment.
//  * Scores are computed transposed, S^T[token, head] = tile . Q^T, with
//    v_mfma_f32_32x32x16_bf16: the tile is the A operand (LDS), the query the
//    B operand (registers for the whole kernel).  In the accumulator layout
//    each lane owns one head, so the softmax max and sum need one cross-lane
//    step (lane l <-> l^32).
//  * The probabilities stay in registers: the S^T accumulator converted to
//    bf16 is exactly the B operand of O^T[latent, head] += V^T . P^T, with the
//    token (K) index permuted identically on both operands.
//  * Software pipeline, one wave per SIMD: step t issues the softmax
//    arithmetic of tile t between the score MFMAs of tile t+1, so the matrix
//    pipe has independent work while that arithmetic runs, then the PV product
//    of tile t.  Tiles t and t+1 are resident in the ring during step t,
//    tiles t+2 and t+3 in flight.
//  * The running max only moves when a tile's max exceeds it by more than 8
//    (exp2 units), so the accumulator rescale runs rarely and p <= 256.

#include <type_traits>
#include <utility>

#include "device_common.h"

namespace mla {
namespace {

constexpr int kRow = 576;             // d_latent + d_rope
constexpr int kRowBytes = kRow * 2;
constexpr int kTile = 32;             // tokens per step
constexpr int kTileBytes = kTile * kRowBytes;        // 36864
constexpr int kStages = 4;            // LDS ring depth
constexpr int kGroups = kRow / 64;    // 9 column groups of 128 bytes
constexpr int kKSteps = kRow / 16;    // 36 score K-steps
constexpr int kCBlocks = 512 / 32;    // 16 latent blocks
constexpr int kPv = 2 * kCBlocks;     // 32 PV MFMAs per tile
constexpr int kKWindow = 3;           // score operand reads in flight
constexpr int kVWindow = 4;           // PV operands (two reads each) in flight
constexpr int kSoftSlots = 17;        // score MFMAs the softmax arithmetic is spread over
constexpr int kLdsBytes = kStages * kTileBytes;
constexpr float kRescaleThreshold = 8.f;             // log2 units

static_assert(kTileBytes == 4 * kGroups * 1024, "each wave issues kGroups loads per tile");

// Low-bit cache rows (one OCP E4M3 byte per element and one fp32 scale per
// row).  A 32-token tile of codes is copied, as the 32 rows back to back,
// into the upper half of its ring stage, and its 32 scales into a small ring
// of their own; at the start of the step that first reads the tile, the
// workgroup converts the codes into the bf16 layout above (code * scale in
// fp32, rounded to bf16), so the products and the softmax are those of a
// bf16 cache.
// Copying 18,432 bytes takes 18 sixteen-byte load instructions; with the
// scale load twice, every wave issues five loads per tile.
constexpr int kFp8RowBytes = kRow;
constexpr int kFp8TileBytes = kTile * kFp8RowBytes;            // 18432
constexpr int kFp8PieceLoads = kFp8TileBytes / 1024;          // 18
constexpr int kFp8Loads = 5;                                   // per wave per tile
constexpr int kFp8RawOffset = kTileBytes - kFp8TileBytes;      // codes: upper half
constexpr int kFp8ScaleBytes = 64 * 4;                        // one scale load, per stage
static_assert(kFp8PieceLoads + 2 == 4 * kFp8Loads, "two scale loads complete the count");
static_assert(kFp8RowBytes % 16 == 0 && (kFp8RowBytes / 8) % 9 == 0, "");
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
static_assert((kStages & (kStages - 1)) == 0, "stage index uses a mask");
static_assert(kMfmaHeadsPerGroup == 4 * 32 && kMfmaTokenGranule == kTile, "");

// s_waitcnt immediate: wait until at most `n` vector-memory loads are
// outstanding; expcnt and lgkmcnt are left at their maxima (no wait).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// s_waitcnt immediate: wait until no LDS access is outstanding; vmcnt and
// expcnt are left at their maxima (no wait).
constexpr int kLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);
// Both: at most `n` vector-memory loads and no LDS access outstanding.
constexpr int vmcnt_lgkm0_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4); }

struct MfmaParams {
  const uint16_t* q_cat;  // [B, n_rows, 576] bf16
  CacheView cache;
  // Query rows per request: q_len tokens x heads_per_token heads, token-major.
  int n_rows, heads_per_token, q_len;
  int split_tokens, num_splits, head_groups, work_items;
  // Length-balanced partitions (split_tokens == 0): about part_target
  // partitions of at most part_max_tokens tokens, sized from the lengths of
  // the batch requests; the partition table goes to part_table.
  int batch, part_target, part_max_tokens;
  int32_t* part_table;
  float scale_log2;       // softmax scale * log2(e)
  uint16_t* part_o;       // bf16 partials
  float2* part_ml;        // per (request, split, head): (base-2 log-sum-exp, m)
  // One split only: when set, the kernel writes the normalised rows here
  // ([B, n_rows, 512] bf16) and the natural-log lse to lse_out (if set)
  // instead of partials.
  uint16_t* out_lat;
  float* lse_out;
};

// 16-byte direct-to-LDS load: every lane reads 16 bytes at `src` and writes
// them at LDS byte address lds_base + 16 * lane (lds_base wave-uniform, in M0).
// Issued as inline asm so the compiler's wait insertion does not see it: it
// cannot tell the ring stages apart and would otherwise drain every
// outstanding load before each LDS read.  The kernel waits for these loads
// itself (s_waitcnt vmcnt) before the barrier that publishes a stage.  The
// instruction has no result registers; its address (`src` plus the
// immediate kOffset) is read at issue.  No other instruction in this kernel
// uses M0.  The result lands at lds_base + 16 * lane.
template <int kOffset>
__device__ __forceinline__ void load_to_lds16(const void* src, unsigned lds_base) {
  // The immediate offset is added to the LDS address as well as to the
  // global one, so M0 carries the LDS base minus that offset.
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off offset:%2"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base) - kOffset), "i"(kOffset)
               : "memory", "m0");
}

// The same 16-byte and 4-byte loads from a wave-uniform base address (in
// SGPRs) plus a 32-bit per-lane byte offset: one VGPR per address.
__device__ __forceinline__ void load_to_lds16_sbase(unsigned voff, const void* sbase,
                                                    unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
__device__ __forceinline__ void load_to_lds4_sbase(unsigned voff, const void* sbase,
                                                   unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}

// The kGroups column groups of one token row: group gi sits gi * 128 bytes
// into the row (an immediate offset) and fills LDS at dst + gi * 4096.
template <int... gi>
__device__ __forceinline__ void load_row_groups(const void* src, unsigned dst,
                                                std::integer_sequence<int, gi...>) {
  (load_to_lds16<gi * 128>(src, dst + gi * 4096), ...);
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, in order.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// The two products are issued through inline asm so that they keep the
// order written below: the compiler may not sink the softmax arithmetic
// behind them or regroup them, which would serialise the matrix pipe behind
// LDS latency.  Scores accumulate in ordinary VGPRs (the O accumulators fill
// the whole accumulation register file), O in accumulation registers.  The
// compiler does not see these as MFMAs, so it inserts none of the wait
// states the hardware needs around them.  In this kernel every product's
// operands come from LDS reads (covered by s_waitcnt), from the previous
// product accumulating into the same registers (no wait states needed), or
// from VALU results written long before; mfma_first, used outside the loop,
// keeps two wait states in front of it.  After the last product into an
// accumulator an explicit drain precedes any other access.  A test compiles
// the kernel and checks these rules on the generated code.
__device__ __forceinline__ void mfma_first(f32x16_t& c, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x16_t& c, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_a(f32x16_t& c, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// Wait states between the last product writing an accumulator and any other
// access to it: at least 18 once the product has started (s_nop n waits
// n + 1).  An MFMA issued right behind an independent one may start up to a
// whole product later, so every drain below follows either a dependent chain
// (which starts each product as soon as it issues) or further MFMAs, or uses
// the longer drain at the end of the kernel.
__device__ __forceinline__ void drain_v(f32x16_t& c) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(c));
}
// Copies the score accumulator out with VALU moves issued right here (an
// asm statement keeps its place among the asm products): a copy the compiler
// placed itself could land right behind the product that writes `c`.
__device__ __forceinline__ void take_scores(float (&dst)[16], const f32x16_t& c) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const f32x2_t in = {c[2 * k], c[2 * k + 1]};
    f32x2_t out;
    asm volatile("v_mov_b64 %0, %1" : "=v"(out) : "v"(in));
    dst[2 * k] = out[0];
    dst[2 * k + 1] = out[1];
  }
}

// Pins the computation of x before this point of the instruction stream.
__device__ __forceinline__ void anchor(float x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void anchor(float x, float y) { asm volatile("" ::"v"(x), "v"(y)); }
// Keeps every computation on x after this point of the instruction stream.
__device__ __forceinline__ void launder(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void launder(int& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ float fmax3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

__device__ __forceinline__ unsigned lds_address(const void* p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>((MLA_LDS const void*)p));
}

// XOR key of token n's 128-byte rows.  The LDS has 64 four-byte banks: 16
// lanes reading one chunk of 16 consecutive tokens (the score operand) and
// 32 lanes reading four chunks of 4 consecutive tokens (the transposing PV
// operand read) each cover all 64 banks exactly once.  Rows of tokens of one
// parity share a bank half, so the key is a bijection of (n / 2) % 8 whose
// bit 2 differs between n and n + 2 when n % 4 < 2.
__device__ __forceinline__ int swz_key(int n) {
  const int j = (n >> 1) & 7;
  return j ^ ((j & 1) << 2);
}

// LDS byte offset (within a tile) of 16-byte chunk `chunk` (0..71) of token `n`.
__device__ __forceinline__ int swz(int n, int chunk) {
  return (((chunk >> 3) * kTile + n) << 7) + (((chunk & 7) ^ swz_key(n)) << 4);
}

// Length-balanced partitions.  Cutting a request's rows into partitions
// leaves the merged result unchanged up to rounding, so a launch may choose
// the cut from the lengths themselves, on the device: one partition length c
// for the whole batch, a multiple of 32 tokens, the smallest at which the
// partition counts n_b = ceil(len_b / c) add up to at most `target` (one
// workgroup per compute unit), capped at c_max (then the launch's capacity,
// sized on the host for that cap, holds them).  Requests own consecutive
// partition numbers, request b from off_b = n_0 + ... + n_(b-1).  Every wave
// computes this on its own from seq_lens (lane l keeps the lengths of
// requests kPer*l .. kPer*l + kPer-1 in registers; kPer = 1 up to 64
// requests, 4 up to 256), with register-only cross-lane arithmetic (DPP,
// lane swaps, ballots), so it costs a few hundred cycles and neither a
// launch nor a host synchronisation.
struct Partition {
  int b = -1, s = 0, c = 32;  // b < 0: the item is past the last partition
  int len = 0;                // seq_lens[b]
};

// Sum over the wave, in every lane: within each row of 16 lanes by DPP lane
// permutations (pairs, quads, halves of the row, the row), then across rows
// with the 16- and 32-lane swaps (each adds a row group to its partner).
__device__ __forceinline__ int wave_sum_int(int v) {
  v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xf, 0xf, false);   // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xf, 0xf, false);  // row_half_mirror
  v += __builtin_amdgcn_mov_dpp(v, 0x140, 0xf, 0xf, false);  // row_mirror
  const unsigned u = static_cast<unsigned>(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned w = r16[0] + r16[1];
  const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return static_cast<int>(r32[0] + r32[1]);
}

// Sum of v over the lanes below this one (v >= 0), one bit plane at a time:
// mbcnt counts the lanes below with the bit set.
__device__ __forceinline__ int wave_exclusive_sum(int v) {
  int excl = 0;
  for (int bit = 0; bit < 31; ++bit) {
    if (__ballot((v >> bit) != 0) == 0) break;
    const unsigned long long m = __ballot(((v >> bit) & 1) != 0);
    const int below = __builtin_amdgcn_mbcnt_hi(
        static_cast<unsigned>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(m), 0));
    excl += below << bit;
  }
  return excl;
}

// ceil(len / c) for 0 <= len <= 2^22 and 32 <= c (c a multiple of 32), with
// rc ~ 1 / c: the fp32 quotient is within 1/8 of the exact one, which one
// correction step each way absorbs.
__device__ __forceinline__ int ceil_div_len(int len, int c, float rc) {
  int q = static_cast<int>(static_cast<float>(len) * rc);
  int r = len - q * c;
  if (r < 0) { --q; r += c; }
  if (r >= c) { ++q; r -= c; }
  return q + (r > 0 ? 1 : 0);
}

template <int kPer>
__device__ Partition balanced_partition(const int32_t* __restrict__ seq_lens, int batch,
                                        int target, int c_max, int item, int lane,
                                        int32_t* table) {
  int len[kPer];
  int sum = 0, nz = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int bb = lane * kPer + k;
    len[k] = bb < batch ? seq_lens[bb] : 0;
    sum += len[k];
    nz += len[k] > 0 ? 1 : 0;
  }
  sum = wave_sum_int(sum);
  nz = wave_sum_int(nz);
  auto count = [&](int c) {
    const float rc = __builtin_amdgcn_rcpf(static_cast<float>(c));
    int n = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) n += ceil_div_len(len[k], c, rc);
    return wave_sum_int(n);
  };
  auto up32 = [](int x) { return (x + 31) / 32 * 32; };
  // sum / target bounds c from below; sum / (target - nz) from above
  // (n_b < len_b / c + 1 for every non-empty request).  Equal lengths meet
  // the target at the lower bound, so that is tried first.  When the cap
  // binds (lo == hi == c_max) c is the cap, whatever the count.
  int lo = max(32, up32((sum + target - 1) / target));
  int hi = target > nz ? up32((sum + (target - nz) - 1) / (target - nz)) : c_max;
  hi = max(32, min(hi, c_max));
  lo = min(lo, hi);
  if (lo < hi && count(lo) > target) {
    lo += 32;
    while (lo < hi) {
      const int mid = lo + (hi - lo) / 64 * 32;
      if (count(mid) <= target) hi = mid; else lo = mid + 32;
    }
  }
  const int c = lo;
  const float rc = __builtin_amdgcn_rcpf(static_cast<float>(c));
  int n[kPer], tot = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    n[k] = ceil_div_len(len[k], c, rc);
    tot += n[k];
  }
  int off = wave_exclusive_sum(tot), mine = -1, mine_len = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    if (table != nullptr && lane * kPer + k < batch) table[1 + lane * kPer + k] = off;
    // request (< 256) and partition (< 2^22 / 32) packed in one lane value
    if (item >= off && item < off + n[k]) {
      mine = (lane * kPer + k) << 23 | (item - off);
      mine_len = len[k];
    }
    off += n[k];
  }
  if (table != nullptr && lane == 63) {
    table[0] = c;
    table[1 + batch] = off;  // lane 63's running sum is the total
  }
  Partition pt;
  pt.c = c;
  const unsigned long long hit = __ballot(mine >= 0);
  if (hit != 0) {
    const int src = __ffsll(static_cast<long long>(hit)) - 1;
    const int v = __shfl(mine, src, 64);
    pt.len = __shfl(mine_len, src, 64);
    pt.b = v >> 23;
    pt.s = v & 0x7fffff;
  }
  return pt;
}

// kDirect: one split, the rows are normalised and written to out_lat (with
// lse) instead of partials; a separate instantiation keeps that epilogue out
// of the split kernels.
// kGH: query rows per workgroup.  128: wave w owns rows 32w..32w+31 over the
// whole score contraction and the whole latent output.  64: the two waves of
// head block hb = w % 2 split the work by kh = w / 2: wave kh takes the score
// k-steps 4i + 2kh and 4i + 2kh + 1 (i < 9; half of the 576-long contraction,
// RoPE columns included) and latent blocks 8kh .. 8kh + 7 of the output;
// after each tile's products the two partial score sums meet in LDS (fp32,
// added in the same order by both waves, so both hold the same scores, take
// the same softmax and keep the same running max and sum).  Half the query
// and half the partial sums per workgroup, for twice the workgroups per
// request.
template <bool kPaged, bool kFp8, bool kDirect, int kGH>
__global__ __launch_bounds__(256, 1) void decode_mfma_kernel(MfmaParams p) {
  constexpr bool kHalf = kGH == 64;
  static_assert(kGH == 128 || (kGH == 64 && !kFp8), "64-row groups: bf16 rows only");
  // Score k-steps, latent blocks and PV products per wave and tile.
  constexpr int kWK = kHalf ? kKSteps / 2 : kKSteps;
  constexpr int kWCB = kHalf ? kCBlocks / 2 : kCBlocks;
  constexpr int kWPv = 2 * kWCB;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];
  // Low-bit rows: the scales of the tile in each ring stage.
  __shared__ __attribute__((aligned(16))) uint8_t sc_lds[kFp8 ? kStages * kFp8ScaleBytes : 16];
  // 64-row groups: each wave's partial scores of the next tile (16 fp32 per
  // lane, four 16-byte chunks: chunk k of lane l at (k * 64 + l) * 16).
  __shared__ __attribute__((aligned(16))) uint8_t xch[kHalf ? 4 * 4096 : 16];
  // Loads per wave per tile, and cache bytes per row.
  constexpr int kLoads = kFp8 ? kFp8Loads : kGroups;
  constexpr int kSrcRowBytes = kFp8 ? kFp8RowBytes : kRowBytes;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int hb = kHalf ? (wave & 1) : wave;  // head block of 32 rows in the group
  const int kh = kHalf ? (wave >> 1) : 0;     // score / latent half (64-row groups)

  // XCD-aware work mapping: workgroup x runs on XCD x % 8; give every XCD a
  // contiguous range of work ids (the partitions of a request stay together).
  const int nwg = gridDim.x;
  const int work = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  if (work >= p.work_items) return;
  const int g = work % p.head_groups;
  const int item = work / p.head_groups;
  // Partition `item` (all head groups of a partition are consecutive work
  // ids, so they share an XCD): request b, its partition s of c tokens, and
  // its number pidx in the partial layout.
  int b, s, c, pidx, req_len;
  if (p.split_tokens == 0) {
    int32_t* table = work == 0 && wave == 0 ? p.part_table : nullptr;
    const Partition pt =
        p.batch <= 64 ? balanced_partition<1>(p.cache.seq_lens, p.batch, p.part_target,
                                              p.part_max_tokens, item, lane, table)
                      : balanced_partition<4>(p.cache.seq_lens, p.batch, p.part_target,
                                              p.part_max_tokens, item, lane, table);
    // The same in every lane; readfirstlane tells the compiler so (the
    // addresses built from them stay in scalar registers).
    b = __builtin_amdgcn_readfirstlane(pt.b);
    if (b < 0) return;
    s = __builtin_amdgcn_readfirstlane(pt.s);
    c = __builtin_amdgcn_readfirstlane(pt.c);
    req_len = __builtin_amdgcn_readfirstlane(pt.len);
    pidx = item;
  } else {
    s = item % p.num_splits;
    b = item / p.num_splits;
    c = p.split_tokens;
    req_len = p.cache.seq_lens[b];
    pidx = item;
  }

  // Query token j of the request (head group g covers rows g*kGH ..) sees
  // the rows up to its own position: q_len - 1 - j fewer than the request.
  const int len = req_len - (p.q_len - 1 - g * kGH / p.heads_per_token);
  const int t0 = s * c;
  const int t1 = min(t0 + c, len);
  const int hblock = g * (kGH / 32) + hb;
  const int head = hblock * 32 + l32;
  if (t0 >= t1) {
    // The combine never reads partitions past the length.  Written directly,
    // a row with nothing visible is o = 0, lse = -inf.
    if constexpr (kDirect) {
      constexpr int kZRows = kHalf ? 16 : 32;  // rows of the head block this wave clears
      uint16_t* z = p.out_lat +
                    (static_cast<size_t>(b) * p.n_rows + hblock * 32 + kh * kZRows) * 512 +
                    lane * 8;
      bf16x8_t zero;
#pragma unroll
      for (int e = 0; e < 8; ++e) zero[e] = static_cast<__bf16>(0.f);
      for (int r = 0; r < kZRows; ++r) *reinterpret_cast<bf16x8_t*>(z + r * 512) = zero;
      if (p.lse_out != nullptr && half == 0 && kh == 0)
        p.lse_out[static_cast<size_t>(b) * p.n_rows + head] = -INFINITY;
    }
    return;
  }

  f32x16_t acc[kWCB];
#pragma unroll
  for (int cb = 0; cb < kWCB; ++cb)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[cb][v] = 0.f;
  float m = -INFINITY, l = 0.f;

  // Loader: wave w fills token octet w of every column group.  This lane's
  // token is w*8 + lane/8 and it fills LDS position lane%8 of that token's
  // group, which holds logical chunk (lane%8) ^ swz_key(token).  Rows past the
  // partition are clamped to t1 - 1: never read past the request, and their
  // probabilities are forced to 0.
  const int n_load = wave * 8 + (lane >> 3);
  const int chunk_off = ((lane & 7) ^ swz_key(n_load)) * 16;
  const uint8_t* req_base =
      kPaged ? p.cache.data
             : p.cache.data + static_cast<size_t>(b) * p.cache.max_len * kSrcRowBytes;
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
  // This lane's source address for the tile starting at token tile_t0, and
  // this wave's LDS destination in a ring stage.
  auto tile_src = [&](int tile_t0) {
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
    return src + chunk_off;
  };
  auto tile_dst = [&](int stage) { return lds_address(lds + stage * kTileBytes) + wave * 1024; };

  // Low-bit rows: load j of this wave for the tile at tile_t0 is instruction
  // i = wave + 4j; instructions 0..17 copy 16-byte pieces (lane l of
  // instruction i: piece i*64 + l, i.e. token piece / 36, byte (piece % 36) * 16
  // of its row), 18 and 19 the scales (lane l: token min(l, 31)).  A tile
  // lies within one page (page_size % 32 == 0).
  // Low-bit rows, loads of the tile at tile_t0 into `stage`: instruction
  // i < 18 copies 16-byte pieces (lane l: piece i*64 + l, i.e. token
  // piece / 36, byte (piece % 36) * 16 of its row; the rows of a tile are
  // contiguous), instructions 18 and 19 the 32 scales (lane l: token
  // min(l, 31)).  Wave w issues pieces w, w+4, w+8, w+12 between its products
  // (fp8_piece, branch-free) and, from fp8_extra, piece 16 + w (w < 2) or the
  // scales (w >= 2): five loads per wave per tile.  Tiles past the partition
  // re-read its last row, so addresses start at tile_a = min(tile_t0, t1 - 1)
  // and tokens past lim (the last valid one, >= 0) re-read row lim.  A tile
  // lies within one page (page_size % 32 == 0).
  struct Fp8Tile {
    const uint8_t* codes;   // row of token tile_a
    const float* scales;    // its scale
    int lim;
    unsigned lds;           // the stage
    unsigned lds_scales;    // its scales
  };
  auto fp8_tile = [&](int tile_t0, int stage) {
    Fp8Tile f;
    const int tile_a = min(tile_t0, t1 - 1);
    f.lim = min(t1 - 1 - tile_a, kTile - 1);
    size_t row0;
    if constexpr (kPaged) {
      const int page =
          __builtin_amdgcn_readlane(page_of_lane, tile_a / p.cache.page_size - first_page);
      row0 = static_cast<size_t>(page) * p.cache.page_size + tile_a % p.cache.page_size;
    } else {
      row0 = static_cast<size_t>(b) * p.cache.max_len + tile_a;
    }
    f.codes = p.cache.data + row0 * kFp8RowBytes;
    f.scales = p.cache.scales + row0;
    f.lds = lds_address(lds + stage * kTileBytes);
    f.lds_scales = lds_address(sc_lds + stage * kFp8ScaleBytes);
    return f;
  };
  auto fp8_piece_at = [&](const Fp8Tile& f, int i) {
    const int piece = i * 64 + lane;
    const int tok = piece / 36;
    const unsigned off = min(tok, f.lim) * kFp8RowBytes + (piece - tok * 36) * 16;
    load_to_lds16_sbase(off, f.codes, f.lds + kFp8RawOffset + i * 1024);
  };
  auto fp8_piece = [&](const Fp8Tile& f, int j) { fp8_piece_at(f, wave_u + 4 * j); };
  auto fp8_extra = [&](const Fp8Tile& f) {
    if (wave_u < 2)
      fp8_piece_at(f, 16 + wave_u);
    else
      load_to_lds4_sbase(min(lane, f.lim) * 4, f.scales, f.lds_scales);
  };
  static_assert(4 * 4 + 2 == kFp8PieceLoads && kFp8Loads == 5, "four pieces and one extra");
  // This wave's load J (< kGroups) of a bf16 tile: column group J of its
  // token octet (src = tile_src(tile_t0), dst = tile_dst(stage)).
  auto issue_load = [&](auto J, const uint8_t* src, unsigned dst) {
    load_to_lds16<decltype(J)::value * 128>(src, dst + decltype(J)::value * 4096);
  };
  auto issue_tile = [&](int stage, int tile_t0) {
    if constexpr (kFp8) {
      const Fp8Tile f = fp8_tile(tile_t0, stage);
      fp8_extra(f);
#pragma unroll
      for (int j = 0; j < 4; ++j) fp8_piece(f, j);
    } else {
      load_row_groups(tile_src(tile_t0), tile_dst(stage),
                      std::make_integer_sequence<int, kGroups>{});
    }
  };
  // Low-bit rows: turn the codes of the tile in `stage` into the bf16 layout
  // of that stage (code * scale rounded to bf16).  Lane (token
  // n = w*8 + lane/8, part = lane%8) converts bf16 chunk part + 8k of its
  // token for k = 0..8, i.e. the part-th chunk of every column group k (8
  // code bytes each).  Groups 0-3 lie below the codes, so they are written at
  // once; groups 4-8 overwrite codes and are written after a barrier that
  // follows every lane's reads.  A second barrier publishes the tile.
  auto fp8_convert = [&](int stage) {
    typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
    static_assert(4 * 4096 <= kFp8RawOffset, "groups 0-3 lie below the codes");
    uint8_t* st = lds + stage * kTileBytes;
    const int part = lane & 7;
    const MLA_LDS uint8_t* raw =
        (MLA_LDS const uint8_t*)(st + kFp8RawOffset + n_load * kFp8RowBytes + part * 8);
    const float sc = *(MLA_LDS const float*)(uintptr_t)(lds_address(sc_lds) +
                                                       stage * kFp8ScaleBytes + n_load * 4);
    u32x2_t w[kGroups];
#pragma unroll
    for (int k = 0; k < kGroups; ++k) w[k] = *(MLA_LDS const u32x2_t*)(raw + k * 64);
    // code * scale in fp32, rounded to bf16.
    auto put = [&](int k) {
      typedef float f32x2_t __attribute__((ext_vector_type(2)));
      const f32x2_t x0 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[k][0]), false);
      const f32x2_t x1 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[k][0]), true);
      const f32x2_t x2 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[k][1]), false);
      const f32x2_t x3 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[k][1]), true);
      bf16x8_t v;
      v[0] = static_cast<__bf16>(x0[0] * sc);
      v[1] = static_cast<__bf16>(x0[1] * sc);
      v[2] = static_cast<__bf16>(x1[0] * sc);
      v[3] = static_cast<__bf16>(x1[1] * sc);
      v[4] = static_cast<__bf16>(x2[0] * sc);
      v[5] = static_cast<__bf16>(x2[1] * sc);
      v[6] = static_cast<__bf16>(x3[0] * sc);
      v[7] = static_cast<__bf16>(x3[1] * sc);
      *(MLA_LDS bf16x8_t*)(st + swz(n_load, part + 8 * k)) = v;
    };
#pragma unroll
    for (int k = 0; k < 4; ++k) put(k);
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 4; k < kGroups; ++k) put(k);
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Per-lane LDS offsets within a tile.  Score operand of K-step ks:
  // swz(l32, 2 ks + half) = qoff[ks % 4] + (ks / 4) * 4096.  PV operand of
  // latent block cb, K-step kk, read lo/hi (tokens 8 apart, which have
  // different XOR keys): voff[hi * 2 + cb % 2] + (cb / 2) * 4096 + kk * 2048.  The transposing read of lane (16-lane group G,
  // index r) addresses token {0,8} + (G/2)*4 + r/4 at latent column
  // 16*(G%2) + 4*(r%4) of its block.
  // 64-row groups: local score k-step i of wave kh is global k-step
  // 4 (i / 2) + 2 kh + i % 2, i.e. offsets qoff[i % 2] + (i / 2) * 4096 with
  // qoff[q] = the 128-row form's qoff[2 kh + q]; its latent blocks start at
  // 8 kh (16384 bytes further into the tile).
  constexpr int kQP = kHalf ? 2 : 4;  // period of the score-operand offsets
  const int tr_tok = (half << 2) + ((lane >> 2) & 3);
  const int tr_col = (((lane >> 4) & 1) << 4) + ((lane & 3) << 2);
  int qoff0[4], voff0[4];
#pragma unroll
  for (int q = 0; q < kQP; ++q) qoff0[q] = lds_address(lds) + swz(l32, (q + 2 * kh) * 2 + half);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = (q & 1) * 32 + tr_col;
    voff0[q] = lds_address(lds) + swz(tr_tok + (q >> 1) * 8, c >> 3) + (c & 7) * 2 +
               kh * (kWCB / 2) * 4096;
  }
  const int ntiles = (t1 - t0 + kTile - 1) / kTile;

  // Operand reads.  Score operand of local K-step ks of the tile whose
  // offsets are in `qoff`; PV operand i = kk * kWCB + cb of the tile whose
  // offsets are in `voff` (consecutive PV MFMAs then update different
  // accumulators).
  auto read_k = [&](const int (&qoff)[4], int ks) {
    return *(MLA_LDS const bf16x8_t*)(uintptr_t)(qoff[ks % kQP] + (ks / kQP) * 4096);
  };
  auto read_v = [&](const int (&voff)[4], int i) {
    const int kk = i / kWCB, cb = i % kWCB;
    const unsigned a = (cb >> 1) * 4096 + kk * 2048;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MLA_LDS i16x4_t*)(uintptr_t)(voff[cb & 1] + a));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MLA_LDS i16x4_t*)(uintptr_t)(voff[2 + (cb & 1)] + a));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // Operand offsets of ring stages; the empty asm keeps the compiler from
  // precomputing every operand address of every stage.
  auto k_offsets = [&](int stage, int (&qoff)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) qoff[q] = q < kQP ? qoff0[q] + stage * kTileBytes : 0;
    asm volatile("" : "+v"(qoff[0]), "+v"(qoff[1]), "+v"(qoff[2]), "+v"(qoff[3]));
  };
  auto v_offsets = [&](int stage, int (&voff)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) voff[q] = voff0[q] + stage * kTileBytes;
    asm volatile("" : "+v"(voff[0]), "+v"(voff[1]), "+v"(voff[2]), "+v"(voff[3]));
  };

  // Query as the B operand: lane holds head `head`, K slots half*8..+7 of
  // each of the 36 K-steps.  The workgroup's 128 query rows have the shape of
  // four tiles (head block j = rows 32j..32j+31) and go through the ring with
  // the tile loader: every load reads whole 128-byte lines, where loading the
  // fragments straight into registers would touch 32 lines per instruction.
  // Each wave then reads its fragments with the (bank-conflict free)
  // score-operand reads.  Two rounds through stages 2 and 3, so that tiles 0
  // and 1 stream into stages 0 and 1 meanwhile: round 0 carries head blocks
  // 2 and 3 (read by waves 2 and 3), round 1 head blocks 0 and 1.  The
  // barrier closing each round waits for LDS reads only, never for the tile
  // loads still in flight.
  // 64-row groups: one round, head blocks 0 and 1 into stages 2 and 3 while
  // tiles 0 and 1 stream into stages 0 and 1; every wave reads its own k-steps
  // of its head block.
  static_assert(kStages == 4 && kMfmaHeadsPerGroup == kStages * kTile, "query fills the ring");
  bf16x8_t qf[kWK];
  {
    const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(p.q_cat) +
                          (static_cast<size_t>(b) * p.n_rows + g * kGH + n_load) * kRowBytes +
                          chunk_off;
    if constexpr (kHalf) {
      load_row_groups(qsrc, tile_dst(2), std::make_integer_sequence<int, kGroups>{});
      load_row_groups(qsrc + kTile * kRowBytes, tile_dst(3),
                      std::make_integer_sequence<int, kGroups>{});
      issue_tile(0, t0);
      issue_tile(1, t0 + kTile);
      // Loads complete in issue order: the query has landed, tiles 0 and 1
      // may be in flight.
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLoads));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      int qo[4];
      k_offsets(2 + hb, qo);
#pragma unroll
      for (int ks = 0; ks < kWK; ++ks) qf[ks] = read_k(qo, ks);
      // Every wave's reads of stages 2 and 3 are done before they are
      // refilled, and tile 0 has landed (tile 1 may be in flight).
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoads));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else {
      for (int round = 0; round < 2; ++round) {
        const int hb0 = 2 - 2 * round;  // first head block of this round
        load_row_groups(qsrc + hb0 * kTile * kRowBytes, tile_dst(2),
                        std::make_integer_sequence<int, kGroups>{});
        load_row_groups(qsrc + (hb0 + 1) * kTile * kRowBytes, tile_dst(3),
                        std::make_integer_sequence<int, kGroups>{});
        // Tile 0 follows the first round's query loads and tile 1 the second
        // round's, so the second wait need not cover tile 1: when every
        // workgroup starts at once, the query and tile 0 arrive sooner with
        // tile 1 not yet competing for the memory system.  Loads complete in
        // issue order, so vmcnt(kLoads) means: everything but the tile just
        // issued has landed.
        issue_tile(round, t0 + round * kTile);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoads));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if ((wave & 2) == hb0) {
          int qo[4];
          k_offsets(2 + (wave & 1), qo);
#pragma unroll
          for (int ks = 0; ks < kWK; ++ks) qf[ks] = read_k(qo, ks);
        }
        // Every wave's reads of stages 2 and 3 are done before they are
        // refilled.
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
    }
  }
  // The softmax takes its max on raw scores and folds the scale into the
  // exponent, which needs a scale >= 0: a negative scale moves onto the query
  // (an exact sign flip of every element).
  const float scale = fabsf(p.scale_log2);
  if (p.scale_log2 < 0.f) {
    typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int ks = 0; ks < kWK; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8_t, __builtin_bit_cast(u32x4_t, qf[ks]) ^ 0x80008000u);
  }

  // Scores S^T accumulate in one chain of dependent products (on gfx950 a
  // 32x32x16 product that accumulates onto the previous one's result still
  // issues every 32 cycles).
  f32x16_t sc;
  auto qk = [&](bf16x8_t (&ta)[kWK], const int (&qoff)[4], int ks) {
    if (ks + kKWindow < kWK) ta[ks + kKWindow] = read_k(qoff, ks + kKWindow);
    if (ks == 0)
      mfma_first(sc, ta[ks], qf[ks]);
    else
      mfma_v(sc, ta[ks], qf[ks]);
  };

  // Prologue: tile 0 landed with the query (the wait of the second query
  // round); tile 1 may still be in flight.  The compiler does not see these
  // loads (inline asm), and the tile loads are governed only by the waits
  // below.  Every step issues exactly one tile (past the last tile they
  // re-read the partition's last row into a stage that is never read
  // again), so at step t "this wave's loads of tile t+1 have landed" while
  // those of tile t+2 may stay in flight is always vmcnt(kLoads).
  //
  // Scores of tile 0, with the loads of tile 2 one behind each of the first
  // kLoads score products (low-bit rows: tile 0 is converted first).
  if constexpr (kFp8) fp8_convert(0);
  {
    int qoff[4];
    k_offsets(0, qoff);
    // Tile 0's score operands run eight reads ahead (the loop keeps three:
    // there the softmax arithmetic fills the gaps, here nothing does).
    bf16x8_t ta[kWK];
    constexpr int kW0 = 8;
#pragma unroll
    for (int ks = 0; ks < kW0; ++ks) ta[ks] = read_k(qoff, ks);
    const uint8_t* src2 = kFp8 ? nullptr : tile_src(t0 + 2 * kTile);
    const unsigned dst2 = tile_dst(2);
    Fp8Tile f2{};
    if constexpr (kFp8) {
      f2 = fp8_tile(t0 + 2 * kTile, 2);
      fp8_extra(f2);
    }
    static_for<kWK>([&](auto K) {
      constexpr int ks = decltype(K)::value;
      if constexpr (ks + kW0 < kWK) ta[ks + kW0] = read_k(qoff, ks + kW0);
      if constexpr (ks == 0)
        mfma_first(sc, ta[ks], qf[ks]);
      else
        mfma_v(sc, ta[ks], qf[ks]);
      if constexpr (kFp8) {
        if constexpr (ks < 4) fp8_piece(f2, ks);
      } else if constexpr (ks < kGroups) {
        issue_load(K, src2, dst2);
      }
    });
    drain_v(sc);
  }
  float s_next[16];
  take_scores(s_next, sc);

  // 64-row groups: this wave's partial scores of the next tile go to its
  // slot of xch; after the next barrier the partner wave (same head block,
  // other half) adds them to its own.  A slot is rewritten only after a
  // second barrier that follows the partner's read of it.
  auto put_partial = [&](const float (&sp)[16]) {
    if constexpr (kHalf) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *(MLA_LDS f32x4_t*)(uintptr_t)(lds_address(xch) + wave * 4096 + (k * 64 + lane) * 16) =
            f32x4_t{sp[4 * k], sp[4 * k + 1], sp[4 * k + 2], sp[4 * k + 3]};
    }
  };
  auto get_partial = [&](f32x4_t (&pp)[4]) {
    if constexpr (kHalf) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        pp[k] = *(MLA_LDS const f32x4_t*)(uintptr_t)(lds_address(xch) + (wave ^ 2) * 4096 +
                                                       (k * 64 + lane) * 16);
    }
  };
  put_partial(s_next);

  // One step.  The softmax arithmetic of tile t (stage t % 4) is spread over
  // the first kSoftSlots score MFMAs of tile t+1 (stage (t+1) % 4), a few VALU
  // instructions behind each product, where they issue while the matrix pipe
  // works; then the PV products of tile t, the first ones paired with the
  // remaining score MFMAs, and between them the loads of tile t+3, one column
  // group every second PV product (issued in a burst, the four waves' loads
  // queue behind each other in the CU's address unit).
  auto step = [&](int t, auto has_next) {
    constexpr bool kNext = decltype(has_next)::value;
    // The scores of tile t, taken out of the accumulator at the end of the
    // previous step (or after the prologue).
    float sv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) sv[v] = s_next[v];

    // Wait for this wave's loads of tile t+1 (tile t+2 may stay in flight),
    // then for everyone's.  A raw s_barrier, not __syncthreads(): the latter
    // also waits for every outstanding global load and would drain the
    // prefetch.  The compiler fence keeps LDS accesses on their side of the
    // barrier.  After it every wave is past step t-1, so the stage of tile
    // t-1, (t+3) % 4, is refilled with tile t+3.
    // (64-row groups: this wave's partial scores of tile t, written at the
    // end of the previous step, are complete too.)
    __builtin_amdgcn_s_waitcnt(kHalf ? vmcnt_lgkm0_imm(kLoads) : vmcnt_imm(kLoads));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    f32x4_t pp[4];
    get_partial(pp);
    // Low-bit rows: tile t+1, read by this step's score products, is
    // converted now (tile t was converted one step earlier).
    if constexpr (kFp8 && kNext) fp8_convert((t + 1) & (kStages - 1));

    const int nvalid = t1 - (t0 + t * kTile);
    int qoff[4], voff[4];
    k_offsets((t + 1) & (kStages - 1), qoff);
    v_offsets(t & (kStages - 1), voff);
    const int next_t0 = t0 + (t + 3) * kTile;
    const int next_stage = (t + 3) & (kStages - 1);
    const uint8_t* next_src = kFp8 ? nullptr : tile_src(next_t0);
    const unsigned next_dst = tile_dst(next_stage);
    Fp8Tile fn{};
    if constexpr (kFp8) {
      fn = fp8_tile(next_t0, next_stage);
      fp8_extra(fn);
    }

    bf16x8_t ta[kWK];
    if constexpr (kNext) {
#pragma unroll
      for (int ks = 0; ks < kKWindow; ++ks) ta[ks] = read_k(qoff, ks);
    }
    auto qk_at = [&](int ks) {
      if constexpr (kNext) qk(ta, qoff, ks);
      if constexpr (kHalf && !kFp8) {
        // Tile t+3's first four column groups (every step issues them, as it
        // issues the other five, so vmcnt counts stay uniform).
        if (ks == 3) issue_load(std::integral_constant<int, 0>{}, next_src, next_dst);
        if (ks == 7) issue_load(std::integral_constant<int, 1>{}, next_src, next_dst);
        if (ks == 11) issue_load(std::integral_constant<int, 2>{}, next_src, next_dst);
        if (ks == 15) issue_load(std::integral_constant<int, 3>{}, next_src, next_dst);
      }
    };

    // Accumulator row of register v in this lane: token (v/4)*8 + half*4 +
    // v%4, valid while (v/4)*8 + v%4 < nvalid - half*4.  Only a partition's
    // last tile can be partial; its invalid scores are excluded from the max
    // here and their probabilities zeroed below.
    // (The limit is laundered inside each branch so that the compiler does
    // not hoist its comparisons into every full tile.)
    const bool partial = nvalid < kTile;
    const int lim = nvalid - half * 4;
    auto mask_partial = [&]() {
      if (partial) {
        int lim_p = lim;
        launder(lim_p);
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if ((v >> 2) * 8 + (v & 3) >= lim_p) sv[v] = -INFINITY;
      }
    };
    if constexpr (!kHalf) mask_partial();

    // Tile max of the raw scores (the scale is >= 0 here, so it commutes with
    // the max), over both lane halves, then scaled to exp2 units.
    qk_at(0);
    if constexpr (kHalf) {
      // The partner's half of the scores (fp32 addition commutes, so both
      // waves hold the same sums).  The second barrier:
      // every wave has read its partner's slot before any slot is rewritten
      // at the end of this step.
#pragma unroll
      for (int v = 0; v < 16; ++v) sv[v] += pp[v >> 2][v & 3];
#pragma unroll
      for (int v = 0; v < 16; v += 2) anchor(sv[v], sv[v + 1]);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      mask_partial();
    }
#pragma unroll
    for (int v = 0; v < 12; ++v) launder(sv[v]);
    const float a0 = fmax3(sv[0], sv[1], sv[2]), a1 = fmax3(sv[3], sv[4], sv[5]);
    const float a2 = fmax3(sv[6], sv[7], sv[8]), a3 = fmax3(sv[9], sv[10], sv[11]);
    anchor(a0, a1);
    anchor(a2, a3);
    qk_at(1);
#pragma unroll
    for (int v = 12; v < 16; ++v) launder(sv[v]);
    float tmax = fmaxf(fmax3(a0, a1, sv[15]), fmax3(a2, a3, fmax3(sv[12], sv[13], sv[14])));
    anchor(tmax);
    qk_at(2);
    tmax = halves_max(tmax) * scale;
    anchor(tmax);
    qk_at(3);
    // The new running max is decided here; the (rare) accumulator rescale it
    // implies runs after the softmax.
    const bool rescale = __builtin_amdgcn_ballot_w64(tmax > m + kRescaleThreshold) != 0;
    const float m_new = rescale ? fmaxf(m, tmax) : m;
    anchor(m_new);

    // p = exp2(scale * s - m_new), two per product.
    float pv[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qk_at(4 + j);
      launder(sv[2 * j]);
      launder(sv[2 * j + 1]);
      pv[2 * j] = __builtin_amdgcn_exp2f(fmaf(sv[2 * j], scale, -m_new));
      pv[2 * j + 1] = __builtin_amdgcn_exp2f(fmaf(sv[2 * j + 1], scale, -m_new));
      anchor(pv[2 * j], pv[2 * j + 1]);
    }
    if (partial) {
      int lim_p = lim;
      launder(lim_p);
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if ((v >> 2) * 8 + (v & 3) >= lim_p) pv[v] = 0.f;
    }
    // bf16 probabilities (the PV B operand) and their sum, four per product.
    bf16x8_t pb[2];
    float s4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      qk_at(12 + k);
#pragma unroll
      for (int e = 0; e < 4; ++e) pb[k >> 1][(k & 1) * 4 + e] = static_cast<__bf16>(pv[4 * k + e]);
      s4[k] = (pv[4 * k] + pv[4 * k + 1]) + (pv[4 * k + 2] + pv[4 * k + 3]);
      anchor(s4[k]);
    }
    // The PV operand is complete before the last softmax-phase score product:
    // at least that product separates its VALU writes from the first PV
    // product that reads it (two wait states needed).
    asm volatile("" ::"v"(pb[0]), "v"(pb[1]));
    qk_at(16);
    const float psum = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    static_assert(kSoftSlots == 17, "the softmax above occupies score products 0..16");

    bf16x8_t va[kWPv];
#pragma unroll
    for (int i = 0; i < kVWindow; ++i) va[i] = read_v(voff, i);

    // On the first tile every lane's running max is -inf and the accumulators
    // and the sum are still zero: nothing to rescale.  Skipping it saves 768
    // VALU instructions (about 4000 cycles) at the start of every partition.
    if (rescale && t != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      // Scale the accumulators in place in the accumulation registers.  The
      // PV MFMAs that last wrote them retired a whole score pass ago; the
      // s_nops cover the MFMA-to-read wait states regardless.
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory");
#pragma unroll
      for (int cb = 0; cb < kWCB; ++cb)
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
    }
    l += psum;
    m = m_new;

    // PV of tile t; the first ones paired with the remaining score MFMAs of
    // tile t+1, every second one followed by one column group of tile t+3.
    // (64-row groups: half as many PV products per wave; four of the nine
    // tile loads go between the score products of the softmax phase, the
    // other five after every third PV product, so that the four waves' loads
    // do not queue at the address unit at once.)
    static_for<kWPv>([&](auto I) {
      constexpr int i = decltype(I)::value;
      if constexpr (i + kVWindow < kWPv) va[i + kVWindow] = read_v(voff, i + kVWindow);
      mfma_a(acc[i % kWCB], va[i], pb[i / kWCB]);
      if constexpr (kNext && kSoftSlots + i < kWK) qk(ta, qoff, kSoftSlots + i);
      if constexpr (kFp8) {
        if constexpr (i % 2 == 0 && i / 2 < 4) fp8_piece(fn, i / 2);
      } else if constexpr (kHalf) {
        if constexpr (i % 3 == 1 && i / 3 < kGroups - 4)
          issue_load(std::integral_constant<int, 4 + i / 3>{}, next_src, next_dst);
      } else if constexpr (i % 2 == 0 && i / 2 < kGroups) {
        issue_load(std::integral_constant<int, i / 2>{}, next_src, next_dst);
      }
    });
    static_assert(kWK - kSoftSlots <= kWPv, "every score MFMA is paired");
    static_assert(!kHalf || (kGroups - 4 <= (kWPv + 1) / 3 && kSoftSlots > 15),
                  "every column group of tile t+3 is issued once per step");
    // The scores of tile t+1 leave the accumulator behind the last PV
    // products, which issue after the last score product: it has retired by
    // then, with far more than the 18 wait states a VALU read of an MFMA
    // result needs.
    static_assert(kWPv - (kWK - kSoftSlots) >= 4, "PV products behind the last score product");
    if constexpr (kNext) {
      take_scores(s_next, sc);
      put_partial(s_next);
    }
  };

  for (int t = 0; t + 1 < ntiles; ++t) step(t, std::true_type{});
  step(ntiles - 1, std::false_type{});
  // The trailing loads must land before the workgroup's LDS is released, and
  // the last PV products before the accumulators are read.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int cb = 0; cb < kWCB; ++cb) asm volatile("" : "+a"(acc[cb]));

  // Softmax sum over both lane halves (each half saw half of the tokens).
  l = halves_sum(l);

  constexpr bool direct = kDirect;
  // bf16 partial, partition-major: part_o[(pidx * n_rows + row) * 512 + c]
  // (with one split per request pidx = b, the layout of out_lat), written as
  // accumulated
  // (relative to the running max m, not divided by l: the combine applies
  // both factors as one weight, which saves a multiply per element here).
  // Register v of latent block cb holds column cb*32 + (v/4)*8 + half*4 +
  // v%4.  The rows pass through LDS (free once every wave is past its last
  // step) so that each global store writes a whole 1 KiB row: head block hb
  // owns rows hb*32 .. hb*32+31, kOutStride bytes apart (64-row groups: the
  // two waves of a head block write the two latent halves of its rows, then
  // each stores 16 of them).
  constexpr int kOutStride = 1024 + 16;
  static_assert(4 * 32 * kOutStride <= kLdsBytes, "epilogue rows fit in the ring");
  __syncthreads();
  uint8_t* rows = lds + hb * 32 * kOutStride;
  const float inv_l = direct ? 1.f / l : 1.f;
#pragma unroll
  for (int cb = 0; cb < kWCB; ++cb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      bf16x4_t v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = static_cast<__bf16>(acc[cb][gq * 4 + e] * inv_l);
      *reinterpret_cast<bf16x4_t*>(rows + l32 * kOutStride +
                                   ((kh * kWCB + cb) * 32 + gq * 8 + half * 4) * 2) = v4;
    }
  if constexpr (kHalf) __syncthreads();
  // The workgroup's rows of one partition are contiguous.
  constexpr int kStRows = kHalf ? 16 : 32;  // rows this wave stores
  uint16_t* dst = (direct ? p.out_lat : p.part_o) +
                  (static_cast<size_t>(pidx) * p.n_rows + hblock * 32 + kh * kStRows) * 512 +
                  lane * 8;
  constexpr size_t row_stride = 512;
  // Plain stores: the combine that reads the partials right after this
  // kernel finds them in the last-level cache (non-temporal stores make this
  // kernel slightly faster but the whole step slower).
#pragma unroll 8
  for (int r = 0; r < kStRows; ++r)
    *reinterpret_cast<bf16x8_t*>(dst + r * row_stride) =
        *reinterpret_cast<const bf16x8_t*>(rows + (kh * kStRows + r) * kOutStride + lane * 16);
  if (half == 0 && kh == 0) {
    if (direct) {
      if (p.lse_out != nullptr)
        p.lse_out[static_cast<size_t>(b) * p.n_rows + head] = (m + __log2f(l)) * kLn2;
    } else {
      p.part_ml[static_cast<size_t>(pidx) * p.n_rows + head] = make_float2(m + __log2f(l), m);
    }
  }
}

}  // namespace

hipError_t launch_partials_mfma(const DecodeArgs& a) {
  if (a.batch == 0) return hipSuccess;
  MfmaParams p;
  p.q_cat = static_cast<const uint16_t*>(a.q_cat);
  p.cache = a.cache;
  p.n_rows = a.q_len * a.n_heads;
  p.heads_per_token = a.n_heads;
  p.q_len = a.q_len;
  p.split_tokens = a.split_tokens;
  p.num_splits = a.num_splits;
  p.head_groups = a.head_groups;
  p.work_items = a.partitions * a.head_groups;
  p.batch = a.batch;
  p.part_target = a.part_target;
  p.part_max_tokens = a.part_max_tokens;
  p.part_table = a.part_table;
  if (a.split_tokens == 0 &&
      (a.batch > kBalancedMaxBatch || a.cache.max_len > kBalancedMaxLen || a.direct ||
       a.part_table == nullptr || a.part_target < 1 || a.part_max_tokens < 32 ||
       a.part_max_tokens % 32 != 0))
    return hipErrorInvalidValue;
  p.scale_log2 = a.softmax_scale * kLog2e;
  p.part_o = static_cast<uint16_t*>(a.part_o);
  p.part_ml = reinterpret_cast<float2*>(a.part_lse);
  if (a.direct && a.num_splits != 1) return hipErrorInvalidValue;
  p.out_lat = a.direct ? static_cast<uint16_t*>(a.out_lat) : nullptr;
  p.lse_out = a.direct ? a.lse : nullptr;
  const int grid = (p.work_items + 7) / 8 * 8;  // multiple of the 8 XCDs
  const bool paged = a.cache.page_table != nullptr, fp8 = a.cache.fp8 != 0;
  // The direct form exists for bf16 rows only (the low-bit one would spill),
  // and so does the 64-row form.
  if (a.direct && fp8) return hipErrorInvalidValue;
  if (a.group_rows != 128 && (a.group_rows != 64 || fp8)) return hipErrorInvalidValue;
  using Kernel = void (*)(MfmaParams);
  Kernel kernel;
  if (a.group_rows == 64)
    kernel = a.direct ? (paged ? decode_mfma_kernel<true, false, true, 64>
                               : decode_mfma_kernel<false, false, true, 64>)
                      : (paged ? decode_mfma_kernel<true, false, false, 64>
                               : decode_mfma_kernel<false, false, false, 64>);
  else if (a.direct)
    kernel = paged ? decode_mfma_kernel<true, false, true, 128>
                   : decode_mfma_kernel<false, false, true, 128>;
  else
    kernel = paged ? (fp8 ? decode_mfma_kernel<true, true, false, 128>
                          : decode_mfma_kernel<true, false, false, 128>)
                   : (fp8 ? decode_mfma_kernel<false, true, false, 128>
                          : decode_mfma_kernel<false, false, false, 128>);
  kernel<<<grid, 256, 0, a.stream>>>(p);
  return hipGetLastError();
}

}  // namespace mla
