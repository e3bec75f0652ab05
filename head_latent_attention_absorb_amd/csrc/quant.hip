// Low-bit cache rows: OCP E4M3 codes with one fp32 scale per row.
//
// At deployment the KV cache is quantised to about 6 bits per element
// (ai-library "DeepSeek-V2" notes, "Training and Inference Efficiency" /
// "Inference cost"), with scales computed online from the data (V3
// read-through, 2kiu.com/news/6340724, section 4.4).  Here every row of the
// cache, [c^KV | k^R], gets the scale s = max|x| / 448 (448 being E4M3's
// largest finite value; 1 for an all-zero row) and the codes E4M3(x / s),
// rounded to nearest with ties to even.  Both divisions are IEEE fp32
// divisions, so the codes are a fixed function of the fp32 inputs.
//
// One wave per row: lanes take consecutive element pairs, the row maximum is
// a wave reduction, and each pair is converted with v_cvt_pk_fp8_f32 and
// stored as two bytes.

#include "device_common.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr float kE4m3Max = 448.f;

template <typename T>
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(const T* __restrict__ src,
                                                                 uint8_t* __restrict__ dst,
                                                                 float* __restrict__ scales,
                                                                 int64_t n_rows, int width) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (r >= n_rows) return;
  const T* x = src + r * width;
  float amax = 0.f;
  for (int j = lane; j < width; j += 64) amax = fmaxf(amax, fabsf(ld(x + j)));
  amax = wave_max(amax);
  const float s = amax > 0.f ? amax / kE4m3Max : 1.f;
  uint8_t* q = dst + r * width;
  for (int j = 2 * lane; j < width; j += 128) {
    const float a = fminf(fmaxf(ld(x + j) / s, -kE4m3Max), kE4m3Max);
    const float b = j + 1 < width ? fminf(fmaxf(ld(x + j + 1) / s, -kE4m3Max), kE4m3Max) : 0.f;
    const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    q[j] = static_cast<uint8_t>(packed & 0xFF);
    if (j + 1 < width) q[j + 1] = static_cast<uint8_t>((packed >> 8) & 0xFF);
  }
  if (lane == 0) scales[r] = s;
}

}  // namespace

hipError_t launch_quantize_rows(int src_dtype, int64_t n_rows, int width, const void* src,
                                void* dst, float* scales, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  const int64_t blocks = (n_rows + kThreads / 64 - 1) / (kThreads / 64);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (src_dtype == 1)
    quantize_rows_kernel<__bf16><<<static_cast<unsigned>(blocks), kThreads, 0, stream>>>(
        static_cast<const __bf16*>(src), static_cast<uint8_t*>(dst), scales, n_rows, width);
  else
    quantize_rows_kernel<float><<<static_cast<unsigned>(blocks), kThreads, 0, stream>>>(
        static_cast<const float*>(src), static_cast<uint8_t*>(dst), scales, n_rows, width);
  return hipGetLastError();
}

}  // namespace mla
