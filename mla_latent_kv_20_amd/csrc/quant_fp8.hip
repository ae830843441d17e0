// Quantized latent cache: rows [c^KV ; k^R] to FP8 E4M3 codes with one scale per row.
//
// Pages cited: [review] "DeepSeek-V2 review", section 4 ("Inference efficiency": the served
// model's KV cache is quantized to about 6 bits per element); [report] "Техотчёт DeepSeek-V2
// (2024): MLA и экономика инференса", the 93.3% derivation and the economics section.  The
// pages name no format; this one is OCP FP8 E4M3 ("fn": bias 7, largest value 448, no
// infinity) for every element of the row and one fp32 scale per row:
//
//   s_r    = amax_r / 448                   (fp32, correctly rounded; amax_r = max |x_rk|)
//   code   = E4M3 nearest to fp32(x / s_r), ties to even, magnitudes above 448 saturated
//   x^     = value(code) * s_r
// A row of zeros gets s_r = 0 and all codes 0.  Every decision is taken in fp32.
//
// One wave per row; not on the decode's hot loop (it runs once per new row).
#include "mla_common.h"

namespace mla {
namespace {

constexpr int kQWaves = 4;

struct QuantParams {
  const void* src;          // [n, src_stride] bf16 or fp32
  int64_t src_stride;       // elements
  const int64_t* dst;       // [n] code row of source row i, or null: row i
  uint8_t* codes;           // code rows of code_stride bytes
  int64_t code_stride;
  float* scales;            // one per code row
  int64_t n;
  int width;                // d_c + d_r
  bool bf16;
};

// E4M3 code of y (sign bit from y), nearest value, ties to even, saturated at 448.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t bits = __float_as_uint(y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t mag;
  if (a < 0.015625f) {                          // below 2^-6: steps of 2^-9, codes 0..8
    mag = (uint32_t)__builtin_rintf(a * 512.0f);  // exact scaling; rint rounds ties to even
  } else {
    const uint32_t ab = bits & 0x7fffffffu;
    const int e = (int)(ab >> 23) - 127;        // a in [2^e, 2^(e+1)), e >= -6
    if (e > 8) {
      mag = 0x7Eu;
    } else {
      const uint32_t m = ab & 0x7fffffu;
      const uint32_t keep = ((uint32_t)(e + 7) << 3) | (m >> 20);   // exponent and 3 mantissa bits
      const uint32_t rest = m & 0xfffffu;                          // the 20 bits dropped
      const uint32_t up = (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ? 1u : 0u;
      mag = keep + up;                          // a carry moves to the next binade
    }
  }
  return sign | (mag > 0x7Eu ? 0x7Eu : mag);
}

__global__ void __launch_bounds__(kQWaves * 64)
quantize_rows_kernel(QuantParams P) {
  const int64_t row = (int64_t)blockIdx.x * kQWaves + (threadIdx.x >> 6);
  if (row >= P.n) return;                       // wave-uniform
  const int lane = threadIdx.x & 63;
  const int per_lane = (P.width + 63) / 64;     // <= 16
  float x[16];
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int e = lane + 64 * k;
    x[k] = 0.f;
    if (k < per_lane && e < P.width) {
      x[k] = P.bf16 ? bf16_to_f32(((const bf16_bits*)P.src)[row * P.src_stride + e])
                    : ((const float*)P.src)[row * P.src_stride + e];
      amax = fmaxf(amax, fabsf(x[k]));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float s = amax / 448.0f;                // correctly rounded fp32 division
  const int64_t out = P.dst ? P.dst[row] : row;
  uint8_t* c = P.codes + out * P.code_stride;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int e = lane + 64 * k;
    if (k < per_lane && e < P.width) c[e] = (uint8_t)(s > 0.f ? e4m3_code(x[k] / s) : 0u);
  }
  if (lane == 0) P.scales[out] = s;
}

}  // namespace

bool quantize_rows_supported(int width) { return width > 0 && width <= 1024; }

hipError_t launch_quantize_rows(bool bf16, const void* src, int64_t src_stride, int64_t n,
                                const int64_t* dst_rows, uint8_t* codes, int64_t code_stride, float* scales,
                                int width, hipStream_t stream) {
  QuantParams P{src, src_stride, dst_rows, codes, code_stride, scales, n, width, bf16};
  const int64_t blocks = (n + kQWaves - 1) / kQWaves;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)blocks), dim3(kQWaves * 64), 0, stream, P);
  return hipGetLastError();
}

}  // namespace mla
