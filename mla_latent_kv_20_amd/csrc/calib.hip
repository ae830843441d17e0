// Calibration kernels: the achievable bf16 MFMA rate and HBM read rate of the device, measured
// beside the published peaks.  Not part of the decode path; the benchmark times them.
#include "../../include/mla_calib.h"

#include "mla_common.h"

namespace mla {
namespace {

constexpr int kCalibWaves = 4;
constexpr int kCalibThreads = kCalibWaves * 64;
constexpr int kChains = 4;                // independent accumulators per wave

// Back-to-back v_mfma_f32_32x32x16_bf16 on every SIMD: kChains independent accumulator chains
// per wave, one wave per SIMD, operands in registers.
__global__ void __launch_bounds__(kCalibThreads, 1) calib_mfma_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)i);
  }
  f32x16 c[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) c[j][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = mfma32x32x16(a, b, c[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[j][i];
  out[blockIdx.x * kCalibThreads + threadIdx.x] = s;
}

// Streaming read: workgroup g reads bytes [g * per_wg, (g + 1) * per_wg) of src as 36 KiB
// tiles of 16-byte direct-to-LDS loads (9 per wave), one tile in flight behind the one
// landing -- the decode's own load form, without its compute.
constexpr int kTile = 36864;
constexpr int kLoadsPerWave = kTile / (kCalibWaves * 1024);   // 9

__global__ void __launch_bounds__(kCalibThreads, 1) calib_read_kernel(const char* src, int64_t tiles_per_wg,
                                                                      float* out) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const char* s = src + (size_t)blockIdx.x * (size_t)tiles_per_wg * kTile;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  for (int64_t t = 0; t < tiles_per_wg; ++t) {
    const char* tsrc = s + (size_t)t * kTile;
    const uint32_t stage = lds0 + (uint32_t)(t & 1) * kTile;
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      const int blk = wave * kLoadsPerWave + i;
      global_to_lds16_sv(tsrc, (uint32_t)(blk * 1024 + lane * 16), __builtin_amdgcn_readfirstlane(stage + blk * 1024));
    }
    if (t > 0) wait_vmcnt<kLoadsPerWave>();       // the previous tile has landed
    lds_barrier();
  }
  wait_vmcnt<0>();
  lds_barrier();
  if (threadIdx.x == 0) out[blockIdx.x] = (float)smem[(blockIdx.x * 7) % (2 * kTile)];
}

}  // namespace
}  // namespace mla

extern "C" {

int32_t mla_calib_mfma_grid(void) { return 1024; }

mla_status_t mla_calib_mfma(int32_t iters, float* out, hipStream_t stream) {
  if (iters < 1) return MLA_ERR_SHAPE;
  if (!out) return MLA_ERR_NULL;
  hipLaunchKernelGGL(mla::calib_mfma_kernel, dim3(1024), dim3(mla::kCalibThreads), 0, stream, iters, out);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

double mla_calib_mfma_flop(int32_t iters) {
  return iters < 1 ? 0.0 : 1024.0 * mla::kCalibWaves * (double)iters * mla::kChains * (2.0 * 32 * 32 * 16);
}

mla_status_t mla_calib_read(const void* src, int64_t bytes, int32_t workgroups, float* out, hipStream_t stream) {
  if (!src || !out) return MLA_ERR_NULL;
  if (workgroups < 1 || bytes < 0) return MLA_ERR_SHAPE;
  if (((uintptr_t)src & 15) != 0) return MLA_ERR_ALIGN;
  const int64_t tiles = bytes / ((int64_t)workgroups * mla::kTile);
  if (tiles < 1) return MLA_ERR_SHAPE;
  static const hipError_t attr = hipFuncSetAttribute((const void*)mla::calib_read_kernel,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 2 * mla::kTile);
  if (attr != hipSuccess) return MLA_ERR_LAUNCH;
  hipLaunchKernelGGL(mla::calib_read_kernel, dim3(workgroups), dim3(mla::kCalibThreads), 2 * mla::kTile, stream,
                     (const char*)src, tiles, out);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

int64_t mla_calib_read_bytes(int64_t bytes, int32_t workgroups) {
  if (workgroups < 1 || bytes < 0) return 0;
  return bytes / ((int64_t)workgroups * mla::kTile) * (int64_t)workgroups * mla::kTile;
}

}  // extern "C"
