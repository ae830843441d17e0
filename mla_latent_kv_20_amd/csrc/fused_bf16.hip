// Split merge fused with the value up-projection, bf16 MFMA on gfx950.
//
// Pages cited: [notes] "MLA(Multi-head Latent Attention): DeepSeek-V2 논문정리";
// [report] "Техотчёт DeepSeek-V2 (2024): MLA и экономика инференса".
//
// For each (query n, head i):
//   M = max_s lse_s, w_s = exp(lse_s - M), o_lat = sum_s w_s o_s / sum_s w_s,
//   lse = M + ln sum_s w_s        (softmax over the union of the splits' disjoint rows)
//   o_c[n, i, :] = W^UV_i o_lat   ([notes] "Value에 대한 수식 전개")
// o_lat stays on chip: it is rounded to bf16 into LDS, where it is the MFMA A operand.
// The arithmetic follows mla_merge_splits and then mla_out_proj operation for operation
// (same split order, same reductions, same k split of the projection), so the outputs
// equal those of the two calls bit for bit; only the fp32 o_lat round trip through HBM
// and one launch are gone.
#include "mla_common.h"

namespace mla {
namespace {

constexpr int kFThreads = 512;
constexpr int kFWaves = kFThreads / 64;
constexpr int kFDc = 512;                    // latent width handled (one 512-wide stripe)
constexpr int kFQBlock = 32;                 // query rows per round (the MFMA M dimension)
constexpr int kFPitch = kFDc * 2 + 16;       // bf16 o_lat row in LDS, padded against conflicts
constexpr int kFCols = 64;                   // output columns (of d_h) per workgroup
constexpr int kFSteps = kFDc / 64;           // k-steps of 16 per wave: a quarter of d_c
constexpr int kFFast = 8;                    // splits whose loads all go out at once

struct FusedParams {
  const void* o_part;      // [S, n_q, n_h, 512] fp16 or fp32
  const float* lse_part;   // [S, n_q, n_h]
  const bf16_bits* w_uv;   // [n_h, d_h, 512]
  bf16_bits* o_c;          // [n_q, n_h, d_h]
  float* lse;              // [n_q, n_h] or null
  float* o_lat;            // [n_q, n_h, 512] or null
  int n_q, n_h, d_h, num_splits;
};

template <typename PartT>
__device__ __forceinline__ void load8p(const PartT* p, float* v);
template <>
__device__ __forceinline__ void load8p<float>(const float* p, float* v) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
}
template <>
__device__ __forceinline__ void load8p<_Float16>(const _Float16* p, float* v) {
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  const f16x8 a = *(const f16x8*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
}

__device__ __forceinline__ float fwave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float fwave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Merge of one (query, head): lane l returns outputs 8l .. 8l+7 (o = acc / z), with M and z.
// M == -inf means no split saw a row (the outputs are then zero).
template <typename PartT>
__device__ __forceinline__ void merge_one(const PartT* o_part, const float* lse_part, int qh_count,
                                          int qh, int num_splits, int lane, float* o, float& M,
                                          float& z) {
  if (num_splits <= kFFast) {
    const float lse_l = lane < num_splits ? lse_part[(size_t)lane * qh_count + qh] : -INFINITY;
    float v[kFFast][8];
#pragma unroll
    for (int k = 0; k < kFFast; ++k)
      if (k < num_splits) load8p(o_part + ((size_t)k * qh_count + qh) * kFDc + 8 * lane, v[k]);
    M = fwave_max(lse_l);
    if (M == -INFINITY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = 0.f;
      z = 0.f;
      return;
    }
    const float w_l = expf(lse_l - M);
    z = fwave_sum(w_l);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kFFast; ++k) {
      if (k < num_splits) {
        const float ws = __shfl(w_l, k);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(ws, v[k][e], acc[e]);
      }
    }
    const float inv_z = 1.0f / z;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = acc[e] * inv_z;
    return;
  }
  M = -INFINITY;
  for (int s0 = 0; s0 < num_splits; s0 += 64) {
    const int s = s0 + lane;
    M = fmaxf(M, s < num_splits ? lse_part[(size_t)s * qh_count + qh] : -INFINITY);
  }
  M = fwave_max(M);
  if (M == -INFINITY) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    z = 0.f;
    return;
  }
  z = 0.f;
  for (int s0 = 0; s0 < num_splits; s0 += 64) {
    const int s = s0 + lane;
    z += s < num_splits ? expf(lse_part[(size_t)s * qh_count + qh] - M) : 0.f;
  }
  z = fwave_sum(z);
  const float inv_z = 1.0f / z;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int c = 8 * lane;
  for (int s0 = 0; s0 < num_splits; s0 += 64) {
    const int sl = s0 + lane;
    const float wl = sl < num_splits ? expf(lse_part[(size_t)sl * qh_count + qh] - M) : 0.f;
    const int cnt = num_splits - s0 < 64 ? num_splits - s0 : 64;
    int u = 0;
    for (; u + 8 <= cnt; u += 8) {
      float v[8][8];
#pragma unroll
      for (int k = 0; k < 8; ++k) load8p(o_part + ((size_t)(s0 + u + k) * qh_count + qh) * kFDc + c, v[k]);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float ws = __shfl(wl, u + k);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(ws, v[k][e], acc[e]);
      }
    }
    for (; u < cnt; ++u) {
      float v[8];
      load8p(o_part + ((size_t)(s0 + u) * qh_count + qh) * kFDc + c, v);
      const float ws = __shfl(wl, u);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(ws, v[e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = acc[e] * inv_z;
}

// Fast path (num_splits <= 8) for kRows (query, head) rows at once: every load of the
// rows (lse values and split results, kept as raw 16-byte vectors) is issued before the
// first reduction, so the wave waits on one memory latency for all of them.  Per row the
// arithmetic is that of merge_one.
template <typename PartT, int kRows>
__device__ __forceinline__ void merge_rows_fast(const PartT* o_part, const float* lse_part,
                                                int qh_count, const int* qh, int nrows,
                                                int num_splits, int lane, float (*o)[8], float* M,
                                                float* z) {
  constexpr int kVec = 16 / (int)sizeof(PartT);       // elements per 16-byte load
  typedef PartT pvec __attribute__((ext_vector_type(kVec)));
  float lse_l[kRows];
  pvec raw[kRows][kFFast][8 / kVec];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const bool live = r < nrows;
    lse_l[r] = live && lane < num_splits ? lse_part[(size_t)lane * qh_count + qh[r]] : -INFINITY;
#pragma unroll
    for (int k = 0; k < kFFast; ++k)
      if (live && k < num_splits)
#pragma unroll
        for (int h = 0; h < 8 / kVec; ++h)
          raw[r][k][h] = *(const pvec*)(o_part + ((size_t)k * qh_count + qh[r]) * kFDc + 8 * lane + kVec * h);
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    if (r >= nrows) break;
    M[r] = fwave_max(lse_l[r]);
    if (M[r] == -INFINITY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][e] = 0.f;
      z[r] = 0.f;
      continue;
    }
    const float w_l = expf(lse_l[r] - M[r]);
    z[r] = fwave_sum(w_l);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kFFast; ++k) {
      if (k < num_splits) {
        const float ws = __shfl(w_l, k);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(ws, (float)raw[r][k][e / kVec][e % kVec], acc[e]);
      }
    }
    const float inv_z = 1.0f / z[r];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[r][e] = acc[e] * inv_z;
  }
}

// Workgroup = (head i, block of 64 output columns); workgroups are dealt round-robin over
// the 8 XCDs and the column blocks of head i all run on XCD i % 8, so the head's split
// results are fetched into one L2.  Per round of 32 queries: each of the 8 waves merges
// 4 (query, head) rows into LDS; then wave w multiplies the block by W^UV for column
// half (w & 1) over k quarter (w >> 1), and the four k quarters are summed through LDS.
template <typename PartT>
__global__ void __launch_bounds__(kFThreads)
merge_out_proj_kernel(FusedParams P) {
  __shared__ __attribute__((aligned(16))) char o_lds[kFQBlock * kFPitch];
  __shared__ f32x16 red[kFWaves][64];
  const int nblk = P.d_h / kFCols;
  const int xcd = blockIdx.x & 7;
  const int kq = blockIdx.x >> 3;
  const int i = (kq / nblk) * 8 + xcd;
  const int cb = (kq % nblk) * kFCols;
  if (i >= P.n_h) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int qh_count = P.n_q * P.n_h;
  const PartT* o_part = (const PartT*)P.o_part;

  // B operands, loaded once: lane l holds W^UV_i[ncol + l%32][k0 + 16s .. +7]
  const int half = wave & 1;
  const int kqtr = wave >> 1;
  const int ncol = cb + 32 * half;
  const int k0 = kqtr * kFSteps * 16 + 8 * (lane >> 5);
  bf16x8 wb[kFSteps];
  const bf16_bits* w = P.w_uv + ((size_t)i * P.d_h + ncol + (lane & 31)) * kFDc + k0;
#pragma unroll
  for (int s = 0; s < kFSteps; ++s) wb[s] = *(const bf16x8*)(w + 16 * s);

  for (int mb = 0; mb < P.n_q; mb += kFQBlock) {
    const int rows = P.n_q - mb < kFQBlock ? P.n_q - mb : kFQBlock;
    // ---- merge rows mb .. mb+rows-1 of head i into LDS as bf16; wave w takes rows
    // w, w + 8, w + 16, w + 24 (kRowsFast at a time when every split's loads fit in flight)
    constexpr int kRowsFast = 2;
    for (int r0 = wave; r0 < rows; r0 += kFWaves * kRowsFast) {
      int qh[kRowsFast];
      int nr = 0;
#pragma unroll
      for (int j = 0; j < kRowsFast; ++j) {
        const int r = r0 + j * kFWaves;
        qh[j] = (mb + (r < rows ? r : r0)) * P.n_h + i;
        nr += r < rows ? 1 : 0;
      }
      float o[kRowsFast][8], M[kRowsFast], z[kRowsFast];
      if (P.num_splits <= kFFast) {
        merge_rows_fast<PartT, kRowsFast>(o_part, P.lse_part, qh_count, qh, nr, P.num_splits, lane, o, M, z);
      } else {
        for (int j = 0; j < nr; ++j) merge_one(o_part, P.lse_part, qh_count, qh[j], P.num_splits, lane, o[j], M[j], z[j]);
      }
#pragma unroll
      for (int j = 0; j < kRowsFast; ++j) {
        if (j >= nr) break;
        const int r = r0 + j * kFWaves;
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        *(u32x4*)(o_lds + r * kFPitch + 16 * lane) =
            u32x4{pack_bf16x2(o[j][0], o[j][1]), pack_bf16x2(o[j][2], o[j][3]),
                  pack_bf16x2(o[j][4], o[j][5]), pack_bf16x2(o[j][6], o[j][7])};
        if (cb == 0) {
          if (P.o_lat) {
            float* dst = P.o_lat + (size_t)qh[j] * kFDc + 8 * lane;
            *(f32x4*)dst = f32x4{o[j][0], o[j][1], o[j][2], o[j][3]};
            *(f32x4*)(dst + 4) = f32x4{o[j][4], o[j][5], o[j][6], o[j][7]};
          }
          if (P.lse && lane == 0) P.lse[qh[j]] = M[j] == -INFINITY ? -INFINITY : M[j] + logf(z[j]);
        }
      }
    }
    __syncthreads();

    // ---- o_c block = o_lat block (bf16) . W^UV_i^T, this wave's k quarter
    const int m = lane & 31;
    const char* a = o_lds + (m < rows ? m : 0) * kFPitch + 2 * k0;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < kFSteps; ++s) acc = mfma32x32x16(*(const bf16x8*)(a + 32 * s), wb[s], acc);
    red[wave][lane] = acc;
    __syncthreads();
    // wave (half, kqtr) sums registers 4 kqtr .. 4 kqtr + 3 of column half `half` over the
    // four k quarters, in quarter order.  D[m][n]: lane l, reg r -> row 8(r/4) + 4(l/32) + r%4.
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 4 * kqtr + q;
      const float v = red[half][lane][r] + red[half + 2][lane][r] + red[half + 4][lane][r] +
                      red[half + 6][lane][r];
      const int mm = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (mm < rows)
        P.o_c[((size_t)(mb + mm) * P.n_h + i) * P.d_h + ncol + (lane & 31)] = f32_to_bf16(v);
    }
    __syncthreads();                               // o_lds and red are reused next round
  }
}

}  // namespace

bool merge_out_proj_bf16_supported(int d_h, int d_c) { return d_c == kFDc && d_h % kFCols == 0; }

hipError_t launch_merge_out_proj_bf16(const void* o_part, bool f16_partials, const float* lse_part,
                                      const bf16_bits* w_uv, bf16_bits* o_c, float* lse, float* o_lat,
                                      int n_q, int n_h, int d_h, int num_splits, hipStream_t stream) {
  FusedParams P{o_part, lse_part, w_uv, o_c, lse, o_lat, n_q, n_h, d_h, num_splits};
  const int grid = 8 * ((n_h + 7) / 8) * (d_h / kFCols);
  if (f16_partials)
    hipLaunchKernelGGL(merge_out_proj_kernel<_Float16>, dim3(grid), dim3(kFThreads), 0, stream, P);
  else
    hipLaunchKernelGGL(merge_out_proj_kernel<float>, dim3(grid), dim3(kFThreads), 0, stream, P);
  return hipGetLastError();
}

}  // namespace mla
