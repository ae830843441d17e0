// Split-KV log-sum-exp merge and the plain fp32 kernels of the MLA decode library.
//
// Pages cited: [notes] "MLA(Multi-head Latent Attention): DeepSeek-V2 논문정리";
// [report] "Техотчёт DeepSeek-V2 (2024): MLA и экономика инференса";
// [v3] DeepSeek-V3 Technical Report notes (xuxeong.tistory.com).
//
// merge: softmax over the union of disjoint row sets.  With M = max_s lse_s and
// w_s = exp(lse_s - M), o = sum_s w_s o_s / sum_s w_s and lse = M + ln sum_s w_s.
// A split of weight zero (an empty split, lse = -inf, whose o_s the decode does not
// write) is left out of the sum, so whatever its o_s holds never enters it.
//
// The fp32 kernels compute the same four steps with no bf16 rounding, for any shape.
// They are simple (one thread per output element, or one workgroup per query head)
// and serve the fp32 dtype, whose use is exactness on small problems.
#include "mla_common.h"

namespace mla {
namespace {

// ---------------------------------------------------------------------------
// merge: one wave per (query, head); lane l owns 8 consecutive outputs of each 512-wide
// stripe, read as 16 bytes (fp16 partials) or 2 x 16 bytes (fp32).  The split weights
// depend only on the (query, head), so every lane computes them from the same lse values.
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 256;
constexpr int kMergeWaves = kMergeThreads / 64;
constexpr int kFastSplits = 8;
static_assert(kFastSplits == 8, "the split-weight sum of the fast path is written out for 8 splits");

template <typename PartT>
__device__ __forceinline__ void load8(const PartT* p, float* v);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
}
template <>
__device__ __forceinline__ void load8<_Float16>(const _Float16* p, float* v) {
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  const f16x8 a = *(const f16x8*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
}
template <typename PartT>
__device__ __forceinline__ float load1(const PartT* p) { return (float)*p; }

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// The lse values of up to 64 splits are held one per lane; the weights w_s = exp(lse_s - M)
// are broadcast from lane s.  More splits go in chunks of 64.
template <typename PartT>
__global__ void __launch_bounds__(kMergeThreads)
merge_splits_kernel(const PartT* __restrict__ o_part, const float* __restrict__ lse_part,
                    float* __restrict__ o_lat, float* __restrict__ lse, int qh_count, int d_c,
                    int num_splits) {
  const int qh = __builtin_amdgcn_readfirstlane(blockIdx.x * kMergeWaves + (threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  if (qh >= qh_count) return;
  if (num_splits <= kFastSplits && d_c == 8 * 64) {
    // One 512-wide stripe and at most 8 splits: every load (the lse values and all partial
    // rows) is issued before the first reduction, so the wave waits on one memory latency.
    // Every lane holds all the split lse values (wave-uniform loads), so the maximum, the
    // weights and their sum need no cross-lane exchange; the sum runs in the tree a
    // butterfly over lanes 0..7 forms, ((w0 + w4) + (w2 + w6)) + ((w1 + w5) + (w3 + w7)),
    // with zero weights for absent splits.
    // The loads are unconditional (a split past the last re-reads the last one; its weight
    // is zero): a load under a branch leaves its register undefined on the other path, and
    // the compiler then waits for it before issuing the next.  The rows stay raw 16-byte
    // vectors until they are used (measured faster here than converting each on arrival).
    constexpr int kVec = 16 / (int)sizeof(PartT);        // elements per 16-byte load
    typedef PartT pvec __attribute__((ext_vector_type(kVec)));
    float lse_s[kFastSplits];
    pvec raw[kFastSplits][8 / kVec];
#pragma unroll
    for (int k = 0; k < kFastSplits; ++k) {
      const int kk = k < num_splits ? k : num_splits - 1;
      lse_s[k] = lse_part[(size_t)kk * qh_count + qh];
#pragma unroll
      for (int h = 0; h < 8 / kVec; ++h)
        raw[k][h] = *(const pvec*)(o_part + ((size_t)kk * qh_count + qh) * d_c + 8 * lane + kVec * h);
    }
#pragma unroll
    for (int k = 0; k < kFastSplits; ++k)
      if (k >= num_splits) lse_s[k] = -INFINITY;
    float M = lse_s[0];
#pragma unroll
    for (int k = 1; k < kFastSplits; ++k) M = fmaxf(M, lse_s[k]);
    // No branch between the loads and their use (the compiler would otherwise sink the
    // loads below it): a row that no split saw (M = -inf) gets zero weights and, at the end,
    // zero outputs and lse = -inf.
    const bool none = M == -INFINITY;
    const float m_ref = none ? 0.f : M;
    float w[kFastSplits];
#pragma unroll
    for (int k = 0; k < kFastSplits; ++k) w[k] = k < num_splits ? expf(lse_s[k] - m_ref) : 0.f;
    const float z = ((w[0] + w[4]) + (w[2] + w[6])) + ((w[1] + w[5]) + (w[3] + w[7]));
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kFastSplits; ++k) {
      const float ws = w[k];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = ws != 0.f ? fmaf(ws, (float)raw[k][e / kVec][e % kVec], acc[e]) : acc[e];
    }
    const float inv_z = 1.0f / z;
    float* out = o_lat + (size_t)qh * d_c + 8 * lane;
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = none ? 0.f : acc[e] * inv_z;
    *(f32x4*)out = f32x4{r[0], r[1], r[2], r[3]};
    *(f32x4*)(out + 4) = f32x4{r[4], r[5], r[6], r[7]};
    if (lane == 0) lse[qh] = none ? -INFINITY : M + logf(z);
    return;
  }
  // Up to 64 splits: lane s holds split s's lse (one load).  Splits of weight zero (empty
  // ones) are not accumulated, and their rows are not fetched from memory.
  const bool one_chunk = num_splits <= 64;
  float lse_l = -INFINITY;
  float M;
  if (one_chunk) {
    lse_l = lane < num_splits ? lse_part[(size_t)lane * qh_count + qh] : -INFINITY;
    M = wave_max(lse_l);
  } else {
    M = -INFINITY;
    for (int s0 = 0; s0 < num_splits; s0 += 64) {
      const int s = s0 + lane;
      M = fmaxf(M, s < num_splits ? lse_part[(size_t)s * qh_count + qh] : -INFINITY);
    }
    M = wave_max(M);
  }
  float* out = o_lat + (size_t)qh * d_c;
  if (M == -INFINITY) {                           // no split saw a row
    for (int c = lane; c < d_c; c += 64) out[c] = 0.f;
    if (lane == 0) lse[qh] = -INFINITY;
    return;
  }
  const float w_own = expf(lse_l - M);             // one_chunk: this lane's split weight
  float z;
  if (one_chunk) {
    z = wave_sum(w_own);
  } else {
    z = 0.f;
    for (int s0 = 0; s0 < num_splits; s0 += 64) {
      const int s = s0 + lane;
      z += s < num_splits ? expf(lse_part[(size_t)s * qh_count + qh] - M) : 0.f;
    }
    z = wave_sum(z);
  }
  const float inv_z = 1.0f / z;
  const bool vec = (d_c & 7) == 0;
  for (int c = vec ? 8 * lane : lane; c < d_c; c += vec ? 8 * 64 : 64) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < num_splits; s0 += 64) {
      const int sl = s0 + lane;
      const float wl = one_chunk ? w_own : (sl < num_splits ? expf(lse_part[(size_t)sl * qh_count + qh] - M) : 0.f);
      const int cnt = num_splits - s0 < 64 ? num_splits - s0 : 64;
      int u = 0;
      for (; u + 8 <= cnt; u += 8) {               // eight splits' loads in flight
        float ws[8];
        float v[8][8];
#pragma unroll
        for (int k = 0; k < 8; ++k) ws[k] = __shfl(wl, u + k);
        // a split of weight zero re-reads the chunk's first row (a cache hit), so that all
        // eight loads go out unconditionally and back to back
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const PartT* p = o_part + ((size_t)(s0 + u + (ws[k] != 0.f ? k : 0)) * qh_count + qh) * d_c + c;
          if (vec) load8(p, v[k]);
          else v[k][0] = load1(p);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = ws[k] != 0.f ? fmaf(ws[k], v[k][e], acc[e]) : acc[e];
        }
      }
      for (; u < cnt; ++u) {
        const float ws = __shfl(wl, u);
        if (ws != 0.f) {
          float v[8];
          const PartT* p = o_part + ((size_t)(s0 + u) * qh_count + qh) * d_c + c;
          if (vec) load8(p, v);
          else v[0] = load1(p);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(ws, v[e], acc[e]);
        }
      }
    }
    if (vec) {
      *(f32x4*)(out + c) = f32x4{acc[0] * inv_z, acc[1] * inv_z, acc[2] * inv_z, acc[3] * inv_z};
      *(f32x4*)(out + c + 4) = f32x4{acc[4] * inv_z, acc[5] * inv_z, acc[6] * inv_z, acc[7] * inv_z};
    } else {
      out[c] = acc[0] * inv_z;
    }
  }
  if (lane == 0) lse[qh] = M + logf(z);
}

// ---------------------------------------------------------------------------
// fp32 absorb_q: one thread per output element.
// ---------------------------------------------------------------------------
__global__ void absorb_q_f32_kernel(const float* __restrict__ q_c, const float* __restrict__ q_r,
                                    const float* __restrict__ w_uk, float* __restrict__ q_abs,
                                    int n_q, int n_h, int d_h, int d_c, int d_r,
                                    const int64_t* __restrict__ pos, RopeSpec rope) {
  const int d_qk = d_c + d_r;
  const size_t total = (size_t)n_q * n_h * d_qk;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const int c = (int)(e % d_qk);
    const size_t ni = e / d_qk;                    // n * n_h + i
    const int i = (int)(ni % n_h);
    if (c < d_c) {
      const float* q = q_c + ni * d_h;
      const float* w = w_uk + (size_t)i * d_h * d_c + c;
      float acc = 0.f;
      for (int d = 0; d < d_h; ++d) acc = fmaf(q[d], w[(size_t)d * d_c], acc);
      q_abs[e] = acc;
    } else if (pos == nullptr) {
      q_abs[e] = q_r[ni * d_r + (c - d_c)];
    } else {                                       // rotated at the token's position
      const int half = d_r / 2;
      const int k = c - d_c;
      const int k0 = k < half ? k : k - half;
      double x = q_r[ni * d_r + k0], y = q_r[ni * d_r + k0 + half];
      rope_pair(x, y, pos[ni / n_h], k0, d_r, rope);
      q_abs[e] = (float)(k < half ? x : y);
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 decode: one workgroup per (query, split, head).  Rows go 256 at a time: each
// thread scores one row, the block takes the max and the sum, and the latent
// accumulator (in LDS) is rescaled and updated with the block's weights.
// ---------------------------------------------------------------------------
constexpr int kDecThreads = 256;

__device__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int k = 1; k < kDecThreads / 64; ++k) r = fmaxf(r, red[k]);
  return r;
}
__device__ float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = 0.f;
  for (int k = 0; k < kDecThreads / 64; ++k) r += red[k];
  return r;
}

__global__ void __launch_bounds__(kDecThreads)
decode_f32_kernel(const float* __restrict__ q_abs, const float* __restrict__ c_kv, int64_t c_stride,
                  const float* __restrict__ k_r, int64_t r_stride, const int64_t* __restrict__ offsets,
                  float* __restrict__ o_part, float* __restrict__ lse_part, int n_q, int n_h, int d_c,
                  int d_r, int q_per_seq, int num_splits, int split_rows, float scale) {
  extern __shared__ float sm[];
  const int d_qk = d_c + d_r;
  float* q = sm;                  // [d_qk]
  float* o = q + d_qk;            // [d_c]
  float* p = o + d_c;             // [256]
  float* red = p + kDecThreads;   // [4]
  const int i = blockIdx.x;
  const int s = blockIdx.y;
  const int n = blockIdx.z;
  const int b = n / q_per_seq, r = n - b * q_per_seq;
  const int64_t row0 = offsets[b];
  const int64_t vis = offsets[b + 1] - row0 - q_per_seq + r + 1;
  int64_t lo = 0, hi = vis;
  if (num_splits > 1) {
    lo = (int64_t)s * split_rows;
    hi = (s == num_splits - 1) ? vis : lo + split_rows;
    lo = lo < vis ? lo : vis;
    hi = hi < vis ? hi : vis;
  }
  if (lo < 0) lo = 0;
  const size_t qh = (size_t)n * n_h + i;
  for (int c = threadIdx.x; c < d_qk; c += kDecThreads) q[c] = q_abs[qh * d_qk + c];
  for (int c = threadIdx.x; c < d_c; c += kDecThreads) o[c] = 0.f;
  float m = -INFINITY, l = 0.f;
  __syncthreads();
  for (int64_t j0 = lo; j0 < hi; j0 += kDecThreads) {
    const int64_t j = j0 + threadIdx.x;
    float x = -INFINITY;
    if (j < hi) {
      const float* cr = c_kv + (row0 + j) * c_stride;
      const float* rr = k_r + (row0 + j) * r_stride;
      float acc = 0.f;
      for (int c = 0; c < d_c; ++c) acc = fmaf(q[c], cr[c], acc);
      for (int c = 0; c < d_r; ++c) acc = fmaf(q[d_c + c], rr[c], acc);
      x = acc * scale;
    }
    const float mt = block_max(x, red);
    const float m_new = fmaxf(m, mt);
    const float alpha = expf(m - m_new);        // 0 on the first block (m = -inf)
    const float pj = (j < hi) ? expf(x - m_new) : 0.f;
    p[threadIdx.x] = pj;
    const float lt = block_sum(pj, red);          // also orders the p[] writes
    l = l * alpha + lt;
    m = m_new;
    const int cnt = (int)((hi - j0) < kDecThreads ? (hi - j0) : kDecThreads);
    for (int c = threadIdx.x; c < d_c; c += kDecThreads) {
      float acc = o[c] * alpha;
      for (int jj = 0; jj < cnt; ++jj) acc = fmaf(p[jj], c_kv[(row0 + j0 + jj) * c_stride + c], acc);
      o[c] = acc;
    }
    __syncthreads();
  }
  const size_t out = (size_t)s * n_q * n_h + qh;
  if (hi <= lo) {                                 // empty split: lse = -inf, o_part not written
    if (threadIdx.x == 0) lse_part[out] = -INFINITY;
    return;
  }
  const float inv = 1.0f / l;
  for (int c = threadIdx.x; c < d_c; c += kDecThreads) o_part[out * d_c + c] = o[c] * inv;
  if (threadIdx.x == 0) lse_part[out] = m + logf(l);
}

// ---------------------------------------------------------------------------
// fp32 out_proj: one thread per output element.
// ---------------------------------------------------------------------------
__global__ void out_proj_f32_kernel(const float* __restrict__ o_lat, const float* __restrict__ w_uv,
                                    float* __restrict__ o_c, int n_q, int n_h, int d_h, int d_c) {
  const size_t total = (size_t)n_q * n_h * d_h;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const int d = (int)(e % d_h);
    const size_t ni = e / d_h;
    const int i = (int)(ni % n_h);
    const float* a = o_lat + ni * d_c;
    const float* w = w_uv + ((size_t)i * d_h + d) * d_c;
    float acc = 0.f;
    for (int c = 0; c < d_c; ++c) acc = fmaf(w[c], a[c], acc);
    o_c[e] = acc;
  }
}

unsigned grid_for(size_t total, int threads) {
  size_t g = (total + threads - 1) / threads;
  return (unsigned)(g < 65536 ? (g ? g : 1) : 65536);
}

}  // namespace

hipError_t launch_merge(const void* o_part, bool f16_partials, const float* lse_part, float* o_lat,
                        float* lse, int n_q, int n_h, int d_c, int num_splits, hipStream_t stream) {
  const int qh = n_q * n_h;
  const dim3 grid((qh + kMergeWaves - 1) / kMergeWaves);
  if (f16_partials)
    hipLaunchKernelGGL(merge_splits_kernel<_Float16>, grid, dim3(kMergeThreads), 0, stream,
                       (const _Float16*)o_part, lse_part, o_lat, lse, qh, d_c, num_splits);
  else
    hipLaunchKernelGGL(merge_splits_kernel<float>, grid, dim3(kMergeThreads), 0, stream,
                       (const float*)o_part, lse_part, o_lat, lse, qh, d_c, num_splits);
  return hipGetLastError();
}

hipError_t launch_absorb_q_f32(const float* q_c, const float* q_r, const float* w_uk, float* q_abs,
                               int n_q, int n_h, int d_h, int d_c, int d_r, const int64_t* positions,
                               const RopeSpec& rope, hipStream_t stream) {
  const size_t total = (size_t)n_q * n_h * (d_c + d_r);
  hipLaunchKernelGGL(absorb_q_f32_kernel, dim3(grid_for(total, 256)), dim3(256), 0, stream, q_c, q_r,
                     w_uk, q_abs, n_q, n_h, d_h, d_c, d_r, positions, rope);
  return hipGetLastError();
}

size_t decode_f32_smem_bytes(int d_c, int d_r) {
  return sizeof(float) * ((size_t)2 * d_c + d_r + kDecThreads + 4);
}

hipError_t launch_decode_f32(const float* q_abs, const float* c_kv, int64_t c_stride, const float* k_r,
                             int64_t r_stride, const int64_t* offsets, float* o_part, float* lse_part,
                             int batch, int q_per_seq, int n_h, int d_c, int d_r, int num_splits,
                             int split_rows, float scale, hipStream_t stream) {
  const int n_q = batch * q_per_seq;
  const size_t smem = decode_f32_smem_bytes(d_c, d_r);
  hipLaunchKernelGGL(decode_f32_kernel, dim3(n_h, num_splits, n_q), dim3(kDecThreads), smem, stream,
                     q_abs, c_kv, c_stride, k_r, r_stride, offsets, o_part, lse_part, n_q, n_h, d_c,
                     d_r, q_per_seq, num_splits, split_rows, scale);
  return hipGetLastError();
}

hipError_t launch_out_proj_f32(const float* o_lat, const float* w_uv, float* o_c, int n_q, int n_h,
                               int d_h, int d_c, hipStream_t stream) {
  const size_t total = (size_t)n_q * n_h * d_h;
  hipLaunchKernelGGL(out_proj_f32_kernel, dim3(grid_for(total, 256)), dim3(256), 0, stream, o_lat,
                     w_uv, o_c, n_q, n_h, d_h, d_c);
  return hipGetLastError();
}

}  // namespace mla
