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
constexpr int kFPitch = kFDc * 2 + 16;       // bf16 o_lat row in LDS, padded against conflicts
constexpr int kFSteps = kFDc / 64;           // k-steps of 16 per wave: a quarter of d_c
constexpr int kFFast = 8;                    // splits whose loads all go out at once
static_assert(kFFast == 8, "the split-weight sum below is written out for 8 splits");
constexpr int kFWRowBytes = kFDc * 2;        // one W^UV row (bf16)

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
        for (int e = 0; e < 8; ++e) acc[e] = ws != 0.f ? fmaf(ws, v[k][e], acc[e]) : acc[e];
      }
    }
    const float inv_z = 1.0f / z;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = acc[e] * inv_z;
    return;
  }
  // Up to 64 splits: lane s holds split s's lse (one load).  Splits of weight zero (empty
  // ones) are not accumulated, and their rows are not fetched from memory.
  const bool one_chunk = num_splits <= 64;
  float lse_l = -INFINITY;
  if (one_chunk) {
    lse_l = lane < num_splits ? lse_part[(size_t)lane * qh_count + qh] : -INFINITY;
    M = fwave_max(lse_l);
  } else {
    M = -INFINITY;
    for (int s0 = 0; s0 < num_splits; s0 += 64) {
      const int s = s0 + lane;
      M = fmaxf(M, s < num_splits ? lse_part[(size_t)s * qh_count + qh] : -INFINITY);
    }
    M = fwave_max(M);
  }
  if (M == -INFINITY) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    z = 0.f;
    return;
  }
  const float w_own = expf(lse_l - M);             // one_chunk: this lane's split weight
  if (one_chunk) {
    z = fwave_sum(w_own);
  } else {
    z = 0.f;
    for (int s0 = 0; s0 < num_splits; s0 += 64) {
      const int s = s0 + lane;
      z += s < num_splits ? expf(lse_part[(size_t)s * qh_count + qh] - M) : 0.f;
    }
    z = fwave_sum(z);
  }
  const float inv_z = 1.0f / z;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int c = 8 * lane;
  for (int s0 = 0; s0 < num_splits; s0 += 64) {
    const int sl = s0 + lane;
    const float wl = one_chunk ? w_own : (sl < num_splits ? expf(lse_part[(size_t)sl * qh_count + qh] - M) : 0.f);
    const int cnt = num_splits - s0 < 64 ? num_splits - s0 : 64;
    int u = 0;
    for (; u + 8 <= cnt; u += 8) {
      float ws[8];
      float v[8][8];
#pragma unroll
      for (int k = 0; k < 8; ++k) ws[k] = __shfl(wl, u + k);
      // a split of weight zero re-reads the chunk's first row (a cache hit), so that all
      // eight loads go out unconditionally and back to back
#pragma unroll
      for (int k = 0; k < 8; ++k)
        load8p(o_part + ((size_t)(s0 + u + (ws[k] != 0.f ? k : 0)) * qh_count + qh) * kFDc + c, v[k]);
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
        load8p(o_part + ((size_t)(s0 + u) * qh_count + qh) * kFDc + c, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(ws, v[e], acc[e]);
      }
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
  // Every lane holds all of a row's split lse values (wave-uniform loads), so the maximum,
  // the weights and their sum need no cross-lane exchange.  The sum runs in the tree a
  // butterfly over lanes 0..7 would form, ((w0 + w4) + (w2 + w6)) + ((w1 + w5) + (w3 + w7)),
  // with zero weights for absent splits.
  // Every load is unconditional: a split past the last re-reads the last one (its weight is
  // zero), a row past the block's end reads a valid row (qh) and is not used.  A load under
  // a branch would leave its register undefined on the other path, and the compiler would
  // wait for it in the middle of issuing the rest.
  float lse[kRows][kFFast];
  pvec raw[kRows][kFFast][8 / kVec];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
#pragma unroll
    for (int k = 0; k < kFFast; ++k) {
      const int kk = k < num_splits ? k : num_splits - 1;
      lse[r][k] = lse_part[(size_t)kk * qh_count + qh[r]];
    }
#pragma unroll
    for (int k = 0; k < kFFast; ++k) {
      const int kk = k < num_splits ? k : num_splits - 1;
#pragma unroll
      for (int h = 0; h < 8 / kVec; ++h)
        raw[r][k][h] = *(const pvec*)(o_part + ((size_t)kk * qh_count + qh[r]) * kFDc + 8 * lane + kVec * h);
    }
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int k = 0; k < kFFast; ++k)
      if (!(r < nrows && k < num_splits)) lse[r][k] = -INFINITY;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    float m = lse[r][0];
#pragma unroll
    for (int k = 1; k < kFFast; ++k) m = fmaxf(m, lse[r][k]);
    M[r] = m;
    // No branch between the loads and their use (the compiler would sink the loads below
    // it): a row that no split saw, or one past the block's end, gets zero weights and zero
    // outputs.
    const bool none = m == -INFINITY;
    const float m_ref = none ? 0.f : m;
    float w[kFFast];
#pragma unroll
    for (int k = 0; k < kFFast; ++k) w[k] = k < num_splits ? expf(lse[r][k] - m_ref) : 0.f;
    const float zz = ((w[0] + w[4]) + (w[2] + w[6])) + ((w[1] + w[5]) + (w[3] + w[7]));
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kFFast; ++k) {
      const float ws = w[k];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = ws != 0.f ? fmaf(ws, (float)raw[r][k][e / kVec][e % kVec], acc[e]) : acc[e];
    }
    const float inv_z = 1.0f / zz;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[r][e] = none ? 0.f : acc[e] * inv_z;
    z[r] = none ? 0.f : zz;
  }
}

// Workgroup = (head i, block of 16 query rows); workgroups are dealt round-robin over the
// 8 XCDs and all query blocks of head i run on XCD i % 8, so W^UV_i is fetched into one L2.
// W^UV_i (128 KiB) first streams into LDS with direct-to-LDS loads of one whole 1 KiB row
// each; read straight into the MFMA operand layout, every load instruction would touch 32
// rows at 32 bytes each (16.5 against 15.3 us at 32 queries).  Each of the 8 waves then
// merges 2 of the block's rows (every load in flight at once) into LDS as bf16.  The
// projection then runs as in mla_out_proj: for each 32-column block of d_h, four k quarters
// of 8 MFMA steps summed in quarter order.  Waves 0-3 take column block w with all four
// quarters as independent chains in registers, so no partial product goes through LDS and
// the other four waves are done after the merge.  The MFMA M dimension is 32, so rows 16-31
// of each product repeat rows 0-15 and are not stored.
constexpr int kFRows = 16;                   // query rows per workgroup
constexpr int kFColBlocks = 4;               // 32-column blocks of d_h = 128

template <typename PartT>
__global__ void __launch_bounds__(kFThreads)
merge_out_proj_kernel(FusedParams P) {
  // LDS: W^UV_i (d_h rows of 1 KiB, chunk c of row r at c ^ (r & 15)), then o_lat rows (bf16)
  extern __shared__ __attribute__((aligned(1024))) char smem_f[];
  char* w_lds = smem_f;
  char* o_lds = smem_f + 32 * kFColBlocks * kFWRowBytes;
  const int qblocks = (P.n_q + kFRows - 1) / kFRows;
  const int xcd = blockIdx.x & 7;
  const int kq = blockIdx.x >> 3;
  const int i = (kq / qblocks) * 8 + xcd;
  const int mb = (kq % qblocks) * kFRows;
  if (i >= P.n_h) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int qh_count = P.n_q * P.n_h;
  const PartT* o_part = (const PartT*)P.o_part;
  const int rows = P.n_q - mb < kFRows ? P.n_q - mb : kFRows;

  // B operands (waves 0-3): lane l holds W^UV_i[32 cbk + l%32][16 (8 q + s) + 8 (l/32) .. +7]
  const int cbk = wave & 3;
  // W^UV_i streams into LDS first: each instruction one whole 1 KiB row (wave w: rows
  // 16w .. 16w+15), lane L filling physical chunk L with logical chunk L ^ (r & 15)
  {
    const char* wsrc = (const char*)(P.w_uv + (size_t)i * P.d_h * kFDc);
    const uint32_t wl = __builtin_amdgcn_readfirstlane(lds_addr(w_lds));
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 16 * wave + j;
      global_to_lds16_sv(wsrc, (uint32_t)(r * kFWRowBytes + ((lane ^ (r & 15)) * 16)), wl + r * kFWRowBytes);
    }
  }

  // ---- merge rows wave and wave + 8 of the block into LDS as bf16
  {
    int qh[2];
    int nr = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = wave + j * kFWaves;
      qh[j] = (mb + (r < rows ? r : 0)) * P.n_h + i;
      nr += r < rows ? 1 : 0;
    }
    // rows past the block's last valid row: their LDS rows still get finite values
    float o[2][8], M[2], z[2];
    if (P.num_splits <= kFFast) {
      merge_rows_fast<PartT, 2>(o_part, P.lse_part, qh_count, qh, nr, P.num_splits, lane, o, M, z);
    } else {
      for (int j = 0; j < nr; ++j) merge_one(o_part, P.lse_part, qh_count, qh[j], P.num_splits, lane, o[j], M[j], z[j]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = wave + j * kFWaves;
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      if (j >= nr) {                               // unused row: zeros in LDS, nothing stored
        *(u32x4*)(o_lds + r * kFPitch + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
        continue;
      }
      *(u32x4*)(o_lds + r * kFPitch + 16 * lane) =
          u32x4{pack_bf16x2(o[j][0], o[j][1]), pack_bf16x2(o[j][2], o[j][3]),
                pack_bf16x2(o[j][4], o[j][5]), pack_bf16x2(o[j][6], o[j][7])};
      if (P.o_lat) {
        float* dst = P.o_lat + (size_t)qh[j] * kFDc + 8 * lane;
        *(f32x4*)dst = f32x4{o[j][0], o[j][1], o[j][2], o[j][3]};
        *(f32x4*)(dst + 4) = f32x4{o[j][4], o[j][5], o[j][6], o[j][7]};
      }
      if (P.lse && lane == 0) P.lse[qh[j]] = M[j] == -INFINITY ? -INFINITY : M[j] + logf(z[j]);
    }
  }
  wait_vmcnt<0>();                                // this wave's W^UV rows have landed
  lds_barrier();

  // ---- o_c block = o_lat block (bf16) . W^UV_i^T: waves 0-3, column block w, all four
  // k quarters as independent chains, summed in quarter order as out_proj does
  if (wave < kFColBlocks) {
    const char* a = o_lds + (lane & 15) * kFPitch + 16 * (lane >> 5);
    const int wr = 32 * cbk + (lane & 31);       // W^UV row of this lane's B operands
    const char* wrow = w_lds + wr * kFWRowBytes;
    f32x16 accq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) accq[q][r] = 0.f;
#pragma unroll
    for (int s = 0; s < kFSteps; ++s)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 2 * (kFSteps * q + s) + (lane >> 5);
        const bf16x8 wb = *(const bf16x8*)(wrow + ((c ^ (wr & 15)) * 16));
        accq[q] = mfma32x32x16(*(const bf16x8*)(a + 32 * (kFSteps * q + s)), wb, accq[q]);
      }
    // registers 0..7 hold rows 0..15 of the D layout (lane l, reg r -> row 8 (r/4) +
    // 4 (l/32) + r%4); rows 16-31 repeat them
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const float v = ((accq[0][rr] + accq[1][rr]) + accq[2][rr]) + accq[3][rr];
      const int mm = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
      if (mm < rows)
        P.o_c[((size_t)(mb + mm) * P.n_h + i) * P.d_h + 32 * cbk + (lane & 31)] = f32_to_bf16(v);
    }
  }
}

}  // namespace

bool merge_out_proj_bf16_supported(int d_h, int d_c) { return d_c == kFDc && d_h == 32 * kFColBlocks; }

hipError_t launch_merge_out_proj_bf16(const void* o_part, bool f16_partials, const float* lse_part,
                                      const bf16_bits* w_uv, bf16_bits* o_c, float* lse, float* o_lat,
                                      int n_q, int n_h, int d_h, int num_splits, hipStream_t stream) {
  FusedParams P{o_part, lse_part, w_uv, o_c, lse, o_lat, n_q, n_h, d_h, num_splits};
  const int grid = 8 * ((n_h + 7) / 8) * ((n_q + kFRows - 1) / kFRows);
  const size_t smem = (size_t)32 * kFColBlocks * kFWRowBytes + (size_t)kFRows * kFPitch;
  static const hipError_t a16 = hipFuncSetAttribute((const void*)merge_out_proj_kernel<_Float16>,
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  static const hipError_t a32 = hipFuncSetAttribute((const void*)merge_out_proj_kernel<float>,
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (a16 != hipSuccess) return a16;
  if (a32 != hipSuccess) return a32;
  if (f16_partials)
    hipLaunchKernelGGL(merge_out_proj_kernel<_Float16>, dim3(grid), dim3(kFThreads), smem, stream, P);
  else
    hipLaunchKernelGGL(merge_out_proj_kernel<float>, dim3(grid), dim3(kFThreads), smem, stream, P);
  return hipGetLastError();
}

}  // namespace mla
