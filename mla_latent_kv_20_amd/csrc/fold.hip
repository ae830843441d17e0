// From the compressed query c^Q to the attention block's output u, unfolded and folded.
//
// Pages cited: [notes] "MLA(Multi-head Latent Attention): DeepSeek-V2 논문정리" (eq. 13:
// q^C = W^UQ c^Q; "Decoupled Rotary Position Embedding": the score's content term is
// (c^Q)^T (W^UQ)^T W^UK c^KV, whose middle product is token independent; "Value에 대한 수식
// 전개": W'^O = W^O W^UV); [report] "Техотчёт DeepSeek-V2 (2024): MLA и экономика инференса",
// "Идея 1" (W^UK absorbed into the queries, W^UV into W^O).
//
// Decode-time products are skinny GEMMs, C[n][m] = sum_k X[n][k] W[m][k] with few rows n (the
// batch's queries) and a weight W read once: gemm_xwt_kernel streams W rows as MFMA B
// operands (a row's k values contiguous), X rows as A operands, 32 rows x 32 columns per
// wave, two batches of eight k-steps of loads alternating with their MFMAs.  Long K is split over
// workgroups; fp32 partial sums go to a caller workspace and gemm_finish_kernel adds them in
// slice order.  The folds themselves are offline: plain fp32 kernels.
#include "mla_common.h"

namespace mla {
namespace {

constexpr int kGThreads = 256;               // 4 waves x 32 output columns
constexpr int kGCols = 128;
constexpr int kGU = 8;                       // k-steps of 16 per load batch
constexpr int kGK = 16 * kGU;                // K granule (128)

struct GemmParams {
  const void* x;            // [batch][M][K] bf16 or fp32, row stride ldx, batch stride bsx
  int64_t ldx, bsx;
  const bf16_bits* w;       // [batch][N][K] bf16, row stride ldw, batch stride bsw
  int64_t ldw, bsw;
  bf16_bits* out;           // direct form: out[b * bso + n * ldo + m]
  int64_t ldo, bso;
  float* ws;                // split form: ws[((z * batch + b) * M + n) * N + m]
  int M, N, K, kslice, batch;
};

template <bool kXf32>
__device__ __forceinline__ bf16x8 load_x8(const void* x, int64_t off) {
  if constexpr (kXf32) {
    const float* p = (const float*)x + off;
    const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                     pack_bf16x2(b[2], b[3])};
    return __builtin_bit_cast(bf16x8, v);
  } else {
    return *(const bf16x8*)((const bf16_bits*)x + off);
  }
}

template <bool kXf32, bool kDirect>
__global__ void __launch_bounds__(kGThreads)
gemm_xwt_kernel(GemmParams P) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nblocks = (P.M + 31) / 32;
  const int b = blockIdx.y / nblocks;
  const int n0 = (blockIdx.y - b * nblocks) * 32;
  const int m0 = blockIdx.x * kGCols + 32 * wave;
  const int k_begin = blockIdx.z * P.kslice;
  const int k_end = k_begin + P.kslice < P.K ? k_begin + P.kslice : P.K;
  // A: X row n0 + l%32 (clamped: rows past M are computed and dropped); B: W row m0 + l%32
  const int n_ld = n0 + (lane & 31) < P.M ? n0 + (lane & 31) : P.M - 1;
  const int64_t xoff = b * P.bsx + (int64_t)n_ld * P.ldx + 8 * (lane >> 5);
  const bf16_bits* wrow = P.w + b * P.bsw + (int64_t)(m0 + (lane & 31)) * P.ldw + 8 * (lane >> 5);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  // two batches of loads: the next batch is in flight while the current one's MFMAs run
  bf16x8 a[2][kGU], bw[2][kGU];
  auto fetch = [&](int h, int k) {
#pragma unroll
    for (int u = 0; u < kGU; ++u) bw[h][u] = *(const bf16x8*)(wrow + k + 16 * u);
#pragma unroll
    for (int u = 0; u < kGU; ++u) a[h][u] = load_x8<kXf32>(P.x, xoff + k + 16 * u);
  };
  auto consume = [&](int h) {
#pragma unroll
    for (int u = 0; u < kGU; ++u) acc = mfma32x32x16(a[h][u], bw[h][u], acc);
  };
  if (k_begin < k_end) fetch(0, k_begin);
  for (int k = k_begin; k < k_end; k += 2 * kGK) {
    const bool more = k + kGK < k_end;
    if (more) fetch(1, k + kGK);
    consume(0);
    if (k + 2 * kGK < k_end) fetch(0, k + 2 * kGK);
    if (more) consume(1);
  }
  // D[n][m]: lane l, reg r -> row n0 + 8(r/4) + 4(l/32) + r%4, column m0 + l%32
  const int m = m0 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int n = n0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (n < P.M) {
      if constexpr (kDirect)
        P.out[b * P.bso + (int64_t)n * P.ldo + m] = f32_to_bf16(acc[r]);
      else
        P.ws[(((int64_t)blockIdx.z * P.batch + b) * P.M + n) * P.N + m] = acc[r];
    }
  }
}

// out[b * bso + n * ldo + m] = bf16(sum over slices z in order of ws[z][b][n][m])
__global__ void gemm_finish_kernel(const float* __restrict__ ws, bf16_bits* __restrict__ out, int slices,
                                   int batch, int M, int N, int64_t ldo, int64_t bso) {
  const int64_t total = (int64_t)batch * M * N;
  const int64_t plane = total;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    float v = 0.f;
    for (int z = 0; z < slices; ++z) v += ws[z * plane + e];
    const int64_t m = e % N;
    const int64_t n = (e / N) % M;
    const int64_t b = e / ((int64_t)N * M);
    out[b * bso + n * ldo + m] = f32_to_bf16(v);
  }
}

// q_abs[n, i, d_c + r] = q_r[n, i, r]
__global__ void copy_rope_kernel(const bf16_bits* __restrict__ q_r, bf16_bits* __restrict__ q_abs, int n_q,
                                 int n_h, int d_c, int d_r) {
  const int64_t total = (int64_t)n_q * n_h * d_r;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x)
    q_abs[(e / d_r) * (d_c + d_r) + d_c + e % d_r] = q_r[e];
}

// G[i][c][k] = sum_d W^UK[i][d][c] W^UQ[i][d][k] (fp32 sums, one bf16 rounding)
__global__ void fold_q_kernel(const bf16_bits* __restrict__ w_uq, const bf16_bits* __restrict__ w_uk,
                              bf16_bits* __restrict__ g, int n_h, int d_h, int d_c, int d_cq) {
  const int64_t total = (int64_t)n_h * d_c * d_cq;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int k = (int)(e % d_cq);
    const int c = (int)((e / d_cq) % d_c);
    const int i = (int)(e / ((int64_t)d_cq * d_c));
    const bf16_bits* uq = w_uq + (int64_t)i * d_h * d_cq + k;
    const bf16_bits* uk = w_uk + (int64_t)i * d_h * d_c + c;
    float acc = 0.f;
    for (int d = 0; d < d_h; ++d) acc = fmaf(bf16_to_f32(uk[(int64_t)d * d_c]), bf16_to_f32(uq[(int64_t)d * d_cq]), acc);
    g[e] = f32_to_bf16(acc);
  }
}

// W'^O[m][i d_c + c] = sum_d W^O[m][i d_h + d] W^UV[i][d][c] (fp32 sums, one bf16 rounding)
__global__ void fold_o_kernel(const bf16_bits* __restrict__ w_o, const bf16_bits* __restrict__ w_uv,
                              bf16_bits* __restrict__ wf, int n_h, int d_h, int d_c, int d_model) {
  const int64_t width = (int64_t)n_h * d_c;
  const int64_t total = (int64_t)d_model * width;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(e % d_c);
    const int i = (int)((e / d_c) % n_h);
    const int64_t m = e / width;
    const bf16_bits* o = w_o + m * ((int64_t)n_h * d_h) + (int64_t)i * d_h;
    const bf16_bits* uv = w_uv + (int64_t)i * d_h * d_c + c;
    float acc = 0.f;
    for (int d = 0; d < d_h; ++d) acc = fmaf(bf16_to_f32(o[d]), bf16_to_f32(uv[(int64_t)d * d_c]), acc);
    wf[e] = f32_to_bf16(acc);
  }
}

unsigned grid_of(int64_t total) { return (unsigned)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536); }

// Split of K over workgroups so that a launch has about 512 of them.
void plan_split(int M, int N, int K, int batch, int* slices, int* kslice) {
  const int64_t wgs = (int64_t)(N / kGCols) * batch * ((M + 31) / 32);
  int s = (int)((512 + wgs - 1) / wgs);
  const int gran = K / kGK;
  s = s < 1 ? 1 : (s > gran ? gran : s);
  int ks = ((K + s - 1) / s + kGK - 1) / kGK * kGK;
  *kslice = ks;
  *slices = (K + ks - 1) / ks;
}

}  // namespace

bool gemm_xwt_supported(int N, int K) { return N > 0 && K > 0 && N % kGCols == 0 && K % kGK == 0; }

size_t gemm_xwt_workspace_bytes(int M, int N, int K, int batch) {
  int slices, kslice;
  plan_split(M, N, K, batch, &slices, &kslice);
  return slices > 1 ? (size_t)slices * batch * M * N * sizeof(float) : 0;
}

// C = X W^T for `batch` (X, W) pairs; bf16 out at out[b * bso + n * ldo + m].  With
// allow_split, K is split over workgroups when that gives more of them (workspace:
// gemm_xwt_workspace_bytes); without it the launch never splits and ws is not used.
hipError_t launch_gemm_xwt(bool x_f32, const void* x, int64_t ldx, int64_t bsx, const bf16_bits* w, int64_t ldw,
                           int64_t bsw, bf16_bits* out, int64_t ldo, int64_t bso, float* ws, int M, int N, int K,
                           int batch, bool allow_split, hipStream_t stream) {
  int slices = 1, kslice = K;
  if (allow_split) plan_split(M, N, K, batch, &slices, &kslice);
  GemmParams P{x, ldx, bsx, w, ldw, bsw, out, ldo, bso, ws, M, N, K, kslice, batch};
  const dim3 grid(N / kGCols, batch * ((M + 31) / 32), slices);
  if (slices == 1) {
    if (x_f32) hipLaunchKernelGGL((gemm_xwt_kernel<true, true>), grid, dim3(kGThreads), 0, stream, P);
    else hipLaunchKernelGGL((gemm_xwt_kernel<false, true>), grid, dim3(kGThreads), 0, stream, P);
    return hipGetLastError();
  }
  if (x_f32) hipLaunchKernelGGL((gemm_xwt_kernel<true, false>), grid, dim3(kGThreads), 0, stream, P);
  else hipLaunchKernelGGL((gemm_xwt_kernel<false, false>), grid, dim3(kGThreads), 0, stream, P);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemm_finish_kernel, dim3(grid_of((int64_t)batch * M * N)), dim3(256), 0, stream, ws, out,
                     slices, batch, M, N, ldo, bso);
  return hipGetLastError();
}

hipError_t launch_copy_rope(const bf16_bits* q_r, bf16_bits* q_abs, int n_q, int n_h, int d_c, int d_r,
                            hipStream_t stream) {
  hipLaunchKernelGGL(copy_rope_kernel, dim3(grid_of((int64_t)n_q * n_h * d_r)), dim3(256), 0, stream, q_r, q_abs,
                     n_q, n_h, d_c, d_r);
  return hipGetLastError();
}

hipError_t launch_fold_q(const bf16_bits* w_uq, const bf16_bits* w_uk, bf16_bits* g, int n_h, int d_h, int d_c,
                         int d_cq, hipStream_t stream) {
  hipLaunchKernelGGL(fold_q_kernel, dim3(grid_of((int64_t)n_h * d_c * d_cq)), dim3(256), 0, stream, w_uq, w_uk, g,
                     n_h, d_h, d_c, d_cq);
  return hipGetLastError();
}

hipError_t launch_fold_o(const bf16_bits* w_o, const bf16_bits* w_uv, bf16_bits* wf, int n_h, int d_h, int d_c,
                         int d_model, hipStream_t stream) {
  hipLaunchKernelGGL(fold_o_kernel, dim3(grid_of((int64_t)d_model * n_h * d_c)), dim3(256), 0, stream, w_o, w_uv,
                     wf, n_h, d_h, d_c, d_model);
  return hipGetLastError();
}

}  // namespace mla
