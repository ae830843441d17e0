// Decode prologue: the new tokens' latent rows, written into the cache.
//
// Pages cited: [notes] "MLA(Multi-head Latent Attention): DeepSeek-V2 논문정리".
//
//   c^KV_t = W^DKV h_t                        ([notes] eq. 9)
//   k^R_t  = RoPE(W^KR h_t, position_t)       ([notes] "Decoupled Rotary Position Embedding",
//                                             items 2-3: one key per token, cached rotated)
//   row dst_t of the cache <- [c^KV_t ; k^R_t] ([notes] "MLA 코드 구현": the new latent rows
//                                             follow the cached ones)
// RoPE rotates the pairs (k, k + d_r/2) by position * theta^(-2k/d_r), the rotate-half form
// of the listing in "MLA 코드 구현"; angles and the rotation are evaluated in fp64.
//
// bf16: one workgroup per (32 tokens, 32 columns of c^KV) or (32 tokens, the 64 columns of
// k^R, whose rotation pairs columns k and k+32 of the same lane).  The eight waves split
// d_model; their 32x32 products meet in LDS.  The down-projection weights are streamed once
// per token block; at decode batch sizes the call is bound by that weight traffic.
#include "mla_common.h"

namespace mla {
namespace {

constexpr int kAppWaves = 8;
constexpr int kAppThreads = kAppWaves * 64;
constexpr int kAppUnroll = 4;                 // k-steps whose loads go out together

struct AppendParams {
  const void* h;           // [n_new, d_model]
  const void* w_dkv;       // [d_c, d_model]
  const void* w_kr;        // [d_r, d_model]
  const int64_t* pos;      // [n_new]
  const int64_t* dst;      // [n_new]
  void* rows;              // cache rows, `stride` elements each
  int64_t stride;
  int n_new, d_model, d_c, d_r;
  double log_theta;        // ln(theta)
};

__global__ void __launch_bounds__(kAppThreads)
kv_append_bf16_kernel(AppendParams P) {
  __shared__ f32x16 red[kAppWaves][2][64];        // [wave][tile][lane] partial products
  const int nlat = P.d_c / 32;
  const int cb = blockIdx.x;
  const bool rope = cb == nlat;                   // the k^R block: two 32-column tiles
  const int tok0 = blockIdx.y * 32;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tok = tok0 + (lane & 31);
  const int tok_ld = tok < P.n_new ? tok : P.n_new - 1;

  // D[col][token] = sum_k W[col][k] h[token][k]: A = W rows (lane l: column l%32, 8
  // consecutive k), B = h^T (lane l: token l%32, 8 consecutive k).
  const bf16_bits* hrow = (const bf16_bits*)P.h + (size_t)tok_ld * P.d_model + 8 * (lane >> 5);
  const bf16_bits* w0 = rope ? (const bf16_bits*)P.w_kr + (size_t)(lane & 31) * P.d_model
                             : (const bf16_bits*)P.w_dkv + (size_t)(32 * cb + (lane & 31)) * P.d_model;
  w0 += 8 * (lane >> 5);
  const bf16_bits* w1 = w0 + (size_t)32 * P.d_model;   // rope: k^R columns 32..63

  const int ksteps = P.d_model / 16;
  const int per_wave = ksteps / kAppWaves;            // d_model % 128 == 0
  const int s_begin = wave * per_wave;
  f32x16 acc0, acc1;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    acc0[r] = 0.f;
    acc1[r] = 0.f;
  }
  for (int s0 = s_begin; s0 < s_begin + per_wave; s0 += kAppUnroll) {
    bf16x8 hb[kAppUnroll], wa[kAppUnroll], wb[kAppUnroll];
#pragma unroll
    for (int u = 0; u < kAppUnroll; ++u) {
      if (s0 + u < s_begin + per_wave) {
        hb[u] = *(const bf16x8*)(hrow + 16 * (s0 + u));
        wa[u] = *(const bf16x8*)(w0 + 16 * (s0 + u));
        if (rope) wb[u] = *(const bf16x8*)(w1 + 16 * (s0 + u));
      }
    }
#pragma unroll
    for (int u = 0; u < kAppUnroll; ++u) {
      if (s0 + u < s_begin + per_wave) {
        acc0 = mfma32x32x16(wa[u], hb[u], acc0);
        if (rope) acc1 = mfma32x32x16(wb[u], hb[u], acc1);
      }
    }
  }
  red[wave][0][lane] = acc0;
  if (rope) red[wave][1][lane] = acc1;
  __syncthreads();
  if (wave != 0) return;

  // Wave 0 sums the partials in wave order, then rotates (k^R block) and stores.
  // D layout: lane l, reg r -> column 8(r/4) + 4(l/32) + r%4 of the tile, token l%32.
  if (tok >= P.n_new) return;
  bf16_bits* dst = (bf16_bits*)P.rows + P.dst[tok] * P.stride;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int col = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    float x = 0.f, y = 0.f;
#pragma unroll
    for (int w = 0; w < kAppWaves; ++w) x += red[w][0][lane][r];
    if (!rope) {
      dst[32 * cb + col] = f32_to_bf16(x);
    } else {
#pragma unroll
      for (int w = 0; w < kAppWaves; ++w) y += red[w][1][lane][r];
      double dx = x, dy = y;
      rope_pair(dx, dy, P.pos[tok], col, P.d_r, P.log_theta);
      dst[P.d_c + col] = f32_to_bf16((float)dx);
      dst[P.d_c + 32 + col] = f32_to_bf16((float)dy);
    }
  }
}

// fp32: one thread per (token, column); a k^R column computes its pair partner's sum too.
__global__ void kv_append_f32_kernel(AppendParams P) {
  const int width = P.d_c + P.d_r;
  const size_t total = (size_t)P.n_new * width;
  const int half = P.d_r / 2;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(e / width);
    const int c = (int)(e % width);
    const float* h = (const float*)P.h + (size_t)t * P.d_model;
    float* dst = (float*)P.rows + P.dst[t] * P.stride;
    if (c < P.d_c) {
      const float* w = (const float*)P.w_dkv + (size_t)c * P.d_model;
      float acc = 0.f;
      for (int m = 0; m < P.d_model; ++m) acc = fmaf(w[m], h[m], acc);
      dst[c] = acc;
    } else {
      const int k = c - P.d_c;
      const int k0 = k < half ? k : k - half;     // first member of the pair
      const float* wx = (const float*)P.w_kr + (size_t)k0 * P.d_model;
      const float* wy = wx + (size_t)half * P.d_model;
      float ax = 0.f, ay = 0.f;
      for (int m = 0; m < P.d_model; ++m) {
        ax = fmaf(wx[m], h[m], ax);
        ay = fmaf(wy[m], h[m], ay);
      }
      double dx = ax, dy = ay;
      rope_pair(dx, dy, P.pos[t], k0, P.d_r, P.log_theta);
      dst[c] = (float)(k < half ? dx : dy);
    }
  }
}

}  // namespace

bool kv_append_bf16_supported(int d_model, int d_c, int d_r) {
  return d_model % (16 * kAppWaves) == 0 && d_model > 0 && d_c % 32 == 0 && d_r == 64;
}

hipError_t launch_kv_append(bool bf16, const void* h, const void* w_dkv, const void* w_kr,
                            const int64_t* positions, const int64_t* dst_rows, void* rows, int64_t stride,
                            int n_new, int d_model, int d_c, int d_r, double theta, hipStream_t stream) {
  AppendParams P{h, w_dkv, w_kr, positions, dst_rows, rows, stride, n_new, d_model, d_c, d_r, log(theta)};
  if (bf16) {
    hipLaunchKernelGGL(kv_append_bf16_kernel, dim3(d_c / 32 + 1, (n_new + 31) / 32), dim3(kAppThreads), 0,
                       stream, P);
  } else {
    const size_t total = (size_t)n_new * (d_c + d_r);
    const unsigned grid = (unsigned)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
    hipLaunchKernelGGL(kv_append_f32_kernel, dim3(grid), dim3(256), 0, stream, P);
  }
  return hipGetLastError();
}

}  // namespace mla
