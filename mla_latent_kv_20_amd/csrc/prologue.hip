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
// of the listing in "MLA 코드 구현" (rope_rotate: fp64 angle, fp32 sine and cosine).
//
// bf16, two kernels.  At decode batch sizes the call is bound by the down-projection
// weights ((d_c + d_r) x d_model), so they are spread over many workgroups: workgroup =
// (32 output columns, 32 tokens, one of kSplitK slices of d_model), four waves splitting
// the slice, every load of a wave in flight at once.  Slice ks runs on XCD ks, so each
// XCD's L2 fetches only its eighth of the hidden states.  Each workgroup writes its fp32 32x32
// product to the caller's workspace; the finishing kernel sums the slices in order,
// rotates the k^R pairs (columns k and k + d_r/2 of one token) and stores bf16 rows.
#include "mla_common.h"

namespace mla {
namespace {

constexpr int kSplitK = 8;                    // slices of d_model over workgroups
static_assert(kSplitK == 8, "one slice of d_model per XCD");
constexpr int kAppWaves = 4;
constexpr int kAppThreads = kAppWaves * 64;
constexpr int kMaxSteps = 16;                 // k-steps of 16 per wave: d_model <= 8*4*16*16

struct AppendParams {
  const void* h;           // [n_new, d_model]
  const void* w_dkv;       // [d_c, d_model]
  const void* w_kr;        // [d_r, d_model]
  const int64_t* pos;      // [n_new]
  const int64_t* dst;      // [n_new]
  void* rows;              // cache rows, `stride` elements each
  float* ws;               // bf16: [kSplitK][n_new][d_c + d_r] partial sums
  int64_t stride;
  int n_new, d_model, d_c, d_r;
  RopeSpec rope;
};

// Kernel 1: partial products of one (column block, token block, K slice).  kStepsT: the
// k-steps per wave fixed at compile time (every load unconditional), or 0 for any d_model.
template <int kStepsT>
__global__ void __launch_bounds__(kAppThreads)
kv_append_partial_kernel(AppendParams P) {
  __shared__ f32x16 red[kAppWaves][64];
  const int width = P.d_c + P.d_r;
  // Workgroups are dealt round-robin over the 8 XCDs (workgroup L on XCD L % 8): slice ks
  // of d_model runs on XCD ks, so each XCD's L2 fetches only its slice of the hidden states.
  const int L = blockIdx.x;
  const int ks = L % kSplitK;                     // K slice
  const int cbs = (P.d_c + P.d_r) / 32;
  const int cb = (L / kSplitK) % cbs;             // 32-column block of [c^KV | k^R]
  const int tok0 = (L / kSplitK / cbs) * 32;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int tok = tok0 + (lane & 31);
  const int tok_ld = tok < P.n_new ? tok : P.n_new - 1;
  const int col = 32 * cb + (lane & 31);          // output column of this lane's W row
  const bf16_bits* wrow = col < P.d_c ? (const bf16_bits*)P.w_dkv + (size_t)col * P.d_model
                                      : (const bf16_bits*)P.w_kr + (size_t)(col - P.d_c) * P.d_model;
  const int steps = kStepsT > 0 ? kStepsT : P.d_model / (16 * kSplitK * kAppWaves);   // k-steps per wave
  const int k0 = (ks * kAppWaves + wave) * steps * 16 + 8 * (lane >> 5);
  const bf16_bits* hp = (const bf16_bits*)P.h + (size_t)tok_ld * P.d_model + k0;
  const bf16_bits* wp = wrow + k0;
  // D[col][token] = sum_k W[col][k] h[token][k]: A = W rows (lane l: column l%32, 8
  // consecutive k), B = h^T (lane l: token l%32, 8 consecutive k)
  bf16x8 a[kMaxSteps], b[kMaxSteps];
#pragma unroll
  for (int s = 0; s < kMaxSteps; ++s) {
    if (s < steps) {
      a[s] = *(const bf16x8*)(wp + 16 * s);
      b[s] = *(const bf16x8*)(hp + 16 * s);
    }
  }
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSteps; ++s)
    if (s < steps) acc = mfma32x32x16(a[s], b[s], acc);
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  // D layout: lane l, reg r -> column 8(r/4) + 4(l/32) + r%4 of the block, token l%32
  if (tok >= P.n_new) return;
  float* out = P.ws + ((size_t)ks * P.n_new + tok) * width + 32 * cb;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kAppWaves; ++w) v += red[w][lane][r];
    out[8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)] = v;
  }
}

// Kernel 2: one thread per (token, c^KV column or k^R pair): slices summed in order,
// the pair rotated, bf16 stored.
__global__ void kv_append_finish_kernel(AppendParams P) {
  const int width = P.d_c + P.d_r;
  const int half = P.d_r / 2;
  const int per_tok = P.d_c + half;
  const size_t total = (size_t)P.n_new * per_tok;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(e / per_tok);
    const int c = (int)(e % per_tok);
    const float* src = P.ws + (size_t)t * width;
    const size_t slice = (size_t)P.n_new * width;
    // Every load of the element (its slices' partial sums, the row index, the position) is
    // issued before the first is used, and the slices are added in slice order.
    const bool lat = c < P.d_c;
    const int k = lat ? 0 : c - P.d_c;
    const int cx = lat ? c : P.d_c + k;
    float vx[kSplitK], vy[kSplitK];
#pragma unroll
    for (int s = 0; s < kSplitK; ++s) {
      vx[s] = src[s * slice + cx];
      vy[s] = src[s * slice + (lat ? cx : cx + half)];
    }
    const int64_t row = P.dst[t];
    const int64_t pos = P.pos[t];
    bf16_bits* dst = (bf16_bits*)P.rows + row * P.stride;
    float x = 0.f, y = 0.f;
#pragma unroll
    for (int s = 0; s < kSplitK; ++s) {
      x += vx[s];
      y += vy[s];
    }
    if (lat) {
      dst[c] = f32_to_bf16(x);
    } else {
      double dx = x, dy = y;
      rope_pair(dx, dy, pos, k, P.d_r, P.rope);
      dst[P.d_c + k] = f32_to_bf16((float)dx);
      dst[P.d_c + k + half] = f32_to_bf16((float)dy);
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
      rope_pair(dx, dy, P.pos[t], k0, P.d_r, P.rope);
      dst[c] = (float)(k < half ? dx : dy);
    }
  }
}

unsigned grid_of(size_t total) { return (unsigned)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536); }

}  // namespace

bool kv_append_bf16_supported(int d_model, int d_c, int d_r) {
  const int unit = 16 * kSplitK * kAppWaves;
  return d_model > 0 && d_model % unit == 0 && d_model / unit <= kMaxSteps && (d_c + d_r) % 32 == 0 &&
         d_r % 2 == 0;
}

size_t kv_append_workspace_bytes(bool bf16, int n_new, int d_c, int d_r) {
  return bf16 ? (size_t)kSplitK * n_new * (d_c + d_r) * sizeof(float) : 0;
}

hipError_t launch_kv_append(bool bf16, const void* h, const void* w_dkv, const void* w_kr,
                            const int64_t* positions, const int64_t* dst_rows, void* rows, int64_t stride,
                            float* workspace, int n_new, int d_model, int d_c, int d_r, const RopeSpec& rope,
                            hipStream_t stream) {
  AppendParams P{h, w_dkv, w_kr, positions, dst_rows, rows, workspace, stride, n_new, d_model, d_c, d_r, rope};
  if (bf16) {
    if (d_model == 16 * kSplitK * kAppWaves * 10)
      hipLaunchKernelGGL(kv_append_partial_kernel<10>, dim3((d_c + d_r) / 32 * ((n_new + 31) / 32) * kSplitK),
                       dim3(kAppThreads), 0, stream, P);
    else
      hipLaunchKernelGGL(kv_append_partial_kernel<0>, dim3((d_c + d_r) / 32 * ((n_new + 31) / 32) * kSplitK),
                       dim3(kAppThreads), 0, stream, P);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kv_append_finish_kernel, dim3(grid_of((size_t)n_new * (d_c + d_r / 2))), dim3(256), 0,
                       stream, P);
  } else {
    hipLaunchKernelGGL(kv_append_f32_kernel, dim3(grid_of((size_t)n_new * (d_c + d_r))), dim3(256), 0, stream, P);
  }
  return hipGetLastError();
}

}  // namespace mla
