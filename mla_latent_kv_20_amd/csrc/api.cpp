// C ABI of the MLA absorbed-decode library: argument checks and kernel dispatch.
// Every check runs before anything is launched; a failed check returns its status.
#include "../../include/mla_kv.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "rope_spec.h"

namespace mla {
typedef uint16_t bf16_bits;
// kernels (decode_bf16.hip, absorb_bf16.hip, merge_f32.hip)
hipError_t launch_decode_bf16(const bf16_bits* q_abs, const bf16_bits* rows, int64_t stride,
                              const int64_t* offsets, void* o_part, bool f16_partials,
                              float* lse_part, int batch, int q_per_seq, int n_h, int num_splits,
                              int split_rows, float scale, hipStream_t stream);
hipError_t launch_absorb_q_bf16(const bf16_bits* q_c, const bf16_bits* q_r, const bf16_bits* w_uk,
                                bf16_bits* q_abs, int n_q, int n_h, int d_h, int d_c, int d_r,
                                const int64_t* positions, const RopeSpec& rope, hipStream_t stream);
hipError_t launch_out_proj_bf16(const float* o_lat, const bf16_bits* w_uv, bf16_bits* o_c, int n_q,
                                int n_h, int d_h, int d_c, hipStream_t stream);
bool absorb_bf16_supported(int d_h, int d_c);
bool merge_out_proj_bf16_supported(int d_h, int d_c);
hipError_t launch_merge_out_proj_bf16(const void* o_part, bool f16_partials, const float* lse_part,
                                      const uint16_t* w_uv, uint16_t* o_c, float* lse, float* o_lat,
                                      int n_q, int n_h, int d_h, int num_splits, hipStream_t stream);
bool out_proj_bf16_supported(int d_h, int d_c);
hipError_t launch_merge(const void* o_part, bool f16_partials, const float* lse_part, float* o_lat,
                        float* lse, int n_q, int n_h, int d_c, int num_splits, hipStream_t stream);
hipError_t launch_absorb_q_f32(const float* q_c, const float* q_r, const float* w_uk, float* q_abs,
                               int n_q, int n_h, int d_h, int d_c, int d_r, const int64_t* positions,
                               const RopeSpec& rope, hipStream_t stream);
// prologue.hip
bool kv_append_bf16_supported(int d_model, int d_c, int d_r);
size_t kv_append_workspace_bytes(bool bf16, int n_new, int d_c, int d_r);
hipError_t launch_kv_append(bool bf16, const void* h, const void* w_dkv, const void* w_kr,
                            const int64_t* positions, const int64_t* dst_rows, void* rows, int64_t stride,
                            float* workspace, int n_new, int d_model, int d_c, int d_r, const RopeSpec& rope,
                            hipStream_t stream);
// noalloc.hip: the fixed device array's address on the current device (checked against stream's)
mla_status_t noalloc_scratch(hipStream_t stream, void** addr);
// quant_fp8.hip, decode_fp8.hip
bool quantize_rows_supported(int width);
hipError_t launch_quantize_rows(bool bf16, const void* src, int64_t src_stride, int64_t n,
                                const int64_t* dst_rows, uint8_t* codes, int64_t code_stride, float* scales,
                                int width, hipStream_t stream);
hipError_t launch_decode_fp8(const bf16_bits* q_abs, const uint8_t* codes, int64_t stride, const float* scales,
                             const int64_t* offsets, void* o_part, bool f16_partials, float* lse_part, int batch,
                             int q_per_seq, int n_h, int num_splits, int split_rows, float scale,
                             hipStream_t stream);
// fold.hip
bool gemm_xwt_supported(int N, int K);
size_t gemm_xwt_workspace_bytes(int M, int N, int K, int batch);
hipError_t launch_gemm_xwt(bool x_f32, const void* x, int64_t ldx, int64_t bsx, const bf16_bits* w, int64_t ldw,
                           int64_t bsw, bf16_bits* out, int64_t ldo, int64_t bso, float* ws, int M, int N, int K,
                           int batch, bool allow_split, hipStream_t stream);
hipError_t launch_copy_rope(const bf16_bits* q_r, bf16_bits* q_abs, int n_q, int n_h, int d_c, int d_r,
                            hipStream_t stream);
hipError_t launch_fold_q(const bf16_bits* w_uq, const bf16_bits* w_uk, bf16_bits* g, int n_h, int d_h, int d_c,
                         int d_cq, hipStream_t stream);
hipError_t launch_fold_o(const bf16_bits* w_o, const bf16_bits* w_uv, bf16_bits* wf, int n_h, int d_h, int d_c,
                         int d_model, hipStream_t stream);
size_t decode_f32_smem_bytes(int d_c, int d_r);
hipError_t launch_decode_f32(const float* q_abs, const float* c_kv, int64_t c_stride, const float* k_r,
                             int64_t r_stride, const int64_t* offsets, float* o_part, float* lse_part,
                             int batch, int q_per_seq, int n_h, int d_c, int d_r, int num_splits,
                             int split_rows, float scale, hipStream_t stream);
hipError_t launch_out_proj_f32(const float* o_lat, const float* w_uv, float* o_c, int n_q, int n_h,
                               int d_h, int d_c, hipStream_t stream);
}  // namespace mla

namespace {

// The bf16 decode kernel's fixed shape: 576-wide rows (512 latent + 64 RoPE), heads in
// groups of 32 per wave.
constexpr int kDecodeDc = 512;
constexpr int kDecodeDr = 64;
constexpr int64_t kMaxElems = (int64_t)1 << 31;   // any one tensor: < 2^31 elements per index

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

mla_status_t check_dims(const mla_dims_t* d) {
  if (!d) return MLA_ERR_NULL;
  if (d->dtype != MLA_F32 && d->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (d->n_h <= 0 || d->d_h <= 0 || d->d_c <= 0 || d->d_r <= 0) return MLA_ERR_SHAPE;
  if (d->n_h > 65535 || d->d_h > 65536 || d->d_c > 65536 || d->d_r > 65536) return MLA_ERR_SHAPE;
  if (d->d_r % 2) return MLA_ERR_SHAPE;       // RoPE pairs
  if (!(d->softmax_scale == d->softmax_scale) || std::isinf(d->softmax_scale)) return MLA_ERR_SHAPE;
  return MLA_OK;
}

float scale_of(const mla_dims_t* d) {
  return d->softmax_scale > 0.f ? d->softmax_scale : (float)(1.0 / std::sqrt((double)(d->d_h + d->d_r)));
}

size_t esize(const mla_dims_t* d) { return d->dtype == MLA_BF16 ? 2 : 4; }

mla_status_t launched(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH; }

bool finite(float x) { return x == x && !std::isinf(x); }

// mla_rope_t -> the kernels' RopeSpec; NULL: theta 10000, no YaRN.
mla_status_t rope_spec(const mla_rope_t* r, mla::RopeSpec* out) {
  const double theta = r && r->theta > 0.f ? (double)r->theta : 10000.0;
  *out = mla::RopeSpec{std::log(theta), 1.0, 1.0, 0.0, 1.0};
  if (!r) return MLA_OK;
  if (!finite(r->theta) || !finite(r->yarn_factor)) return MLA_ERR_SHAPE;
  if (r->yarn_factor > 1.f) {
    if (r->yarn_original_len <= 0 || !finite(r->yarn_alpha) || !finite(r->yarn_beta) ||
        !(r->yarn_beta > r->yarn_alpha))
      return MLA_ERR_SHAPE;
    out->yarn_s = r->yarn_factor;
    out->yarn_len = r->yarn_original_len;
    out->yarn_alpha = r->yarn_alpha;
    out->yarn_beta = r->yarn_beta;
  }
  return MLA_OK;
}

// Every check of mla_kv_append but its workspace's; fills the RoPE spec.  n_new == 0 passes
// after the shape checks (a no-op call).
mla_status_t kv_append_check(const mla_dims_t* dims, int32_t n_new, int32_t d_model, const void* h,
                             const void* w_dkv, const void* w_kr, const int64_t* positions,
                             const int64_t* dst_rows, void* rows, int64_t stride, const mla_rope_t* rope,
                             mla::RopeSpec* spec) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  st = rope_spec(rope, spec);
  if (st != MLA_OK) return st;
  if (n_new < 0 || d_model < 1) return MLA_ERR_SHAPE;
  if (n_new == 0) return MLA_OK;
  if (!h || !w_dkv || !w_kr || !positions || !dst_rows || !rows) return MLA_ERR_NULL;
  if (stride < (int64_t)dims->d_c + dims->d_r) return MLA_ERR_SHAPE;
  if ((int64_t)n_new * d_model >= kMaxElems || (int64_t)dims->d_c * d_model >= kMaxElems) return MLA_ERR_SHAPE;
  if (!aligned(positions, 8) || !aligned(dst_rows, 8)) return MLA_ERR_ALIGN;
  const uintptr_t a = esize(dims);
  if (!aligned(h, a) || !aligned(w_dkv, a) || !aligned(w_kr, a) || !aligned(rows, a)) return MLA_ERR_ALIGN;
  if (dims->dtype == MLA_BF16) {
    if (!mla::kv_append_bf16_supported(d_model, dims->d_c, dims->d_r)) return MLA_ERR_UNSUPPORTED;
    if (!aligned(h, 16) || !aligned(w_dkv, 16) || !aligned(w_kr, 16)) return MLA_ERR_ALIGN;
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

float mla_rope_softmax_scale(const mla_dims_t* dims, const mla_rope_t* rope) {
  if (!dims || dims->d_h + dims->d_r <= 0) return 0.f;
  const double base = dims->softmax_scale > 0.f ? (double)dims->softmax_scale
                                                : 1.0 / std::sqrt((double)(dims->d_h + dims->d_r));
  if (!rope || !(rope->yarn_factor > 1.f)) return (float)base;
  const double sqrt_t = (double)rope->yarn_mscale * std::log((double)rope->yarn_factor) + 1.0;
  return (float)(base * sqrt_t * sqrt_t);
}

const char* mla_status_string(mla_status_t s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_SHAPE: return "a size, count or stride is out of range";
    case MLA_ERR_ALIGN: return "a pointer or stride is not aligned as required";
    case MLA_ERR_DTYPE: return "unknown dtype";
    case MLA_ERR_UNSUPPORTED: return "the library has no kernel for these arguments";
    case MLA_ERR_LAUNCH: return "HIP kernel launch failed";
    case MLA_ERR_SCRATCH: return "the call needs more than the library's fixed scratch array holds";
    case MLA_ERR_DEVICE: return "the stream does not belong to the current device";
  }
  return "unknown status";
}

size_t mla_partial_bytes(const mla_dims_t* dims, int32_t n_q, int32_t num_splits, int32_t partial_dtype) {
  if (check_dims(dims) != MLA_OK || n_q < 0 || num_splits < 1) return 0;
  if (partial_dtype != MLA_F32 && partial_dtype != MLA_F16) return 0;
  return (size_t)num_splits * (size_t)n_q * (size_t)dims->n_h * (size_t)dims->d_c *
         (partial_dtype == MLA_F16 ? 2 : 4);
}

size_t mla_decode_workspace_bytes(const mla_dims_t* dims, int32_t n_q, int32_t num_splits) {
  const size_t o = mla_partial_bytes(dims, n_q, num_splits, MLA_F32);
  if (o == 0 && !(n_q == 0 && check_dims(dims) == MLA_OK && num_splits >= 1)) return 0;
  return o + (size_t)num_splits * (size_t)n_q * (size_t)dims->n_h * sizeof(float);
}

mla_status_t mla_check_offsets(const int64_t* host_offsets, int32_t batch, int32_t q_per_seq,
                               int64_t total_rows) {
  if (batch < 0 || q_per_seq < 1 || total_rows < 0) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!host_offsets) return MLA_ERR_NULL;
  if (host_offsets[0] < 0) return MLA_ERR_SHAPE;
  for (int32_t b = 0; b < batch; ++b)
    if (host_offsets[b + 1] - host_offsets[b] < q_per_seq) return MLA_ERR_SHAPE;
  if (host_offsets[batch] > total_rows) return MLA_ERR_SHAPE;
  return MLA_OK;
}

namespace {
// Shared by mla_absorb_q and mla_absorb_q_rope: positions == nullptr copies q_r as is.
mla_status_t absorb_common(const mla_dims_t* dims, int32_t n_q, const void* q_c, const void* q_r,
                           const void* w_uk, const int64_t* positions, const mla_rope_t* rope, void* q_abs,
                           hipStream_t stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  mla::RopeSpec spec;
  st = rope_spec(rope, &spec);
  if (st != MLA_OK) return st;
  if (n_q < 0) return MLA_ERR_SHAPE;
  if (n_q == 0) return MLA_OK;
  if (!q_c || !q_r || !w_uk || !q_abs) return MLA_ERR_NULL;
  const int64_t d_qk = (int64_t)dims->d_c + dims->d_r;
  if ((int64_t)n_q * dims->n_h * d_qk >= kMaxElems ||
      (int64_t)dims->n_h * dims->d_h * dims->d_c >= kMaxElems)
    return MLA_ERR_SHAPE;
  if (positions && !aligned(positions, 8)) return MLA_ERR_ALIGN;
  const uintptr_t a = esize(dims);
  if (!aligned(q_c, a) || !aligned(q_r, a) || !aligned(w_uk, a) || !aligned(q_abs, a)) return MLA_ERR_ALIGN;
  if (dims->dtype == MLA_F32)
    return launched(mla::launch_absorb_q_f32((const float*)q_c, (const float*)q_r, (const float*)w_uk,
                                             (float*)q_abs, n_q, dims->n_h, dims->d_h, dims->d_c,
                                             dims->d_r, positions, spec, stream));
  if (!mla::absorb_bf16_supported(dims->d_h, dims->d_c) || dims->d_r % 8) return MLA_ERR_UNSUPPORTED;
  if (positions && dims->d_r > 512) return MLA_ERR_UNSUPPORTED;  // a pair index per thread of 256
  if (!aligned(q_c, 16) || !aligned(q_r, 16) || !aligned(w_uk, 16) || !aligned(q_abs, 16)) return MLA_ERR_ALIGN;
  return launched(mla::launch_absorb_q_bf16((const uint16_t*)q_c, (const uint16_t*)q_r,
                                            (const uint16_t*)w_uk, (uint16_t*)q_abs, n_q, dims->n_h,
                                            dims->d_h, dims->d_c, dims->d_r, positions, spec, stream));
}
}  // namespace

mla_status_t mla_absorb_q(const mla_dims_t* dims, int32_t n_q, const void* q_c, const void* q_r,
                          const void* w_uk, void* q_abs, hipStream_t stream) {
  return absorb_common(dims, n_q, q_c, q_r, w_uk, nullptr, nullptr, q_abs, stream);
}

mla_status_t mla_absorb_q_rope(const mla_dims_t* dims, int32_t n_q, const void* q_c, const void* q_r_raw,
                               const void* w_uk, const int64_t* positions, const mla_rope_t* rope, void* q_abs,
                               hipStream_t stream) {
  if (n_q > 0 && !positions) return MLA_ERR_NULL;
  return absorb_common(dims, n_q, q_c, q_r_raw, w_uk, positions, rope, q_abs, stream);
}

size_t mla_kv_append_workspace_bytes(const mla_dims_t* dims, int32_t n_new) {
  if (check_dims(dims) != MLA_OK || n_new < 0) return 0;
  return mla::kv_append_workspace_bytes(dims->dtype == MLA_BF16, n_new, dims->d_c, dims->d_r);
}

mla_status_t mla_kv_append(const mla_dims_t* dims, int32_t n_new, int32_t d_model, const void* h,
                           const void* w_dkv, const void* w_kr, const int64_t* positions,
                           const int64_t* dst_rows, void* rows, int64_t stride, const mla_rope_t* rope,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  mla::RopeSpec spec;
  const mla_status_t st = kv_append_check(dims, n_new, d_model, h, w_dkv, w_kr, positions, dst_rows, rows, stride,
                                          rope, &spec);
  if (st != MLA_OK || n_new == 0) return st;
  const bool bf16 = dims->dtype == MLA_BF16;
  if (bf16) {
    if (!workspace) return MLA_ERR_NULL;
    if (workspace_bytes < mla::kv_append_workspace_bytes(true, n_new, dims->d_c, dims->d_r)) return MLA_ERR_SHAPE;
    if (!aligned(workspace, 4)) return MLA_ERR_ALIGN;
  }
  return launched(mla::launch_kv_append(bf16, h, w_dkv, w_kr, positions, dst_rows, rows, stride,
                                        (float*)workspace, n_new, d_model, dims->d_c, dims->d_r, spec, stream));
}

mla_status_t mla_kv_append_noalloc(const mla_dims_t* dims, int32_t n_new, int32_t d_model, const void* h,
                                   const void* w_dkv, const void* w_kr, const int64_t* positions,
                                   const int64_t* dst_rows, void* rows, int64_t stride, const mla_rope_t* rope,
                                   hipStream_t stream) {
  mla::RopeSpec spec;
  mla_status_t st = kv_append_check(dims, n_new, d_model, h, w_dkv, w_kr, positions, dst_rows, rows, stride, rope,
                                    &spec);
  if (st != MLA_OK || n_new == 0) return st;
  const bool bf16 = dims->dtype == MLA_BF16;
  const size_t need = mla::kv_append_workspace_bytes(bf16, n_new, dims->d_c, dims->d_r);
  if (need > MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_SCRATCH;
  void* ws = nullptr;
  if (need) {
    st = mla::noalloc_scratch(stream, &ws);
    if (st != MLA_OK) return st;
  }
  return launched(mla::launch_kv_append(bf16, h, w_dkv, w_kr, positions, dst_rows, rows, stride, (float*)ws,
                                        n_new, d_model, dims->d_c, dims->d_r, spec, stream));
}

mla_status_t mla_decode(const mla_dims_t* dims, int32_t batch, int32_t q_per_seq, const void* q_abs,
                        const void* c_kv, int64_t c_stride, const void* k_r, int64_t r_stride,
                        const int64_t* seq_offsets, int32_t num_splits, int32_t split_rows,
                        int32_t partial_dtype, void* o_part, float* lse_part, hipStream_t stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (partial_dtype != MLA_F32 && partial_dtype != MLA_F16) return MLA_ERR_DTYPE;
  if (batch < 0 || q_per_seq < 1 || num_splits < 1) return MLA_ERR_SHAPE;
  if (num_splits > 1 && split_rows < 1) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!q_abs || !c_kv || !k_r || !seq_offsets || !o_part || !lse_part) return MLA_ERR_NULL;
  if (c_stride < dims->d_c || r_stride < dims->d_r) return MLA_ERR_SHAPE;
  const int64_t n_q = (int64_t)batch * q_per_seq;
  if (n_q >= kMaxElems / dims->n_h || (int64_t)num_splits * n_q * dims->n_h * dims->d_c >= ((int64_t)1 << 40))
    return MLA_ERR_SHAPE;
  if ((int64_t)num_splits * n_q * dims->n_h >= kMaxElems) return MLA_ERR_SHAPE;
  if (!aligned(seq_offsets, 8) || !aligned(o_part, 4) || !aligned(lse_part, 4)) return MLA_ERR_ALIGN;
  const float scale = scale_of(dims);
  if (dims->dtype == MLA_F32) {
    if (!aligned(q_abs, 4) || !aligned(c_kv, 4) || !aligned(k_r, 4)) return MLA_ERR_ALIGN;
    if (mla::decode_f32_smem_bytes(dims->d_c, dims->d_r) > 64 * 1024) return MLA_ERR_UNSUPPORTED;
    if (num_splits > 65535 || n_q > 65535) return MLA_ERR_UNSUPPORTED;
    if (partial_dtype != MLA_F32) return MLA_ERR_UNSUPPORTED;
    return launched(mla::launch_decode_f32((const float*)q_abs, (const float*)c_kv, c_stride,
                                           (const float*)k_r, r_stride, seq_offsets, (float*)o_part, lse_part,
                                           batch, q_per_seq, dims->n_h, dims->d_c, dims->d_r,
                                           num_splits, split_rows, scale, stream));
  }
  if (dims->d_c != kDecodeDc || dims->d_r != kDecodeDr || dims->n_h % 32) return MLA_ERR_UNSUPPORTED;
  // The kernel streams whole 576-wide rows: the RoPE key must directly follow the latent.
  const bool packed = (const char*)k_r == (const char*)c_kv + 2 * (size_t)dims->d_c && r_stride == c_stride;
  if (!packed) return MLA_ERR_UNSUPPORTED;
  if (!aligned(q_abs, 16) || !aligned(c_kv, 16) || c_stride % 8) return MLA_ERR_ALIGN;
  if (!aligned(o_part, 16)) return MLA_ERR_ALIGN;
  if (c_stride * 2 * 32 >= ((int64_t)1 << 31)) return MLA_ERR_SHAPE;
  return launched(mla::launch_decode_bf16((const uint16_t*)q_abs, (const uint16_t*)c_kv, c_stride,
                                          seq_offsets, o_part, partial_dtype == MLA_F16, lse_part,
                                          batch, q_per_seq, dims->n_h, num_splits, split_rows, scale,
                                          stream));
}

mla_status_t mla_quantize_rows_fp8(const mla_dims_t* dims, int64_t n_rows, const void* rows,
                                   int64_t row_stride, const int64_t* dst_rows, uint8_t* codes,
                                   int64_t code_stride, float* scales, hipStream_t stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  const int64_t width = (int64_t)dims->d_c + dims->d_r;
  if (n_rows < 0 || row_stride < width || code_stride < width) return MLA_ERR_SHAPE;
  if (!mla::quantize_rows_supported((int)width)) return MLA_ERR_UNSUPPORTED;
  if (n_rows == 0) return MLA_OK;
  if (!rows || !codes || !scales) return MLA_ERR_NULL;
  if (n_rows >= ((int64_t)1 << 33) || (n_rows - 1) * row_stride >= ((int64_t)1 << 40)) return MLA_ERR_SHAPE;
  if (!aligned(rows, esize(dims)) || !aligned(scales, 4) || (dst_rows && !aligned(dst_rows, 8))) return MLA_ERR_ALIGN;
  return launched(mla::launch_quantize_rows(dims->dtype == MLA_BF16, rows, row_stride, n_rows, dst_rows, codes,
                                            code_stride, scales, (int)width, stream));
}

mla_status_t mla_decode_fp8(const mla_dims_t* dims, int32_t batch, int32_t q_per_seq, const void* q_abs,
                            const uint8_t* codes, int64_t code_stride, const float* scales,
                            const int64_t* seq_offsets, int32_t num_splits, int32_t split_rows,
                            int32_t partial_dtype, void* o_part, float* lse_part, hipStream_t stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (partial_dtype != MLA_F32 && partial_dtype != MLA_F16) return MLA_ERR_DTYPE;
  if (batch < 0 || q_per_seq < 1 || num_splits < 1) return MLA_ERR_SHAPE;
  if (num_splits > 1 && split_rows < 1) return MLA_ERR_SHAPE;
  if (code_stride < (int64_t)dims->d_c + dims->d_r) return MLA_ERR_SHAPE;
  if (dims->dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (dims->d_c != kDecodeDc || dims->d_r != kDecodeDr || dims->n_h % 32) return MLA_ERR_UNSUPPORTED;
  if (batch == 0) return MLA_OK;
  if (!q_abs || !codes || !scales || !seq_offsets || !o_part || !lse_part) return MLA_ERR_NULL;
  const int64_t n_q = (int64_t)batch * q_per_seq;
  if (n_q >= kMaxElems / dims->n_h || (int64_t)num_splits * n_q * dims->n_h * dims->d_c >= ((int64_t)1 << 40))
    return MLA_ERR_SHAPE;
  if ((int64_t)num_splits * n_q * dims->n_h >= kMaxElems) return MLA_ERR_SHAPE;
  if (code_stride * 32 >= ((int64_t)1 << 31)) return MLA_ERR_SHAPE;
  if (!aligned(seq_offsets, 8) || !aligned(lse_part, 4) || !aligned(scales, 4)) return MLA_ERR_ALIGN;
  if (!aligned(q_abs, 16) || !aligned(codes, 16) || code_stride % 16 || !aligned(o_part, 16)) return MLA_ERR_ALIGN;
  return launched(mla::launch_decode_fp8((const uint16_t*)q_abs, codes, code_stride, scales, seq_offsets, o_part,
                                         partial_dtype == MLA_F16, lse_part, batch, q_per_seq, dims->n_h,
                                         num_splits, split_rows, scale_of(dims), stream));
}

namespace {
// Shared checks of the folding calls: bf16 dims, sizes in range.
mla_status_t fold_dims(const mla_dims_t* dims) {
  const mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  return dims->dtype == MLA_BF16 ? MLA_OK : MLA_ERR_UNSUPPORTED;
}
bool big(int64_t a, int64_t b) { return a * b >= kMaxElems; }
}  // namespace

size_t mla_proj_workspace_bytes(const mla_dims_t* dims, int32_t n_q, int32_t d_model, int32_t d_cq) {
  if (fold_dims(dims) != MLA_OK || n_q <= 0 || d_model <= 0 || d_cq <= 0) return 0;
  const int hd = dims->n_h * dims->d_h, hc = dims->n_h * dims->d_c;
  size_t need = 0;
  if (mla::gemm_xwt_supported(hd, d_cq)) need = mla::gemm_xwt_workspace_bytes(n_q, hd, d_cq, 1);
  if (mla::gemm_xwt_supported(d_model, hd)) {
    const size_t b = mla::gemm_xwt_workspace_bytes(n_q, d_model, hd, 1);
    need = b > need ? b : need;
  }
  if (mla::gemm_xwt_supported(d_model, hc)) {
    const size_t b = mla::gemm_xwt_workspace_bytes(n_q, d_model, hc, 1);
    need = b > need ? b : need;
  }
  return need;
}

mla_status_t mla_q_up(const mla_dims_t* dims, int32_t n_q, int32_t d_cq, const void* c_q, const void* w_uq,
                      void* q_c, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  mla_status_t st = fold_dims(dims);
  if (st != MLA_OK) return st;
  if (n_q < 0 || d_cq < 1) return MLA_ERR_SHAPE;
  const int hd = dims->n_h * dims->d_h;
  if (!mla::gemm_xwt_supported(hd, d_cq)) return MLA_ERR_UNSUPPORTED;
  if (n_q == 0) return MLA_OK;
  if (!c_q || !w_uq || !q_c) return MLA_ERR_NULL;
  if (big(n_q, d_cq) || big(hd, d_cq) || big(n_q, hd)) return MLA_ERR_SHAPE;
  if (!aligned(c_q, 16) || !aligned(w_uq, 16) || !aligned(q_c, 2)) return MLA_ERR_ALIGN;
  const size_t need = mla::gemm_xwt_workspace_bytes(n_q, hd, d_cq, 1);
  if (need && (!workspace || workspace_bytes < need)) return workspace ? MLA_ERR_SHAPE : MLA_ERR_NULL;
  if (need && !aligned(workspace, 4)) return MLA_ERR_ALIGN;
  return launched(mla::launch_gemm_xwt(false, c_q, d_cq, 0, (const uint16_t*)w_uq, d_cq, 0, (uint16_t*)q_c, hd, 0,
                                       (float*)workspace, n_q, hd, d_cq, 1, true, stream));
}

mla_status_t mla_fold_q(const mla_dims_t* dims, int32_t d_cq, const void* w_uq, const void* w_uk, void* g,
                        hipStream_t stream) {
  mla_status_t st = fold_dims(dims);
  if (st != MLA_OK) return st;
  if (d_cq < 1) return MLA_ERR_SHAPE;
  if (!w_uq || !w_uk || !g) return MLA_ERR_NULL;
  if (big((int64_t)dims->n_h * dims->d_c, d_cq) || big((int64_t)dims->n_h * dims->d_h, d_cq)) return MLA_ERR_SHAPE;
  if (!aligned(w_uq, 2) || !aligned(w_uk, 2) || !aligned(g, 2)) return MLA_ERR_ALIGN;
  return launched(mla::launch_fold_q((const uint16_t*)w_uq, (const uint16_t*)w_uk, (uint16_t*)g, dims->n_h,
                                     dims->d_h, dims->d_c, d_cq, stream));
}

mla_status_t mla_absorb_q_folded(const mla_dims_t* dims, int32_t n_q, int32_t d_cq, const void* c_q,
                                 const void* g, const void* q_r, void* q_abs, hipStream_t stream) {
  mla_status_t st = fold_dims(dims);
  if (st != MLA_OK) return st;
  if (n_q < 0 || d_cq < 1) return MLA_ERR_SHAPE;
  if (!mla::gemm_xwt_supported(dims->d_c, d_cq)) return MLA_ERR_UNSUPPORTED;
  if (n_q == 0) return MLA_OK;
  if (!c_q || !g || !q_r || !q_abs) return MLA_ERR_NULL;
  const int64_t d_qk = (int64_t)dims->d_c + dims->d_r;
  if (big(n_q, d_cq) || big((int64_t)dims->n_h * dims->d_c, d_cq) || big((int64_t)n_q * dims->n_h, d_qk))
    return MLA_ERR_SHAPE;
  if (!aligned(c_q, 16) || !aligned(g, 16) || !aligned(q_r, 2) || !aligned(q_abs, 2)) return MLA_ERR_ALIGN;
  st = launched(mla::launch_gemm_xwt(false, c_q, d_cq, 0, (const uint16_t*)g, d_cq, (int64_t)dims->d_c * d_cq,
                                     (uint16_t*)q_abs, dims->n_h * d_qk, d_qk, nullptr, n_q, dims->d_c, d_cq,
                                     dims->n_h, false, stream));
  if (st != MLA_OK) return st;
  return launched(mla::launch_copy_rope((const uint16_t*)q_r, (uint16_t*)q_abs, n_q, dims->n_h, dims->d_c,
                                        dims->d_r, stream));
}

mla_status_t mla_o_proj(const mla_dims_t* dims, int32_t n_q, int32_t d_model, const void* o_c, const void* w_o,
                        void* u, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  mla_status_t st = fold_dims(dims);
  if (st != MLA_OK) return st;
  if (n_q < 0 || d_model < 1) return MLA_ERR_SHAPE;
  const int hd = dims->n_h * dims->d_h;
  if (!mla::gemm_xwt_supported(d_model, hd)) return MLA_ERR_UNSUPPORTED;
  if (n_q == 0) return MLA_OK;
  if (!o_c || !w_o || !u) return MLA_ERR_NULL;
  if (big(n_q, hd) || big(d_model, hd) || big(n_q, d_model)) return MLA_ERR_SHAPE;
  if (!aligned(o_c, 16) || !aligned(w_o, 16) || !aligned(u, 2)) return MLA_ERR_ALIGN;
  const size_t need = mla::gemm_xwt_workspace_bytes(n_q, d_model, hd, 1);
  if (need && (!workspace || workspace_bytes < need)) return workspace ? MLA_ERR_SHAPE : MLA_ERR_NULL;
  if (need && !aligned(workspace, 4)) return MLA_ERR_ALIGN;
  return launched(mla::launch_gemm_xwt(false, o_c, hd, 0, (const uint16_t*)w_o, hd, 0, (uint16_t*)u, d_model, 0,
                                       (float*)workspace, n_q, d_model, hd, 1, true, stream));
}

mla_status_t mla_fold_o(const mla_dims_t* dims, int32_t d_model, const void* w_o, const void* w_uv, void* w_fold,
                        hipStream_t stream) {
  mla_status_t st = fold_dims(dims);
  if (st != MLA_OK) return st;
  if (d_model < 1) return MLA_ERR_SHAPE;
  if (!w_o || !w_uv || !w_fold) return MLA_ERR_NULL;
  if (big(d_model, (int64_t)dims->n_h * dims->d_c) || big(d_model, (int64_t)dims->n_h * dims->d_h)) return MLA_ERR_SHAPE;
  if (!aligned(w_o, 2) || !aligned(w_uv, 2) || !aligned(w_fold, 2)) return MLA_ERR_ALIGN;
  return launched(mla::launch_fold_o((const uint16_t*)w_o, (const uint16_t*)w_uv, (uint16_t*)w_fold, dims->n_h,
                                     dims->d_h, dims->d_c, d_model, stream));
}

mla_status_t mla_out_folded(const mla_dims_t* dims, int32_t n_q, int32_t d_model, const float* o_lat,
                            const void* w_fold, void* u, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  mla_status_t st = fold_dims(dims);
  if (st != MLA_OK) return st;
  if (n_q < 0 || d_model < 1) return MLA_ERR_SHAPE;
  const int hc = dims->n_h * dims->d_c;
  if (!mla::gemm_xwt_supported(d_model, hc)) return MLA_ERR_UNSUPPORTED;
  if (n_q == 0) return MLA_OK;
  if (!o_lat || !w_fold || !u) return MLA_ERR_NULL;
  if (big(n_q, hc) || big(d_model, hc) || big(n_q, d_model)) return MLA_ERR_SHAPE;
  if (!aligned(o_lat, 16) || !aligned(w_fold, 16) || !aligned(u, 2)) return MLA_ERR_ALIGN;
  const size_t need = mla::gemm_xwt_workspace_bytes(n_q, d_model, hc, 1);
  if (need && (!workspace || workspace_bytes < need)) return workspace ? MLA_ERR_SHAPE : MLA_ERR_NULL;
  if (need && !aligned(workspace, 4)) return MLA_ERR_ALIGN;
  return launched(mla::launch_gemm_xwt(true, o_lat, hc, 0, (const uint16_t*)w_fold, hc, 0, (uint16_t*)u, d_model, 0,
                                       (float*)workspace, n_q, d_model, hc, 1, true, stream));
}

mla_status_t mla_merge_splits(const mla_dims_t* dims, int32_t n_q, int32_t num_splits,
                              int32_t partial_dtype, const void* o_part, const float* lse_part,
                              float* o_lat, float* lse, hipStream_t stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (partial_dtype != MLA_F32 && partial_dtype != MLA_F16) return MLA_ERR_DTYPE;
  if (n_q < 0 || num_splits < 1) return MLA_ERR_SHAPE;
  if (n_q == 0) return MLA_OK;
  if (!o_part || !lse_part || !o_lat || !lse) return MLA_ERR_NULL;
  if ((int64_t)n_q * dims->n_h >= kMaxElems || (int64_t)num_splits * n_q * dims->n_h >= kMaxElems)
    return MLA_ERR_SHAPE;
  const uintptr_t a = dims->d_c % 8 == 0 ? 16 : (partial_dtype == MLA_F16 ? 2 : 4);
  if (!aligned(o_part, a) || !aligned(o_lat, dims->d_c % 8 == 0 ? 16 : 4) || !aligned(lse_part, 4) ||
      !aligned(lse, 4))
    return MLA_ERR_ALIGN;
  return launched(mla::launch_merge(o_part, partial_dtype == MLA_F16, lse_part, o_lat, lse, n_q,
                                    dims->n_h, dims->d_c, num_splits, stream));
}

mla_status_t mla_merge_out_proj(const mla_dims_t* dims, int32_t n_q, int32_t num_splits,
                                int32_t partial_dtype, const void* o_part, const float* lse_part,
                                const void* w_uv, void* o_c, float* lse, float* o_lat,
                                hipStream_t stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (partial_dtype != MLA_F32 && partial_dtype != MLA_F16) return MLA_ERR_DTYPE;
  if (n_q < 0 || num_splits < 1) return MLA_ERR_SHAPE;
  if (n_q == 0) return MLA_OK;
  if (!o_part || !lse_part || !w_uv || !o_c) return MLA_ERR_NULL;
  if ((int64_t)n_q * dims->n_h * dims->d_c >= kMaxElems ||
      (int64_t)num_splits * n_q * dims->n_h * dims->d_c >= kMaxElems ||
      (int64_t)dims->n_h * dims->d_h * dims->d_c >= kMaxElems)
    return MLA_ERR_SHAPE;
  if (dims->dtype == MLA_F32) {
    // The plain fp32 kernels, one after the other, with o_lat and lse as the intermediate.
    if (!o_lat || !lse) return MLA_ERR_NULL;
    st = mla_merge_splits(dims, n_q, num_splits, partial_dtype, o_part, lse_part, o_lat, lse, stream);
    if (st != MLA_OK) return st;
    return mla_out_proj(dims, n_q, o_lat, w_uv, o_c, stream);
  }
  if (!mla::merge_out_proj_bf16_supported(dims->d_h, dims->d_c)) return MLA_ERR_UNSUPPORTED;
  if (!aligned(o_part, 16) || !aligned(w_uv, 16) || !aligned(o_c, 2) || !aligned(lse_part, 4) ||
      (lse && !aligned(lse, 4)) || (o_lat && !aligned(o_lat, 16)))
    return MLA_ERR_ALIGN;
  return launched(mla::launch_merge_out_proj_bf16(o_part, partial_dtype == MLA_F16, lse_part,
                                                  (const uint16_t*)w_uv, (uint16_t*)o_c, lse, o_lat,
                                                  n_q, dims->n_h, dims->d_h, num_splits, stream));
}

mla_status_t mla_out_proj(const mla_dims_t* dims, int32_t n_q, const float* o_lat, const void* w_uv,
                          void* o_c, hipStream_t stream) {
  mla_status_t st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (n_q < 0) return MLA_ERR_SHAPE;
  if (n_q == 0) return MLA_OK;
  if (!o_lat || !w_uv || !o_c) return MLA_ERR_NULL;
  if ((int64_t)n_q * dims->n_h * dims->d_c >= kMaxElems ||
      (int64_t)dims->n_h * dims->d_h * dims->d_c >= kMaxElems)
    return MLA_ERR_SHAPE;
  if (!aligned(o_lat, 4) || !aligned(w_uv, esize(dims)) || !aligned(o_c, esize(dims))) return MLA_ERR_ALIGN;
  if (dims->dtype == MLA_F32)
    return launched(mla::launch_out_proj_f32(o_lat, (const float*)w_uv, (float*)o_c, n_q, dims->n_h,
                                             dims->d_h, dims->d_c, stream));
  if (!mla::out_proj_bf16_supported(dims->d_h, dims->d_c)) return MLA_ERR_UNSUPPORTED;
  if (!aligned(o_lat, 16) || !aligned(w_uv, 16)) return MLA_ERR_ALIGN;
  return launched(mla::launch_out_proj_bf16(o_lat, (const uint16_t*)w_uv, (uint16_t*)o_c, n_q,
                                            dims->n_h, dims->d_h, dims->d_c, stream));
}

}  // extern "C"
