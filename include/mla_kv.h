/*
 * mla_kv.h - C ABI of the MLA absorbed-decode library for MI355X (gfx950).
 *
 * Multi-head Latent Attention decode over a compressed KV cache with the
 * up-projections absorbed.  Pages cited (title, then section / equation):
 *   [notes]  "MLA(Multi-head Latent Attention): DeepSeek-V2 논문정리"
 *   [report] "Техотчёт DeepSeek-V2 (2024): MLA и экономика инференса"
 *   [review] "DeepSeek-V2 review" (velog.io/@jmsong62)
 *   [v3]     DeepSeek-V3 Technical Report notes (xuxeong.tistory.com)
 *
 * Each cached token holds one latent row [c^KV (d_c) ; k^R (d_r)]: the
 * compressed latent of eq. 9 [notes] and the shared decoupled RoPE key, cached
 * already rotated ([notes] "Decoupled Rotary Position Embedding"; [report]
 * "Идея 2").  One decode step is four calls:
 *
 *   mla_absorb_q      q_abs = [W^UK_i^T q^C_i ; q^R_i]          (key absorption)
 *   mla_decode        per split of the rows: softmax(q_abs . row * scale)
 *                     weighted sum of c^KV, plus its log-sum-exp
 *   mla_merge_splits  log-sum-exp weighted combination of the splits
 *   mla_out_proj      o^C_i = W^UV_i o_lat_i                     (value absorption)
 *
 * mla_merge_out_proj does the last two in one call, with the same results.
 * mla_plan_splits picks mla_decode's split plan from the sequence lengths (host code).
 *
 * The decode prologue builds this step's inputs from the hidden states:
 *   mla_kv_append     new cache rows [W^DKV h ; RoPE(W^KR h)] at given rows
 *   mla_absorb_q_rope mla_absorb_q with q^R rotated at the tokens' positions
 *
 * From the compressed query c^Q to the block output u, unfolded and with folded weights:
 *   mla_q_up, mla_o_proj                 q^C = W^UQ c^Q;  u = W^O [o^C_1; ...; o^C_nh]
 *   mla_fold_q, mla_absorb_q_folded      G_i = (W^UK_i)^T W^UQ_i;  q_abs = [G_i c^Q ; q^R]
 *   mla_fold_o, mla_out_folded           W'^O = W^O W^UV;  u = W'^O [o_lat_1; ...]
 *
 * A quantized cache keeps each row as FP8 E4M3 codes with one fp32 scale:
 *   mla_quantize_rows_fp8  rows -> codes and scales
 *   mla_decode_fp8         mla_decode over the dequantized rows value(code) * scale
 *
 * Together they compute, for query t and head i,
 *   o_{t,i} = sum_j softmax_j(q_{t,i}^T k_{j,i} * scale) v^C_{j,i}
 * with k_{j,i} = [W^UK_i c^KV_j ; k^R_j], v^C_{j,i} = W^UV_i c^KV_j and
 * scale = 1/sqrt(d_h + d_r) ([v3] eq. 10; [report] "Идея 2").
 *
 * Conventions shared by every call
 *  - All tensor arguments are device pointers, row-major, densely packed unless
 *    a stride is given.  The caller owns every buffer; the library allocates
 *    nothing and keeps no state (mla_kv_append_noalloc's fixed device array, one
 *    per GPU, aside).  Outputs must not overlap inputs.
 *  - Every call only enqueues work on `stream` (0 = the null stream) and
 *    returns; it never synchronizes.  Calls on one stream run in order.
 *  - Arguments are checked on the host before anything is launched; a failed
 *    check returns its MLA_ERR_* code and launches nothing.  MLA_ERR_LAUNCH
 *    reports a HIP launch error.  No call aborts or throws.
 *  - A size of zero (n_q == 0, batch == 0) is a valid no-op.
 *  - dtype MLA_BF16 runs the MFMA kernels (bf16 operands, fp32 accumulation):
 *    mla_decode needs d_c == 512, d_r == 64 and n_h % 32 == 0; mla_absorb_q
 *    needs d_c % 128 == 0, d_h % 16 == 0, d_h <= 256, d_r % 8 == 0;
 *    mla_out_proj needs d_h % 32 == 0, d_c % 64 == 0, d_c <= 512 (the
 *    DeepSeek-V2 attention shape fits all) and 16-byte aligned rows;
 *    mla_merge_out_proj needs d_c == 512 and d_h == 128; mla_kv_append needs
 *    d_model % 512 == 0, d_model <= 8192 and (d_c + d_r) % 32 == 0; mla_absorb_q_rope needs
 *    mla_absorb_q's shapes and d_r <= 512; other
 *    shapes return MLA_ERR_UNSUPPORTED.  dtype MLA_F32 runs plain fp32
 *    kernels for any shape (no bf16 rounding anywhere).
 */
#ifndef MLA_KV_H_
#define MLA_KV_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 10

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,         /* a required pointer is NULL */
  MLA_ERR_SHAPE = 2,        /* a size, count or stride is out of range */
  MLA_ERR_ALIGN = 3,        /* a pointer or stride breaks the alignment rule */
  MLA_ERR_DTYPE = 4,        /* dims->dtype is not an mla_dtype_t value */
  MLA_ERR_UNSUPPORTED = 5,  /* valid arguments the library has no kernel for */
  MLA_ERR_LAUNCH = 6,       /* a HIP launch failed (see hipGetLastError) */
  MLA_ERR_SCRATCH = 7,      /* more than a fixed device array holds (mla_kv_append_noalloc) */
  MLA_ERR_DEVICE = 8        /* the stream is not on the current device (mla_kv_append_noalloc) */
} mla_status_t;

typedef enum mla_dtype {
  MLA_F32 = 0,              /* float32 storage and arithmetic */
  MLA_BF16 = 1,             /* bfloat16 storage, fp32 accumulation */
  MLA_F16 = 2               /* float16: storage of split partials only (see mla_decode) */
} mla_dtype_t;

/* Attention dimensions ([review] 4.1; [v3] MLA dimension list). */
typedef struct mla_dims {
  int32_t n_h;              /* query heads (DeepSeek-V2: 128) */
  int32_t d_h;              /* per-head width of q^C, k^C, v^C (128) */
  int32_t d_c;              /* latent width of c^KV (512) */
  int32_t d_r;              /* decoupled RoPE width d_h^R of q^R and k^R (64) */
  int32_t dtype;            /* mla_dtype_t of every non-fp32 tensor below */
  float softmax_scale;      /* > 0: used as given; <= 0: 1/sqrt(d_h + d_r) */
} mla_dims_t;

/* RoPE of the decoupled key and query (mla_kv_append, mla_absorb_q_rope).  Pair k of a
 * d_r-wide vector turns by f_k = theta^(-2k/d_r) per position ([notes] "MLA 코드 구현").
 * With yarn_factor s > 1 the frequencies follow YaRN's NTK-by-parts, which DeepSeek-V2 applies
 * to the decoupled key only ([report] training and infrastructure section: s = 40, alpha = 1,
 * beta = 32; [review] section 4): a pair that makes r = L f_k / (2 pi) turns over the
 * training length L keeps f_k when r >= beta, turns at f_k / s when r <= alpha, and at
 * (1 - g) f_k / s + g f_k, g = (r - alpha) / (beta - alpha), in between.  The logits' length
 * factor t, sqrt(t) = yarn_mscale * ln s + 1 (DeepSeek-V2: 0.0707), multiplies the softmax
 * scale: mla_rope_softmax_scale gives the value for mla_dims_t.softmax_scale. */
typedef struct mla_rope {
  float theta;              /* > 0: the base; <= 0: 10000 */
  float yarn_factor;        /* s; <= 1: plain RoPE (the other YaRN fields are ignored) */
  int32_t yarn_original_len;/* L, the training length (DeepSeek-V2: 4096); > 0 with s > 1 */
  float yarn_alpha;         /* alpha (1) */
  float yarn_beta;          /* beta (32); > alpha with s > 1 */
  float yarn_mscale;        /* coefficient of ln s in sqrt(t) (0.0707) */
} mla_rope_t;

/* Softmax scale with YaRN's length factor: (dims->softmax_scale > 0 ? it : 1/sqrt(d_h + d_r))
 * * t, t = (yarn_mscale * ln s + 1)^2 for s > 1, else 1.  NULL dims: 0; NULL rope: no factor. */
float mla_rope_softmax_scale(const mla_dims_t* dims, const mla_rope_t* rope);

/* Library ABI version (MLA_ABI_VERSION of the build). */
int32_t mla_abi_version(void);

/* Static text for a status code; never NULL. */
const char* mla_status_string(mla_status_t status);

/*
 * mla_absorb_q - fold W^UK into the query ([notes] "Key에 대한 수식 전개";
 * [report] "Идея 1") and append the RoPE part unchanged ([notes] "Decoupled
 * Rotary Position Embedding", item 4: [a;b].[c;d] = a.c + b.d).
 *
 *   q_abs[n, i, 0:d_c]       = sum_d q_c[n, i, d] * w_uk[i, d, :]
 *   q_abs[n, i, d_c:d_c+d_r] = q_r[n, i, :]
 *
 *   q_c   [n_q, n_h, d_h]        dtype      per-head content query q^C
 *   q_r   [n_q, n_h, d_r]        dtype      per-head RoPE query, already rotated
 *   w_uk  [n_h, d_h, d_c]        dtype      W^UK_i as [d_h, d_c] per head
 *   q_abs [n_q, n_h, d_c + d_r]  dtype      out; bf16 is rounded once from fp32
 *
 * bf16 needs 16-byte aligned q_c, q_r, w_uk and q_abs (MLA_ERR_ALIGN otherwise): the
 * kernels move every operand in 16-byte pieces.
 */
mla_status_t mla_absorb_q(const mla_dims_t* dims, int32_t n_q,
                          const void* q_c, const void* q_r, const void* w_uk,
                          void* q_abs, hipStream_t stream);

/*
 * mla_absorb_q_rope - mla_absorb_q with the RoPE part rotated first: every head's
 * q_r_raw[n, i, :] is rotated at positions[n] ([notes] "MLA 코드 구현": q^R is rotated
 * head by head at the new tokens' positions; RoPE as in mla_kv_append), then
 *   q_abs[n, i, 0:d_c]       = sum_d q_c[n, i, d] * w_uk[i, d, :]
 *   q_abs[n, i, d_c:d_c+d_r] = RoPE(q_r_raw[n, i, :], positions[n])
 *
 *   q_r_raw    [n_q, n_h, d_r]   dtype   per-head RoPE query before rotation
 *   positions  [n_q] int64, device memory: each query token's position
 *   rope       RoPE parameters (mla_rope_t), or NULL: theta = 10000, no YaRN
 * Other arguments and errors as mla_absorb_q; positions must be 8-byte aligned
 * and non-NULL (MLA_ERR_NULL); bf16 needs d_r <= 512.  The angle is fp64, reduced
 * to [-pi, pi] in fp64; its sine and cosine are fp32 (relative error ~1e-7).
 */
mla_status_t mla_absorb_q_rope(const mla_dims_t* dims, int32_t n_q, const void* q_c,
                               const void* q_r_raw, const void* w_uk, const int64_t* positions,
                               const mla_rope_t* rope, void* q_abs, hipStream_t stream);

/*
 * mla_kv_append - the new tokens' latent rows, written into the cache ([notes]
 * eq. 9 and "Decoupled Rotary Position Embedding", items 2-3; "MLA 코드 구현":
 * the down-projections apply to the new tokens only and the cache keeps k^R
 * after rotation).  For new token t:
 *   c^KV_t = W^DKV h_t,   k^R_t = RoPE(W^KR h_t, positions[t])
 *   rows[dst_rows[t] * stride + 0 : d_c]         = c^KV_t
 *   rows[dst_rows[t] * stride + d_c : d_c + d_r] = k^R_t
 * RoPE rotates the pairs (v_k, v_{k+d_r/2}), k < d_r/2, by the angle
 * positions[t] * f_k (mla_rope_t): (v_k cos - v_{k+d_r/2} sin, v_{k+d_r/2} cos + v_k sin),
 * the rotate-half form of the listing in "MLA 코드 구현"; the angle is fp64, reduced
 * to [-pi, pi] in fp64, with fp32 sine and cosine and an fp64 rotation (relative error
 * ~1e-7).  No other cache element is touched.
 *
 *   h          [n_new, d_model]      dtype   hidden states of the new tokens
 *   w_dkv      [d_c, d_model]        dtype   W^DKV
 *   w_kr       [d_r, d_model]        dtype   W^KR
 *   positions  [n_new] int64, device memory: each token's position
 *   dst_rows   [n_new] int64, device memory: each token's cache row; distinct rows,
 *              each below the number of rows behind `rows` (not checked)
 *   rows       cache rows [*, stride] in dtype, packed [c^KV | k^R] (stride >= d_c + d_r)
 *   rope       RoPE parameters (mla_rope_t), or NULL: theta = 10000, no YaRN
 *   workspace  device scratch of at least mla_kv_append_workspace_bytes(dims, n_new)
 *              bytes (bf16: fp32 partial sums over slices of d_model; fp32 needs none and
 *              may pass NULL, 0); its contents on entry do not matter, on return they are
 *              undefined.  Calls that share a workspace must not overlap.
 * bf16: fp32 accumulation (slices of d_model summed in a fixed order), each output
 * rounded once to bf16 (the k^R outputs after the rotation of the fp32 sums);
 * needs d_model % 512 == 0, d_model <= 8192, (d_c + d_r) % 32 == 0 (else
 * MLA_ERR_UNSUPPORTED) and 16-byte aligned h, w_dkv and w_kr.  fp32: any shape.
 * positions and dst_rows 8-byte aligned, workspace 4-byte aligned.  A rope with s > 1 needs
 * yarn_original_len > 0 and yarn_beta > yarn_alpha, all finite (else MLA_ERR_SHAPE); the same
 * holds for mla_absorb_q_rope.
 */
size_t mla_kv_append_workspace_bytes(const mla_dims_t* dims, int32_t n_new);
mla_status_t mla_kv_append(const mla_dims_t* dims, int32_t n_new, int32_t d_model, const void* h,
                           const void* w_dkv, const void* w_kr, const int64_t* positions,
                           const int64_t* dst_rows, void* rows, int64_t stride, const mla_rope_t* rope,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Size of the fixed device array behind mla_kv_append_noalloc: 8 MiB per GPU. */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

/*
 * mla_kv_append_noalloc - mla_kv_append for callers that cannot allocate device memory:
 * code under HIP graph capture, serving loops and harnesses that forbid hipMalloc.  The
 * same arguments and the same checks as mla_kv_append without the workspace; its fp32
 * partial sums go to a fixed array of MLA_NOALLOC_SCRATCH_BYTES inside this library, one
 * per GPU, held from the first call on that GPU until the process ends.  The call itself
 * allocates nothing: no hipMalloc, no hipFree, no allocating library routine.
 *  - needs mla_kv_append_workspace_bytes(dims, n_new) <= MLA_NOALLOC_SCRATCH_BYTES
 *    (at d_c + d_r = 576: n_new <= 455), else MLA_ERR_SCRATCH; fp32 uses no scratch;
 *  - `stream` must belong to the current device, else MLA_ERR_DEVICE;
 *  - the array keeps the last call's partial sums; every call writes each entry before
 *    reading it, so nothing needs clearing;
 *  - every call on one GPU shares that GPU's array: calls that overlap in time (two
 *    streams, two host threads) race, and the caller must order them.
 * Outputs equal mla_kv_append's bit for bit (the same kernels).
 */
mla_status_t mla_kv_append_noalloc(const mla_dims_t* dims, int32_t n_new, int32_t d_model, const void* h,
                                   const void* w_dkv, const void* w_kr, const int64_t* positions,
                                   const int64_t* dst_rows, void* rows, int64_t stride,
                                   const mla_rope_t* rope, hipStream_t stream);

/*
 * mla_quantize_rows_fp8 - quantize cache rows to FP8 E4M3 codes with one scale per row.
 * The pages report a KV cache quantized to about 6 bits per element in serving ([review]
 * section 4, "Inference efficiency"; [report] the 93.3% derivation and the economics
 * section) and give no format; this is a first concrete one.  For source row i, with
 * x its first d_c + d_r elements (the row [c^KV ; k^R]) and every step in fp32:
 *   s     = max_k |x_k| / 448                        (correctly rounded division)
 *   c_k   = the OCP E4M3 ("fn") code nearest to x_k / s (correctly rounded division),
 *           ties to even, magnitudes above 448 saturated to 448; sign bit from x_k / s
 *   a row of zeros gets s = 0 and all codes 0
 *   codes[dst * code_stride + k] = c_k,   scales[dst] = s,   dst = dst_rows ? dst_rows[i] : i
 * Dequantized value: value(c_k) * s, with value(c) = (-1)^(c>>7) 2^(e-7) (1 + m/8) for
 * e = (c>>3)&15 > 0, (-1)^(c>>7) 2^-6 m/8 for e = 0, m = c&7 (0x7F, 0xFF: NaN, never written).
 *
 *   rows       [n_rows, row_stride] in dims->dtype (MLA_BF16 or MLA_F32)
 *   dst_rows   [n_rows] int64 device memory, or NULL; distinct, each below the number
 *              of code rows (not checked)
 *   codes      uint8 code rows of code_stride >= d_c + d_r bytes
 *   scales     fp32, one per code row
 * Needs d_c + d_r <= 1024 (else MLA_ERR_UNSUPPORTED), row_stride >= d_c + d_r, dst_rows
 * 8-byte and scales 4-byte aligned; finite inputs.  One wave per row; not on the decode's
 * hot loop.
 */
mla_status_t mla_quantize_rows_fp8(const mla_dims_t* dims, int64_t n_rows, const void* rows,
                                   int64_t row_stride, const int64_t* dst_rows, uint8_t* codes,
                                   int64_t code_stride, float* scales, hipStream_t stream);

/*
 * mla_decode_fp8 - mla_decode over a quantized cache: row j's key is
 * value(codes_j[0 : d_c + d_r]) * scales[j] and its value value(codes_j[0 : d_c]) * scales[j]
 * (codes and scales as mla_quantize_rows_fp8 writes them).  Sequences, masks, splits,
 * outputs and the empty-split rule are those of mla_decode.
 *
 *   q_abs       [batch*q_per_seq, n_h, d_c+d_r] bf16 (dims->dtype must be MLA_BF16)
 *   codes       code rows of code_stride bytes;  scales  fp32, one per code row
 *   seq_offsets, num_splits, split_rows, partial_dtype, o_part, lse_part  as mla_decode
 * Scores: the codes are E4M3 MFMA operands as stored; each head's bf16 query is scaled by a
 * power of two and split into two E4M3 parts whose sum is exact for every component above
 * 2^-10 of the head's largest.  The E4M3 MFMA adds its products with about 13 bits below
 * the largest of each group of 8 (logit error a few 1e-5 at DeepSeek-V2 scale).  Weighted
 * sum: the codes widen exactly to bf16 MFMA operands.  The row scale multiplies the fp32
 * scores and is folded into each softmax weight before that weight's rounding to bf16.
 * Needs d_c == 512, d_r == 64, n_h % 32 == 0 (else MLA_ERR_UNSUPPORTED); codes, q_abs and
 * o_part 16-byte aligned, code_stride a multiple of 16, scales 4-byte aligned.
 */
mla_status_t mla_decode_fp8(const mla_dims_t* dims, int32_t batch, int32_t q_per_seq, const void* q_abs,
                            const uint8_t* codes, int64_t code_stride, const float* scales,
                            const int64_t* seq_offsets, int32_t num_splits, int32_t split_rows,
                            int32_t partial_dtype, void* o_part, float* lse_part, hipStream_t stream);

/*
 * Weight folding ([notes] eq. 13 and "Decoupled Rotary Position Embedding": the score's content
 * term (c^Q)^T (W^UQ)^T W^UK c^KV has a token-independent middle product; "Value에 대한 수식
 * 전개": W'^O = W^O W^UV; [report] "Идея 1").  bf16 only (dims->dtype MLA_BF16); fp32
 * accumulation, every output rounded once to bf16.  Layouts (row-major):
 *   c_q    [n_q, d_cq]                      compressed query c^Q
 *   w_uq   [n_h, d_h, d_cq]                 head i's rows of W^UQ (q^C_i = W^UQ_i c^Q)
 *   q_c    [n_q, n_h, d_h]                  q^C, the input of mla_absorb_q
 *   g      [n_h, d_c, d_cq]                 G_i = (W^UK_i)^T W^UQ_i: c^Q -> absorbed query
 *   o_c    [n_q, n_h, d_h]                  per-head outputs (mla_out_proj)
 *   w_o    [d_model, n_h * d_h]             W^O; columns i d_h .. i d_h + d_h - 1 act on head i
 *   w_fold [d_model, n_h * d_c]             W'^O_i = W^O_i W^UV_i, side by side
 *   u      [n_q, d_model]                   the block output
 * Decode-time products (mla_q_up, mla_absorb_q_folded, mla_o_proj, mla_out_folded) stream
 * their weight once; long reductions are split over workgroups with fp32 partial sums in the
 * caller's workspace (mla_proj_workspace_bytes; contents undefined on return; calls sharing
 * it must not overlap).  They need d_cq, d_c, d_model, n_h * d_h and n_h * d_c multiples of
 * 128 (DeepSeek-V2: 1536, 512, 5120, 16384, 65536), else MLA_ERR_UNSUPPORTED, and 16-byte
 * aligned tensors.  The folds (mla_fold_q, mla_fold_o) are offline: plain fp32 kernels, any
 * shape.  mla_absorb_q_folded copies q_r (already rotated) into the RoPE part as mla_absorb_q.
 */
size_t mla_proj_workspace_bytes(const mla_dims_t* dims, int32_t n_q, int32_t d_model, int32_t d_cq);
mla_status_t mla_q_up(const mla_dims_t* dims, int32_t n_q, int32_t d_cq, const void* c_q, const void* w_uq,
                      void* q_c, void* workspace, size_t workspace_bytes, hipStream_t stream);
mla_status_t mla_fold_q(const mla_dims_t* dims, int32_t d_cq, const void* w_uq, const void* w_uk, void* g,
                        hipStream_t stream);
mla_status_t mla_absorb_q_folded(const mla_dims_t* dims, int32_t n_q, int32_t d_cq, const void* c_q,
                                 const void* g, const void* q_r, void* q_abs, hipStream_t stream);
mla_status_t mla_o_proj(const mla_dims_t* dims, int32_t n_q, int32_t d_model, const void* o_c, const void* w_o,
                        void* u, void* workspace, size_t workspace_bytes, hipStream_t stream);
mla_status_t mla_fold_o(const mla_dims_t* dims, int32_t d_model, const void* w_o, const void* w_uv, void* w_fold,
                        hipStream_t stream);
/* o_lat [n_q, n_h, d_c] fp32 (rounded to bf16 as the MFMA operand, as mla_out_proj). */
mla_status_t mla_out_folded(const mla_dims_t* dims, int32_t n_q, int32_t d_model, const float* o_lat,
                            const void* w_fold, void* u, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* Bytes of o_part for (n_q, num_splits, partial_dtype):
 * num_splits * n_q * n_h * d_c * (4 for MLA_F32, 2 for MLA_F16).  lse_part holds
 * num_splits * n_q * n_h floats.  Returns 0 on bad arguments. */
size_t mla_partial_bytes(const mla_dims_t* dims, int32_t n_q, int32_t num_splits,
                         int32_t partial_dtype);

/* Bytes of the split buffers of a decode plan with fp32 split results, the larger form:
 * mla_partial_bytes(dims, n_q, num_splits, MLA_F32) for o_part plus
 * num_splits * n_q * n_h * 4 for lse_part.  The caller owns both buffers (the library
 * allocates nothing); fp16 split results need mla_partial_bytes(..., MLA_F16) for o_part.
 * Returns 0 on bad arguments. */
size_t mla_decode_workspace_bytes(const mla_dims_t* dims, int32_t n_q, int32_t num_splits);

/*
 * mla_decode - attention of every query head over the latent rows, one result
 * per split of the rows.
 *
 * Sequence b owns cache rows seq_offsets[b] .. seq_offsets[b+1]-1 (len_b rows,
 * the q_per_seq newest of them being this step's own tokens when q_per_seq > 1).
 * Query r (0 <= r < q_per_seq) of sequence b is query n = b*q_per_seq + r and
 * sees the first vis = len_b - q_per_seq + r + 1 rows (the generalized causal
 * mask of [notes] "MLA 코드 구현", triu with diagonal T_k - T_q + 1).  Row j's
 * key is the whole row [c_kv_j ; k_r_j], shared by all heads; its value is c_kv_j.
 *
 * Split s covers visible rows [s*split_rows, (s+1)*split_rows); the last split
 * (s = num_splits-1) runs to the end of the visible rows; with num_splits == 1
 * the single split covers all of them.  For each (s, n, i), with
 * x_j = q_abs[n,i,:] . row_j * scale over the split's rows:
 *   o_part[s, n, i, :] = sum_j softmax(x)_j * c_kv_j        (fp32)
 *   lse_part[s, n, i]  = ln sum_j exp(x_j)                  (fp32, natural log)
 * A split with no row gets lse_part = -inf and its o_part entries are not
 * written (they keep whatever the buffer held); mla_merge_splits and
 * mla_merge_out_proj give such a split weight zero and do not use its o_part.
 * With num_splits == 1 (and no empty split) the outputs already are the final
 * o_lat and lse.
 *
 *   q_abs       [batch*q_per_seq, n_h, d_c+d_r]  dtype   from mla_absorb_q
 *   c_kv        rows of d_c elements at a stride of c_stride elements  dtype
 *   k_r         rows of d_r elements at a stride of r_stride elements  dtype
 *               (packed rows: k_r = c_kv + d_c with r_stride == c_stride)
 *   seq_offsets [batch+1] int64, device memory, nondecreasing, the last entry at
 *               most the number of rows behind c_kv and k_r; every len_b must be
 *               >= q_per_seq.  Not read on the host, so not checked here: use
 *               mla_check_offsets on a host copy.
 *   num_splits  >= 1;  split_rows >= 1 when num_splits > 1 (ignored otherwise)
 *   partial_dtype  MLA_F32, or MLA_F16 (bf16 dtype only): storage of o_part.  fp16
 *               halves the traffic of the split results (each split's o is a softmax-
 *               weighted mean of latents, rounded once to 11 significant bits); it
 *               needs |c_kv| < 65504.
 *   o_part      [num_splits, batch*q_per_seq, n_h, d_c] out, in partial_dtype
 *   lse_part    [num_splits, batch*q_per_seq, n_h] fp32 out
 * bf16 streams whole 576-element rows, so it needs the packed row layout
 * [c^KV ; k^R]: k_r == c_kv + d_c and r_stride == c_stride (else
 * MLA_ERR_UNSUPPORTED); c_kv, q_abs and o_part 16-byte aligned, c_stride a
 * multiple of 8.  fp32 takes separate c_kv / k_r tensors with any strides.
 */
mla_status_t mla_decode(const mla_dims_t* dims, int32_t batch, int32_t q_per_seq,
                        const void* q_abs,
                        const void* c_kv, int64_t c_stride,
                        const void* k_r, int64_t r_stride,
                        const int64_t* seq_offsets,
                        int32_t num_splits, int32_t split_rows, int32_t partial_dtype,
                        void* o_part, float* lse_part, hipStream_t stream);

/*
 * mla_check_offsets - host-side check of a host copy of seq_offsets against
 * the rules mla_decode relies on: offsets[0] >= 0, nondecreasing, every
 * len_b >= q_per_seq, offsets[batch] <= total_rows.  Returns MLA_OK or
 * MLA_ERR_SHAPE (MLA_ERR_NULL for a NULL array with batch > 0).
 */
mla_status_t mla_check_offsets(const int64_t* host_offsets, int32_t batch,
                               int32_t q_per_seq, int64_t total_rows);

/*
 * mla_plan_splits - choose num_splits and split_rows for mla_decode (and mla_decode_fp8) from
 * the sequences' lengths.  Any partition of a query's visible rows into splits merges to the
 * same attention ([notes] "Key에 대한 수식 전개": one softmax over all visible rows; the
 * merge is exact by log-sum-exp), so the plan only decides speed.  The choice comes from a
 * model of the decode on MI355X: the kernel's own dealing of workgroups to the 8 XCDs and
 * their order within an XCD, every CU taking the next workgroup when it frees up, a fixed
 * start plus a time per 32-row tile for each workgroup, and the split results' bytes for
 * the merge.  Host code only; nothing runs on the GPU.
 *
 *   dims         n_h, d_h and d_c are used (the heads per workgroup, the split results' size
 *                and the weights the merge reads)
 *   host_offsets [batch+1] int64 in host memory: the seq_offsets mla_decode will take
 *   q_per_seq    as mla_decode
 *   max_splits   the largest num_splits the caller's split buffers allow (>= 1)
 *   num_splits, split_rows  out: the plan; split_rows is a multiple of 32, and 0 with
 *                num_splits == 1
 * Returns MLA_OK; MLA_ERR_NULL for a NULL pointer (host_offsets may be NULL when batch is
 * 0: then the plan is one split); MLA_ERR_SHAPE for batch < 0, q_per_seq < 1,
 * max_splits < 1, a negative offset or a sequence shorter than q_per_seq, or a batch too
 * large to model (over 2^20 workgroups even with one split).
 */
mla_status_t mla_plan_splits(const mla_dims_t* dims, const int64_t* host_offsets, int32_t batch,
                             int32_t q_per_seq, int32_t max_splits, int32_t* num_splits,
                             int32_t* split_rows);

/*
 * mla_merge_splits - combine split results.  Softmax over a disjoint union of
 * row sets: with M = max_s lse_s and w_s = exp(lse_s - M),
 *   o_lat = sum_s w_s o_s / sum_s w_s,   lse = M + ln sum_s w_s.
 * Splits with lse_s = -inf get weight 0 and their o_part values are not used
 * (an empty split's o_part is never written by mla_decode); a query head whose
 * every split is empty gets o_lat = 0 and lse = -inf.
 *
 *   o_part   [num_splits, n_q, n_h, d_c] in partial_dtype (MLA_F32 or MLA_F16)
 *   lse_part [num_splits, n_q, n_h] fp32
 *   o_lat    [n_q, n_h, d_c] fp32 out,          lse      [n_q, n_h] fp32 out
 * o_part and o_lat must be 16-byte aligned when d_c % 8 == 0.
 */
mla_status_t mla_merge_splits(const mla_dims_t* dims, int32_t n_q, int32_t num_splits,
                              int32_t partial_dtype, const void* o_part, const float* lse_part,
                              float* o_lat, float* lse, hipStream_t stream);

/*
 * mla_out_proj - value absorption ([notes] "Value에 대한 수식 전개"): project
 * the weighted latent once per head.
 *
 *   o_c[n, i, d] = sum_c w_uv[i, d, c] * o_lat[n, i, c]
 *
 *   o_lat [n_q, n_h, d_c] fp32   (bf16: rounded to bf16 as the MFMA operand)
 *   w_uv  [n_h, d_h, d_c] dtype  W^UV_i as [d_h, d_c] per head
 *   o_c   [n_q, n_h, d_h] dtype  out
 */
mla_status_t mla_out_proj(const mla_dims_t* dims, int32_t n_q, const float* o_lat,
                          const void* w_uv, void* o_c, hipStream_t stream);

/*
 * mla_merge_out_proj - mla_merge_splits followed by mla_out_proj in one call
 * (the merge as defined above, then [notes] "Value에 대한 수식 전개").  For
 * dtype MLA_BF16 the merged latent never goes to memory: it is rounded to bf16
 * on chip and projected there, and every output equals, bit for bit, what the
 * two separate calls write.  Arguments as for those calls:
 *
 *   o_part, lse_part, partial_dtype, num_splits   as for mla_merge_splits
 *   w_uv  [n_h, d_h, d_c] dtype,  o_c [n_q, n_h, d_h] dtype out
 *   lse   [n_q, n_h] fp32 out, or NULL when not wanted
 *   o_lat [n_q, n_h, d_c] fp32 out, or NULL when not wanted
 * dtype MLA_F32 runs the two fp32 kernels in turn and needs lse and o_lat
 * (both written).  MLA_BF16 needs d_c == 512, d_h == 128, 16-byte aligned
 * o_part, w_uv and o_lat.
 */
mla_status_t mla_merge_out_proj(const mla_dims_t* dims, int32_t n_q, int32_t num_splits,
                                int32_t partial_dtype, const void* o_part, const float* lse_part,
                                const void* w_uv, void* o_c, float* lse, float* o_lat,
                                hipStream_t stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* MLA_KV_H_ */
