// Split-KV MLA decode over bf16 latent rows on gfx950 MFMA.
//
// Pages cited: [notes] "MLA(Multi-head Latent Attention): DeepSeek-V2 논문정리";
// [report] "Техотчёт DeepSeek-V2 (2024): MLA и экономика инференса".
//
// Every head scores the same latent row [c^KV ; k^R] (576 bf16) with its absorbed
// query and sums the same c^KV (512 bf16) with its softmax weight ([notes]
// "Key에 대한 수식 전개", "Value에 대한 수식 전개"; [report] "Идея 1", "Идея 2").
// So one row read from HBM serves all 128 heads: per row 128 x 576 multiply-adds
// for the scores and 128 x 512 for the weighted sum -- a dense contraction.
//
// One workgroup = one (query token, split of rows, group of 128 heads); 4 waves,
// wave w owns heads [32w, 32w+32) of the group.  Per 32-row tile:
//   * the tile streams HBM -> LDS with 16-byte direct-to-LDS loads, STAGES deep;
//   * S^T[32 rows x 32 heads] = K_tile[32 x 576] . Q^T (36 MFMA 32x32x16), with the
//     wave's queries resident in VGPRs as MFMA B operands;
//   * online softmax in registers: lane l owns head l%32 (16 of the 32 rows; its
//     partner lane l^32 owns the other 16), max/sum exchanged across the pair;
//   * O^T[512 dv x 32 heads] += V_tile^T . P^T (32 MFMA), V^T operands read from
//     the row-major tile with the LDS transpose read, accumulators in AGPRs.
// The softmax works in the log2 domain (scale folded with log2 e) and rescales
// the accumulators only when a head's running maximum grows by more than 8.
#include "mla_common.h"

namespace mla {
namespace {

constexpr int kDc = 512;                 // latent width (values)
constexpr int kDr = 64;                  // RoPE key width
constexpr int kDqk = kDc + kDr;          // 576: key width
constexpr int kTile = 32;                // rows per tile
constexpr int kChunks = kDqk / 8;        // 16-byte chunks per row (72)
constexpr int kRowChunks = kChunks + 1;  // LDS row pitch in chunks: one chunk of padding
constexpr int kRowBytes = kRowChunks * 16;                    // 1168
constexpr int kTileBytes = kTile * kRowBytes;                 // 37376
constexpr int kTileBlocks = (kTile * kRowChunks + 63) / 64;   // 1 KiB direct-to-LDS blocks (37)
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kHeadsPerWg = kWaves * 32;
constexpr int kLoadsPerThread = (kTileBlocks + kWaves - 1) / kWaves;   // 10 (wave 0), else 9
constexpr int kStages = 3;
constexpr int kKSteps = kDqk / 16;       // 36 MFMA k-steps for the scores
constexpr int kDvTiles = kDc / 32;       // 16 output tiles of 32 dv
constexpr float kRescaleSlack = 8.0f;    // log2 units
constexpr int kKAhead = 4;               // K operand reads in flight
constexpr int kVAhead = 3;               // V^T operand reads in flight
constexpr int kWaitVmcnt0 = 0x0F70;      // s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15) (gfx9 encoding)

static_assert(kStages >= 2 && kStages <= 4, "stage count");

struct DecodeParams {
  const bf16_bits* q_abs;       // [n_q, n_h, 576]
  const bf16_bits* c_kv;        // rows, stride c_stride
  const bf16_bits* k_r;         // rows, stride r_stride
  const int64_t* offsets;       // [batch+1]
  float* o_part;                // [S, n_q, n_h, 512]
  float* lse_part;              // [S, n_q, n_h]
  int64_t c_stride, r_stride;
  int n_q, n_h, q_per_seq, num_splits, split_rows;
  int head_groups, group_size, streams;
  float scale_log2;             // softmax scale * log2(e)
};

// LDS layout of a tile: row r at r * 1168 bytes (73 chunks of 16 bytes, the last one
// padding), chunk c of the row at +16c.  The pitch is 292 dwords = 36 banks mod 64,
// so 16 rows read at one chunk column, and 4 rows x 32 bytes of a transpose read,
// land on distinct banks.
__device__ __forceinline__ int chunk_offset(int r, int c) { return r * kRowBytes + c * 16; }

// Issue the direct-to-LDS loads of one tile (packed rows: k^R follows c^KV in a row).
// Block blk covers LDS slots 64*blk .. 64*blk+63; slot p is row p/73, chunk p%73.  Padding
// slots and slots past the tile are masked off.  Rows past `rmax` re-read row `rmax`
// (their scores are masked).  `tile_row` points at the tile's first row.
__device__ __forceinline__ void issue_tile(const char* tile_row, int64_t stride_bytes, int rmax,
                                           char* stage, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < kLoadsPerThread; ++i) {
    const int blk = wave + kWaves * i;
    if (blk < kTileBlocks) {
      const int p = blk * 64 + lane;
      const int r = p / kRowChunks;
      const int c = p - r * kRowChunks;
      if (c < kChunks && r < kTile) {
        const int rr = r < rmax ? r : rmax;
        global_to_lds16(tile_row + rr * stride_bytes + c * 16,
                        __builtin_amdgcn_readfirstlane(lds_addr(stage + blk * 1024)));
      }
    }
  }
}

// V^T operand of O^T step u (u < 16: rows 0-15, else rows 16-31; dv tile u % 16):
// lane l gets rows {0..3, 8..11} + 4(l/32) (+16) of dv column 32(u%16) + l%32.
// `vbase` is the lane's address for u = 0 (row v_row, dv v_dv).
__device__ __forceinline__ bf16x8 load_vt(const char* vbase, int u) {
  const char* p = vbase + (16 * (u / kDvTiles)) * kRowBytes + 64 * (u % kDvTiles);
  const i16x4 lo4 = lds_read_tr16(p);
  const i16x4 hi4 = lds_read_tr16(p + 8 * kRowBytes);
  const i16x8 v8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
  return __builtin_bit_cast(bf16x8, v8);
}

// Wait until this wave's loads of all but the newest `pending` tiles have landed.
template <int kPending>
__device__ __forceinline__ void wait_tile(int wave) {
  if (wave < kTileBlocks - (kLoadsPerThread - 1) * kWaves) wait_vmcnt<kPending * kLoadsPerThread>();
  else wait_vmcnt<kPending * (kLoadsPerThread - 1)>();
}

__global__ void __launch_bounds__(kThreads, 1)
mla_decode_bf16_kernel(DecodeParams P) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  // ---- work item: (row stream, member); members of one stream share its rows
  // and sit on one XCD (workgroups are dealt round-robin over the 8 XCDs).
  const int L = blockIdx.x;
  const int xcd = L & 7;
  const int k = L >> 3;
  const int member = k % P.group_size;
  const int stream = (k / P.group_size) * 8 + xcd;
  if (stream >= P.streams) return;
  const int hg = member % P.head_groups;
  const int r = member / P.head_groups;
  const int b = stream / P.num_splits;
  const int s = stream - b * P.num_splits;
  const int n = b * P.q_per_seq + r;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int head = hg * kHeadsPerWg + wave * 32 + (lane & 31);
  // Waves past the last head (n_h not a multiple of 128) still load tiles and meet the
  // barriers; they read the last head's query and store nothing.
  const bool active = hg * kHeadsPerWg + wave * 32 < P.n_h;   // wave-uniform
  const int head_ld = active ? head : P.n_h - 1;

  const int64_t row0 = P.offsets[b];
  const int64_t len = P.offsets[b + 1] - row0;
  const int64_t vis = len - P.q_per_seq + r + 1;
  int64_t lo, hi;
  if (P.num_splits == 1) {
    lo = 0;
    hi = vis;
  } else {
    lo = (int64_t)s * P.split_rows;
    hi = (s == P.num_splits - 1) ? vis : lo + P.split_rows;
    lo = lo < vis ? lo : vis;
    hi = hi < vis ? hi : vis;
  }
  if (lo < 0) lo = 0;

  const size_t out_row = ((size_t)s * P.n_q + n) * P.n_h;
  if (hi <= lo) {                      // empty split: zero output, lse = -inf
    if (!active) return;
    float* o = P.o_part + (out_row + head) * kDc;
    for (int c = (lane >> 5) * 4; c < kDc; c += 8) *(f32x4*)(o + c) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (lane < 32) P.lse_part[out_row + head] = -INFINITY;
    return;
  }

  const int ntiles = (int)((hi - lo + kTile - 1) / kTile);
  const int64_t stride_bytes = P.c_stride * 2;
  const char* first_row = (const char*)(P.c_kv + (row0 + lo) * P.c_stride);
  const int last_rel = (int)(hi - 1 - lo);        // last valid row, relative to lo

  // ---- prologue: start the first tiles, then fetch this wave's queries
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t)
    if (t < ntiles) {
      const int rmax = last_rel - t * kTile;
      issue_tile(first_row + (int64_t)t * kTile * stride_bytes, stride_bytes,
                 rmax < kTile - 1 ? rmax : kTile - 1, smem + t * kTileBytes, wave, lane);
    }

  bf16x8 qb[kKSteps];
  {
    const bf16_bits* q = P.q_abs + ((size_t)n * P.n_h + head_ld) * kDqk + (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qb[ks] = *(const bf16x8*)(q + ks * 16);
  }
  // All queries (and the prologue tiles) resident.  A builtin wait, so the compiler knows
  // the queries have landed and places no vmcnt waits for them inside the tile loop,
  // where they would also stall on in-flight tile prefetches.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  f32x16 acc[kDvTiles];
#pragma unroll
  for (int t = 0; t < kDvTiles; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
  float m_ref = -INFINITY;           // running reference maximum (log2 units) of head l%32
  float l_run = 0.f;                 // this lane's share of the softmax denominator

  // lane constants of the operand layouts
  const int k_off = chunk_offset(lane & 31, lane >> 5);        // K operand, k-step 0
  const int v_off = chunk_offset(4 * (lane >> 5) + ((lane & 15) >> 2), 2 * ((lane >> 4) & 1)) +
                    8 * (lane & 3);                              // V^T operand, step 0
  const int row_base = 4 * (lane >> 5);        // S^T rows held: 8(i/4) + row_base + i%4

  for (int t = 0; t < ntiles; ++t) {
    // tile t resident in LDS for every wave; the stage of tile t-1 is free
    if (t + 1 < ntiles && kStages > 2) wait_tile<kStages - 2>(wave);
    else wait_tile<0>(wave);
    lds_barrier();
    {
      const int tn = t + kStages - 1;
      if (tn < ntiles) {
        int lane_v = lane;
        asm volatile("" : "+v"(lane_v));   // recompute load offsets per tile instead of holding them
        const int rmax = last_rel - tn * kTile;
        issue_tile(first_row + (int64_t)tn * kTile * stride_bytes, stride_bytes,
                   rmax < kTile - 1 ? rmax : kTile - 1, smem + (tn % kStages) * kTileBytes, wave,
                   lane_v);
      }
    }

    const char* tile = smem + (t % kStages) * kTileBytes;

    // ---- scores S^T = K . Q^T; K operands read kKAhead steps ahead of their MFMA
    const char* kp = tile + k_off;
    f32x16 st;
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = 0.f;
    bf16x8 ka[kKSteps];
#pragma unroll
    for (int ks = 0; ks < kKAhead; ++ks) ka[ks] = *(const bf16x8*)(kp + 32 * ks);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      if (ks + kKAhead < kKSteps) ka[ks + kKAhead] = *(const bf16x8*)(kp + 32 * (ks + kKAhead));
      st = mfma32x32x16(ka[ks], qb[ks], st);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- online softmax (log2 domain)
    const int rem = last_rel - t * kTile;        // rows of this tile with index <= rem count
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 8 * (i >> 2) + row_base + (i & 3);
      st[i] = row <= rem ? st[i] * P.scale_log2 : -INFINITY;
      mt = fmaxf(mt, st[i]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool grow = mt > m_ref + kRescaleSlack;
    if (__any(grow)) {
      const float m_new = grow ? mt : m_ref;
      const float alpha = fast_exp2(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int tt = 0; tt < kDvTiles; ++tt) scale_acc_agpr(acc[tt], alpha);
      m_ref = m_new;
    }
    uint32_t pw[8];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float p0 = fast_exp2(st[i] - m_ref);
      const float p1 = fast_exp2(st[i + 1] - m_ref);
      l_run += p0 + p1;
      pw[i >> 1] = pack_bf16x2(p0, p1);
    }
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const bf16x8 pb0 = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
    const bf16x8 pb1 = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});

    // ---- O^T += V^T . P^T: 2 row k-steps x 16 dv tiles, V^T operands read kVAhead ahead
    const char* vp = tile + v_off;
    bf16x8 va[2 * kDvTiles];
#pragma unroll
    for (int u = 0; u < kVAhead; ++u) va[u] = load_vt(vp, u);
#pragma unroll
    for (int u = 0; u < 2 * kDvTiles; ++u) {
      if (u + kVAhead < 2 * kDvTiles) va[u + kVAhead] = load_vt(vp, u + kVAhead);
      acc[u % kDvTiles] = mfma32x32x16(va[u], u < kDvTiles ? pb0 : pb1, acc[u % kDvTiles]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- finalize: o = acc / l, lse = ln(sum exp)
  if (!active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  float* o = P.o_part + (out_row + head) * kDc;
#pragma unroll
  for (int mt2 = 0; mt2 < kDvTiles; ++mt2)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dv = 32 * mt2 + 8 * g + row_base;
      *(f32x4*)(o + dv) = f32x4{acc[mt2][4 * g] * inv, acc[mt2][4 * g + 1] * inv,
                                acc[mt2][4 * g + 2] * inv, acc[mt2][4 * g + 3] * inv};
    }
  if (lane < 32) P.lse_part[out_row + head] = (m_ref + __log2f(l_tot)) * kLn2;
}

}  // namespace

// Host launcher (arguments already validated).
hipError_t launch_decode_bf16(const bf16_bits* q_abs, const bf16_bits* c_kv, int64_t c_stride,
                              const bf16_bits* k_r, int64_t r_stride, const int64_t* offsets,
                              float* o_part, float* lse_part, int batch, int q_per_seq,
                              int n_h, int num_splits, int split_rows, float scale,
                              hipStream_t stream) {
  DecodeParams P;
  P.q_abs = q_abs;
  P.c_kv = c_kv;
  P.k_r = k_r;
  P.offsets = offsets;
  P.o_part = o_part;
  P.lse_part = lse_part;
  P.c_stride = c_stride;
  P.r_stride = r_stride;
  P.n_q = batch * q_per_seq;
  P.n_h = n_h;
  P.q_per_seq = q_per_seq;
  P.num_splits = num_splits;
  P.split_rows = split_rows;
  P.head_groups = (n_h + kHeadsPerWg - 1) / kHeadsPerWg;
  P.group_size = P.head_groups * q_per_seq;
  P.streams = batch * num_splits;
  P.scale_log2 = (float)((double)scale * 1.4426950408889634);
  const int stream_slots = (P.streams + 7) / 8;
  const long long grid = (long long)stream_slots * 8 * P.group_size;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const size_t smem = (size_t)kStages * kTileBytes;
  // Dynamic LDS above 64 KiB must be allowed once per function (thread-safe static init).
  static const hipError_t attr_err = hipFuncSetAttribute(
      (const void*)mla_decode_bf16_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (attr_err != hipSuccess) return attr_err;
  hipLaunchKernelGGL(mla_decode_bf16_kernel, dim3((unsigned)grid), dim3(kThreads), smem, stream, P);
  return hipGetLastError();
}

}  // namespace mla
