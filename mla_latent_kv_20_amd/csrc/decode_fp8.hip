// Split-KV MLA decode over a quantized latent cache (FP8 E4M3 codes, one scale per row)
// on gfx950 MFMA.
//
// Pages cited: [notes] "MLA(Multi-head Latent Attention): DeepSeek-V2 논문정리";
// [report] "Техотчёт DeepSeek-V2 (2024): MLA и экономика инференса" (the served cache is
// quantized, economics section); [review] "DeepSeek-V2 review", section 4.
//
// The same attention as the bf16 decode (every head scores the latent row [c^KV ; k^R] with
// its absorbed query and sums c^KV with its softmax weight), over dequantized rows
// x^_r = value(code_r) * s_r.  A row's scale factors out of both products:
//   score_{r,h} = s_r * (q_h . value(code_r)),    o_h += p_{r,h} * s_r * value(code_r)[0:512]
// Every E4M3 value is exact in bf16, so the codes widen to bf16 MFMA operands without
// rounding (v_cvt_scalef32_pk_bf16_fp8 with scale 1); s_r multiplies the fp32 scores and is
// folded into p before p's one rounding to bf16.  Against the bf16 cache this halves the
// bytes every tile moves: HBM -> LDS, and LDS -> registers for both products.
//
// Work item, waves, two-stage direct-to-LDS tile ring, softmax and epilogue are those of
// the bf16 decode.  What differs:
//  * a 32-row tile is 18 KiB: 18 loads of 1 KiB, five per wave (waves 2 and 3 load four
//    and the tile's 32 row scales, with a 4-byte direct-to-LDS load);
//  * K operands: one 16-byte LDS read per lane gives two k-steps (16 codes of one row);
//    the queries' B operands follow the same k order;
//  * V^T operands: the 16-bit transposing LDS read over pairs of codes gives a lane four
//    rows of two adjacent dv columns; the even and odd columns form two operands (byte
//    permutes), so the output tiles hold even and odd dv columns of a 64-wide block.
#include "mla_common.h"

namespace mla {
namespace {

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kDqk = kDc + kDr;          // 576 codes per row
constexpr int kTile = 32;
constexpr int kChunks = kDqk / 16;       // 36 chunks of 16 codes
constexpr int kRowBytes = kDqk;          // 576
constexpr int kTileBytes = kTile * kRowBytes;                 // 18432
constexpr int kTileBlocks = kTileBytes / 1024;                // 18 loads of 1 KiB
constexpr int kScaleArea = 256;          // a 4-byte direct-to-LDS load fills 64 x 4 bytes
constexpr int kStageBytes = kTileBytes + 1024;                // tile, two scale areas, padding
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kHeadsPerWg = kWaves * 32;
constexpr int kLoads = 5;                // loads per wave per tile (block or scales)
constexpr int kStages = 2;
constexpr int kPairs = kDqk / 32;        // 18 LDS reads of 16 codes = 36 k-steps of 16
constexpr int kKSteps = 2 * kPairs;
constexpr int kDvTiles = kDc / 32;       // 16 output tiles (8 blocks of 64 dv, even and odd)
constexpr float kRescaleSlack = 8.0f;    // log2 units
constexpr int kKAhead = 3;               // K reads (of two k-steps each) in flight
constexpr int kVAhead = 3;               // V^T read pairs in flight
constexpr int kOutHalf = kDc / 2;
constexpr int kWaitVmcnt0 = 0x0F70;      // s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15) (gfx9 encoding)

static_assert(kTileBlocks == 4 * kLoads - 2, "waves 0-1 load five blocks, waves 2-3 four and the scales");
static_assert(kStageBytes % 1024 == 0 && kTileBytes + 2 * kScaleArea <= kStageBytes, "stage layout");

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct DecodeParams {
  const bf16_bits* q_abs;       // [n_q, n_h, 576] bf16
  const uint8_t* codes;         // code rows, `stride` bytes each
  const float* scales;          // one per code row
  const int64_t* offsets;       // [batch+1]
  void* o_part;                 // [S, n_q, n_h, 512] fp32 or fp16
  float* lse_part;              // [S, n_q, n_h]
  int64_t stride;               // bytes
  int n_q, n_h, q_per_seq, num_splits, split_rows;
  int head_groups, group_size, streams, streams_per_xcd;
  int batch;
  int seqs_per_xcd;
  float scale_log2;
};

// LDS layout of a tile: row r at r * 576 bytes; logical chunk c (16 codes) stored at
// physical chunk c ^ swz8(r), a swap inside the row's aligned groups of 4 chunks.  Rows
// start 64 bytes apart modulo the 256-byte bank space.  With swz8(r) = (r >> 2) & 3:
//  - a K read (16 rows at one logical chunk per 16-lane pass) hits 16 distinct 16-byte
//    slots: r % 4 picks the 64-byte quarter, swz8 the slot inside it;
//  - a transposing V^T read (4 consecutive rows, 64 bytes each, per 32-lane pass) hits
//    4 distinct quarters.
__host__ __device__ constexpr int swz8(int r) { return (r >> 2) & 3; }

// Per-lane chunk swaps of this wave's tile blocks: block i of wave w is tile block
// w + 4i; lane l fills LDS slot p = 64 (w + 4i) + l with global chunk p + delta_i,
// delta_i in [-3, 3] (4-bit fields).
__device__ __forceinline__ uint32_t make_deltas(int wave, int lane) {
  uint32_t d = 0;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int blk = wave + 4 * i;
    if (blk < kTileBlocks) {
      const int p = 64 * blk + lane;
      const int r = p / kChunks;
      const int pc = p - r * kChunks;
      d |= (uint32_t)(((pc ^ swz8(r)) - pc) & 15) << (4 * i);
    }
  }
  return d;
}

// 4-byte direct-to-LDS load: lane l's 4 bytes land at lds_base + 4*l.
__device__ __forceinline__ void global_to_lds4_sv(const void* sbase, uint32_t voff, uint32_t lds_base) {
  uint32_t saved_m0;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved_m0)
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory");
}

// One tile's loads by this wave: its code blocks, and for waves 2 and 3 the scales of
// rows row0 .. row0+63 (clamped to `rmax`; only the first 32 are used, wave 3's copy is
// not read).  `rmax` (tile-relative, < 32) also clamps the code rows unless the tile is
// full and the rows are contiguous (`fast`).
__device__ __forceinline__ void load_tile(const uint8_t* codes0, int64_t stride, const float* scales0,
                                          int tile_row0, int rmax, bool fast, char* stage, int wave,
                                          int lane, uint32_t deltas) {
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int blk = wave + 4 * i;
    if (blk < kTileBlocks) {
      uint32_t off;
      if (fast) {
        const int delta = ((int)((deltas >> (4 * i)) << 28)) >> 28;
        off = (uint32_t)(blk * 1024 + lane * 16 + delta * 16);
      } else {
        const int p = 64 * blk + lane;
        const int r = p / kChunks;
        const int pc = p - r * kChunks;
        const int rr = r < rmax ? r : rmax;
        off = (uint32_t)(rr * stride + (pc ^ swz8(r)) * 16);
      }
      global_to_lds16_sv(codes0 + (int64_t)tile_row0 * stride, off,
                         __builtin_amdgcn_readfirstlane(lds_addr(stage + blk * 1024)));
    } else {
      const int rr = lane < rmax ? lane : rmax;
      global_to_lds4_sv(scales0 + tile_row0, (uint32_t)(rr * 4),
                        __builtin_amdgcn_readfirstlane(lds_addr(stage + kTileBytes + (wave - 2) * kScaleArea)));
    }
  }
}

template <int kPending>
__device__ __forceinline__ void wait_tile() {
  wait_vmcnt<kPending * kLoads>();
}

// Two bf16 k-steps from 16 codes (one 16-byte LDS read): bytes 0-7 and 8-15.
__device__ __forceinline__ void widen16(u32x4 raw, bf16x8& x, bf16x8& y) {
  const u32x4 lo = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, true)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, true))};
  const u32x4 hi = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[2], 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[2], 1.0f, true)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[3], 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[3], 1.0f, true))};
  x = __builtin_bit_cast(bf16x8, lo);
  y = __builtin_bit_cast(bf16x8, hi);
}

// Even and odd V^T operands from two transposing reads: a = rows 0-3, b = rows 8-11 (of
// this lane's row set), each 4 x (even code, odd code).
__device__ __forceinline__ void widen_vt(u32x2 a, u32x2 b, bf16x8& ev, bf16x8& od) {
  const uint32_t ae = __builtin_amdgcn_perm(a[1], a[0], 0x06040200u);
  const uint32_t ao = __builtin_amdgcn_perm(a[1], a[0], 0x07050301u);
  const uint32_t be = __builtin_amdgcn_perm(b[1], b[0], 0x06040200u);
  const uint32_t bo = __builtin_amdgcn_perm(b[1], b[0], 0x07050301u);
  const u32x4 e = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ae, 1.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ae, 1.0f, true)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(be, 1.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(be, 1.0f, true))};
  const u32x4 o = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ao, 1.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ao, 1.0f, true)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(bo, 1.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(bo, 1.0f, true))};
  ev = __builtin_bit_cast(bf16x8, e);
  od = __builtin_bit_cast(bf16x8, o);
}

__device__ __forceinline__ u32x2 read_tr(const char* p) {
  return __builtin_bit_cast(u32x2, lds_read_tr16(p));
}

// acc += A . B with the accumulator in VGPRs (as mfma_acc_vgpr), preceded by two wait
// states: the operands come straight from VALU conversions, which the compiler cannot
// order against an MFMA it does not see.
__device__ __forceinline__ void mfma_acc_vgpr_after_valu(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

template <typename OutT>
__host__ __device__ constexpr int out_row_bytes() { return kOutHalf * (int)sizeof(OutT) + 16; }

__device__ __forceinline__ void put8(float* p, const float (&v)[8]) {
  *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
  *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}
__device__ __forceinline__ void put8(_Float16* p, const float (&v)[8]) {
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  *(f16x8*)p = f16x8{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3],
                     (_Float16)v[4], (_Float16)v[5], (_Float16)v[6], (_Float16)v[7]};
}

template <typename OutT>
__global__ void __launch_bounds__(kThreads, 1)
mla_decode_fp8_kernel(DecodeParams P) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  // ---- work item: as the bf16 decode (round-robin XCDs; streams of one sequence on one
  // XCD; with 16 or more sequences, length-ranked snake order and only non-empty splits).
  const int L = blockIdx.x;
  const int xcd = L & 7;
  const int k = L >> 3;
  const int member = k % P.group_size;
  const int j = k / P.group_size;
  if (j >= P.streams_per_xcd) return;
  int b, s;
  int used_splits = P.num_splits;
  if (P.seqs_per_xcd > 0) {
    const int bpad = (P.batch + 3) & ~3;
    int* lens = (int*)smem;
    int* by_rank = lens + bpad;
    for (int i = threadIdx.x; i < bpad; i += kThreads)
      lens[i] = i < P.batch ? (int)(P.offsets[i + 1] - P.offsets[i]) : -1;
    __syncthreads();
    for (int c = threadIdx.x; c < P.batch; c += kThreads) {
      const int lc = lens[c];
      int rank = 0;
      for (int i = 0; i < bpad; i += 4) {
        typedef int i32x4 __attribute__((ext_vector_type(4)));
        const i32x4 v = *(const i32x4*)(lens + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) rank += (v[e] > lc || (v[e] == lc && i + e < c)) ? 1 : 0;
      }
      by_rank[rank] = c;
    }
    __syncthreads();
    int base = 0;
    b = -1;
    s = 0;
    for (int m = 0; m < P.seqs_per_xcd; ++m) {
      const int p = 8 * m + ((m & 1) ? 7 - xcd : xcd);
      if (p >= P.batch) break;
      const int bm = by_rank[p];
      const int len = lens[bm];
      int ns = P.split_rows > 0 ? (len + P.split_rows - 1) / P.split_rows : P.num_splits;
      ns = ns < 1 ? 1 : (ns > P.num_splits ? P.num_splits : ns);
      if (j < base + ns) {
        b = bm;
        s = j - base;
        used_splits = ns;
        break;
      }
      base += ns;
    }
    __syncthreads();
    if (b < 0) return;
  } else {
    const int stream = xcd * P.streams_per_xcd + j;
    if (stream >= P.streams) return;
    b = stream / P.num_splits;
    s = stream - b * P.num_splits;
  }
  const int hg = member % P.head_groups;
  const int r = member / P.head_groups;
  const int n = b * P.q_per_seq + r;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int head = hg * kHeadsPerWg + wave * 32 + (lane & 31);
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
  if (s == 0 && used_splits < P.num_splits && active && lane < 32) {
    for (int se = used_splits; se < P.num_splits; ++se) P.lse_part[((size_t)se * P.n_q + n) * P.n_h + head] = -INFINITY;
  }
  if (hi <= lo) {
    if (active && lane < 32) P.lse_part[out_row + head] = -INFINITY;
    return;
  }

  const int ntiles = (int)((hi - lo + kTile - 1) / kTile);
  const uint8_t* codes0 = P.codes + (row0 + lo) * P.stride;
  const float* scales0 = P.scales + (row0 + lo);
  const int last_rel = (int)(hi - 1 - lo);
  const bool contiguous = P.stride == kRowBytes;
  const bool last_full = ((hi - lo) % kTile) == 0;
  const uint32_t deltas = make_deltas(wave, lane);

  // ---- prologue: tile 0's loads, then the queries straight into their B-operand
  // registers.  k-step 2p + x of lane l covers row codes 32p + 16(l/32) + 8x .. +8, the
  // order in which one 16-byte read of a K row gives two k-steps.
  {
    const int rmax = last_rel < kTile - 1 ? last_rel : kTile - 1;
    load_tile(codes0, P.stride, scales0, 0, rmax, contiguous && (0 < ntiles - 1 || last_full), smem, wave,
              lane, deltas);
  }
  bf16x8 qb[kKSteps];
  {
    const bf16_bits* qh = P.q_abs + ((size_t)n * P.n_h + head_ld) * kDqk + 16 * (lane >> 5);
#pragma unroll
    for (int p = 0; p < kPairs; ++p) {
      qb[2 * p] = *(const bf16x8*)(qh + 32 * p);
      qb[2 * p + 1] = *(const bf16x8*)(qh + 32 * p + 8);
    }
  }
  wait_vmcnt<0>();
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  f32x16 acc[kDvTiles];
#pragma unroll
  for (int t = 0; t < kDvTiles; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
  float m_ref = -INFINITY;
  float l_run = 0.f;

  // lane constants of the operand layouts
  const int a_row = lane & 31;
  int kb[2];                                   // K read of pair p at kb[p & 1] + 64 (p >> 1)
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) kb[jj] = a_row * kRowBytes + 16 * ((2 * jj + (lane >> 5)) ^ swz8(a_row));
  // V^T reads: rows v_row (+8 for the second read) of the row half, 8 bytes at chunk
  // v_cl of each 64-dv block (+ 64 per block), byte 8 (l & 1)
  const int v_row = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int v_cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int vbA = v_row * kRowBytes + 16 * (v_cl ^ swz8(v_row)) + 8 * (lane & 1);
  const int vbB = (v_row + 8) * kRowBytes + 16 * (v_cl ^ swz8(v_row + 8)) + 8 * (lane & 1);
  const int row_base = 4 * (lane >> 5);        // S^T rows held: 8(i/4) + row_base + i%4

  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) wait_tile<kStages - 2>();
    else wait_tile<0>();
    lds_barrier();

    uint32_t dd = deltas;
    int lane_v = lane;
    asm volatile("" : "+v"(dd), "+v"(lane_v));

    const char* tile = smem + (t % kStages) * kStageBytes;
    const int tn = t + kStages - 1;
    if (tn < ntiles) {
      const int rem_n = last_rel - tn * kTile;
      const int rmax = rem_n < kTile - 1 ? rem_n : kTile - 1;
      load_tile(codes0, P.stride, scales0, tn * kTile, rmax, contiguous && (tn < ntiles - 1 || last_full),
                smem + (tn % kStages) * kStageBytes, wave, lane_v, dd);
    }

    // ---- scores S^T = K . Q^T, two chains (even / odd k-steps)
    f32x16 st, st1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      st[i] = 0.f;
      st1[i] = 0.f;
    }
    u32x4 kr[kPairs];
#pragma unroll
    for (int p = 0; p < kKAhead; ++p) kr[p] = *(const u32x4*)(tile + kb[p & 1] + 64 * (p >> 1));
#pragma unroll
    for (int p = 0; p < kPairs; ++p) {
      if (p + kKAhead < kPairs) {
        const int pn = p + kKAhead;
        kr[pn] = *(const u32x4*)(tile + kb[pn & 1] + 64 * (pn >> 1));
      }
      bf16x8 kx, ky;
      widen16(kr[p], kx, ky);
      mfma_acc_vgpr_after_valu(st, kx, qb[2 * p]);
      mfma_acc_vgpr_after_valu(st1, ky, qb[2 * p + 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_vgpr_drain2(st, st1);
    st += st1;

    // ---- row scales (wave 2's copy), then the online softmax (log2 domain)
    const char* scl = tile + kTileBytes;
    f32x4 sc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) sc[g] = *(const f32x4*)(scl + 4 * (8 * g + row_base));
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = st[i] * sc[i >> 2][i & 3] * P.scale_log2;
    const int rem = last_rel - t * kTile;
    if (rem < kTile - 1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + row_base + (i & 3);
        if (row > rem) st[i] = -INFINITY;
      }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mt = fmaxf(mt, st[i]);
    mt = pair_max(mt);
    const bool grow = mt > m_ref + kRescaleSlack;
    if (t == 0) {
      m_ref = mt;
    } else if (__any(grow)) {
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
      pw[i >> 1] = pack_bf16x2(p0 * sc[i >> 2][i & 3], p1 * sc[i >> 2][(i & 3) + 1]);
    }
    const bf16x8 pb0 = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
    const bf16x8 pb1 = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});

    // ---- O^T += V^T . P^T: row halves h x 64-dv blocks g, two tiles (even, odd dv) each
    u32x2 va[2 * 8][2];
#pragma unroll
    for (int u = 0; u < kVAhead; ++u) {
      const int off = (16 * (u >> 3)) * kRowBytes + 64 * (u & 7);
      va[u][0] = read_tr(tile + vbA + off);
      va[u][1] = read_tr(tile + vbB + off);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (u + kVAhead < 16) {
        const int un = u + kVAhead;
        const int off = (16 * (un >> 3)) * kRowBytes + 64 * (un & 7);
        va[un][0] = read_tr(tile + vbA + off);
        va[un][1] = read_tr(tile + vbB + off);
      }
      bf16x8 ev, od;
      widen_vt(va[u][0], va[u][1], ev, od);
      const bf16x8 pb = u < 8 ? pb0 : pb1;
      acc[2 * (u & 7)] = mfma32x32x16(ev, pb, acc[2 * (u & 7)]);
      acc[2 * (u & 7) + 1] = mfma32x32x16(od, pb, acc[2 * (u & 7) + 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- finalize: o = acc / l, lse.  Tile 2g + x holds dv 64g + 2m + x at M row m
  // (m = 8(i/4) + 4(l/32) + i%4 for register i): even and odd interleave into 8
  // consecutive dv per register group.  Two rounds of 256 dv through LDS, as the bf16 decode.
  lds_barrier();
  int lane_e = (int)threadIdx.x & 63;
  asm volatile("" : "+v"(lane_e));
  const int row_base_e = 4 * (lane_e >> 5);
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  constexpr int kRowB = out_row_bytes<OutT>();
  char* ost = smem + wave * 32 * kRowB;
  OutT* o = (OutT*)P.o_part + (out_row + hg * kHeadsPerWg + wave * 32) * kDc;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int g = 4 * half + g4;
        const f32x16& ae = acc[2 * g];
        const f32x16& ao = acc[2 * g + 1];
        const float v[8] = {ae[4 * gg] * inv,     ao[4 * gg] * inv,     ae[4 * gg + 1] * inv, ao[4 * gg + 1] * inv,
                            ae[4 * gg + 2] * inv, ao[4 * gg + 2] * inv, ae[4 * gg + 3] * inv, ao[4 * gg + 3] * inv};
        const int dv = 64 * g4 + 2 * (8 * gg + row_base_e);      // within the round
        put8((OutT*)(ost + (lane_e & 31) * kRowB) + dv, v);
      }
    constexpr int kLanesPerRow = kOutHalf * (int)sizeof(OutT) / 16;
    constexpr int kRowsPerStore = 64 / kLanesPerRow;
    const int rr = lane_e / kLanesPerRow;
    const int cc = lane_e % kLanesPerRow;
#pragma unroll
    for (int h0 = 0; h0 < 32; h0 += kRowsPerStore) {
      const int h = h0 + rr;
      const f32x4 v = *(const f32x4*)(ost + h * kRowB + cc * 16);
      if (active) *(f32x4*)((char*)(o + (size_t)h * kDc + half * kOutHalf) + cc * 16) = v;
    }
  }
  if (active && lane_e < 32)
    P.lse_part[out_row + hg * kHeadsPerWg + wave * 32 + lane_e] = (m_ref + __log2f(l_tot)) * kLn2;
}

}  // namespace

// Host launcher (arguments already validated): code rows of `stride` bytes.
hipError_t launch_decode_fp8(const bf16_bits* q_abs, const uint8_t* codes, int64_t stride, const float* scales,
                             const int64_t* offsets, void* o_part, bool f16_partials, float* lse_part, int batch,
                             int q_per_seq, int n_h, int num_splits, int split_rows, float scale,
                             hipStream_t stream) {
  DecodeParams P;
  P.q_abs = q_abs;
  P.codes = codes;
  P.scales = scales;
  P.offsets = offsets;
  P.o_part = o_part;
  P.lse_part = lse_part;
  P.stride = stride;
  P.n_q = batch * q_per_seq;
  P.n_h = n_h;
  P.q_per_seq = q_per_seq;
  P.num_splits = num_splits;
  P.split_rows = split_rows;
  P.head_groups = (n_h + kHeadsPerWg - 1) / kHeadsPerWg;
  P.group_size = P.head_groups * q_per_seq;
  P.streams = batch * num_splits;
  P.batch = batch;
  P.seqs_per_xcd = batch >= 16 ? (batch + 7) / 8 : 0;
  P.streams_per_xcd = P.seqs_per_xcd > 0 ? P.seqs_per_xcd * num_splits : (P.streams + 7) / 8;
  P.scale_log2 = (float)((double)scale * 1.4426950408889634);
  size_t smem = (size_t)kStages * kStageBytes;
  const size_t out_stage = (size_t)kWaves * 32 * (f16_partials ? out_row_bytes<_Float16>() : out_row_bytes<float>());
  smem = smem > out_stage ? smem : out_stage;
  if (P.seqs_per_xcd > 0 && (size_t)(2 * (batch + 3)) * sizeof(int) > smem) {
    P.seqs_per_xcd = 0;
    P.streams_per_xcd = (P.streams + 7) / 8;
  }
  const long long grid = (long long)P.streams_per_xcd * 8 * P.group_size;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  static const hipError_t attr32 = hipFuncSetAttribute(
      (const void*)mla_decode_fp8_kernel<float>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  static const hipError_t attr16 = hipFuncSetAttribute(
      (const void*)mla_decode_fp8_kernel<_Float16>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr32 != hipSuccess) return attr32;
  if (attr16 != hipSuccess) return attr16;
  if (f16_partials)
    hipLaunchKernelGGL(mla_decode_fp8_kernel<_Float16>, dim3((unsigned)grid), dim3(kThreads), smem, stream, P);
  else
    hipLaunchKernelGGL(mla_decode_fp8_kernel<float>, dim3((unsigned)grid), dim3(kThreads), smem, stream, P);
  return hipGetLastError();
}

}  // namespace mla
