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
// Against the bf16 cache this halves the bytes every tile moves: HBM -> LDS, and LDS ->
// registers for both products.
//
// Scores: the codes are MFMA operands as they are (v_mfma_f32_32x32x64_f8f6f4, E4M3 x E4M3).
// Each head's bf16 query is scaled by a power of two 2^e_h that puts its largest magnitude
// in [128, 256) and split into two E4M3 parts, q 2^e_h = hi + lo (lo = the E4M3 rounding of
// the remainder); hi + lo is exact for every component above 2^-10 of the head's largest,
// and two MFMAs (hi, lo) give the score.  The MFMA sums its products with about 13 bits
// below the largest product of each group of 8: with the parts' scaling that is a relative
// error near 1e-4 of the largest product term, a few 1e-5 in the logits here.  2^-e_h and
// s_r multiply the fp32 scores.
// Weighted sum: every E4M3 value is exact in bf16, so the codes widen to bf16 MFMA operands
// without rounding (v_cvt_scalef32_pk_bf16_fp8, scale 1); s_r is folded into p before p's
// one rounding to bf16.
//
// Work item, waves, softmax and epilogue are those of the bf16 decode.  What differs:
//  * the direct-to-LDS tile ring has two stages and the scores and weighted sum of a tile
//    run in sequence (the bf16 decode interleaves them over a third stage);
//  * a 32-row tile is 18 KiB: 18 loads of 1 KiB, five per wave (waves 2 and 3 load four
//    and the tile's 32 row scales, with a 4-byte direct-to-LDS load);
//  * K operands: two 16-byte LDS reads per lane give one 64-code k-step;
//  * V^T operands: the 8-bit transposing LDS read gives a lane 8 rows of its dv column;
//    the P^T operand's rows are regrouped to that order across the wave's two halves.
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
constexpr int kQStageWave = 32 * 1024;   // query staging per wave: 32 heads x 512 latent bf16
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kHeadsPerWg = kWaves * 32;
constexpr int kLoads = 5;                // loads per wave per tile (block or scales)
constexpr int kStages = 2;
constexpr int kKSteps = kDqk / 64;       // 9 k-steps of 64 codes for the scores
constexpr int kDvTiles = kDc / 32;       // 16 output tiles (8 blocks of 64 dv, even and odd)
constexpr float kRescaleSlack = 8.0f;    // log2 units
constexpr int kKAhead = 2;               // K k-steps (two 16-byte reads each) in flight
constexpr int kVAhead = 6;               // V^T reads in flight
constexpr int kOutHalf = kDc / 2;
constexpr int kWaitVmcnt0 = 0x0F70;      // s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15) (gfx9 encoding)

static_assert(kTileBlocks == 4 * kLoads - 2, "waves 0-1 load five blocks, waves 2-3 four and the scales");
static_assert(kStageBytes % 1024 == 0 && kTileBytes + 2 * kScaleArea <= kStageBytes, "stage layout");
static_assert(kStageBytes + kWaves * kQStageWave <= 160 * 1024, "tile 0 and the query staging fit in LDS");

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

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
// start 64 bytes apart modulo the 256-byte bank space, so rows r, r+4, r+8, r+12 share a
// 64-byte quarter.  swz8 maps bit 2 of r to bit 1 of the chunk and bit 3 to bit 0:
//  - a K read (16 rows at one logical chunk per 16-lane pass) hits 16 distinct 16-byte
//    slots (r % 4 picks the quarter, swz8 a distinct slot in it);
//  - an 8-bit transposing V^T read (8 consecutive rows, 2 adjacent chunks each, per
//    32-lane pass) hits distinct banks: rows r and r+4 take opposite chunk pairs.
__host__ __device__ constexpr int swz8(int r) { return (((r >> 2) & 1) << 1) | ((r >> 3) & 1); }

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

// 8 codes -> 8 bf16 (exact: every E4M3 value is a bf16 value).
__device__ __forceinline__ bf16x8 widen8(i32x2 raw) {
  const u32x4 v = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, true)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, true))};
  return __builtin_bit_cast(bf16x8, v);
}

// 8-bit transposing LDS read: in each group of 16 lanes, lane pair (2k, 2k+1) names row k
// (8 bytes each), and lane i receives byte i of rows 0..7.
__device__ __forceinline__ i32x2 read_tr8(const char* p) {
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)((__attribute__((address_space(3))) const char*)p));
}

// acc += A . B, v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3), accumulator in VGPRs: as
// mfma_acc_vgpr, the compiler does not see it (operands come from LDS reads or long-settled
// registers; the chain forwards srcC; mfma8_drain2 before any other read of acc).
__device__ __forceinline__ void mfma8_acc_vgpr(f32x16& acc, const i32x8& a, const i32x8& b) {
  asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// The first MFMA of a chain: two wait states after the VALU writes that zero the accumulator.
__device__ __forceinline__ void mfma8_acc_vgpr_first(f32x16& acc, const i32x8& a, const i32x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// wait states between the 16-pass MFMA's result and a VALU read (more than it needs)
__device__ __forceinline__ void mfma8_drain2(f32x16& acc0, f32x16& acc1) {
  asm volatile("s_nop 15\n\ts_nop 7" : "+v"(acc0), "+v"(acc1));
}

// E4M3 codes of the hi and lo parts of x[0..3] (already scaled into range): hi = E4M3(x),
// lo = E4M3(x - hi), both rounded to nearest even.
__device__ __forceinline__ void split4(float x0, float x1, float x2, float x3, int& hi, int& lo) {
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, h, true);
  const auto b0 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
  const auto b1 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
  int l = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - b0[0], x1 - b0[1], 0, false);
  l = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - b1[0], x3 - b1[1], l, true);
  hi = h;
  lo = l;
}

template <typename OutT>
__host__ __device__ constexpr int out_row_bytes() { return kOutHalf * (int)sizeof(OutT) + 16; }

__device__ __forceinline__ void put4(float* p, float a, float b, float c, float d) {
  *(f32x4*)p = f32x4{a, b, c, d};
}
__device__ __forceinline__ void put4(_Float16* p, float a, float b, float c, float d) {
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  *(f16x4*)p = f16x4{(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
}

template <typename OutT>
__global__ void __launch_bounds__(kThreads, 1)
mla_decode_fp8_kernel(DecodeParams P) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  // ---- work item: as the bf16 decode (round-robin XCDs; fewer than 8 streams: items dealt
  // round-robin; else streams of one sequence on one XCD; with 16 or more sequences,
  // length-ranked snake order and only non-empty splits, the ranks read off at once when
  // every length is equal, an XCD's items longest first when they are not).
  const int L = blockIdx.x;
  const int xcd = L & 7;
  const int k = L >> 3;
  int member = k % P.group_size;
  const int j = k / P.group_size;
  if (P.streams >= 8 && j >= P.streams_per_xcd) return;
  int b, s;
  int used_splits = P.num_splits;
  int64_t row0_l = -1, len_l = 0;                  // from LDS when the ranked mapping read them
  if (P.streams < 8) {
    // fewer streams than XCDs (one long prefill, a few sequences): (stream, member) items
    // dealt round-robin over the XCDs, so that every XCD works
    const int stream = L / P.group_size;
    if (stream >= P.streams) return;
    member = L - stream * P.group_size;
    b = stream / P.num_splits;
    s = stream - b * P.num_splits;
  } else if (P.seqs_per_xcd > 0) {
    // offsets and lengths in LDS (free until the first loads), the lengths padded to a
    // multiple of 16 with -1, which ranks below every length
    const int bpad = (P.batch + 15) & ~15;
    int64_t* offs = (int64_t*)smem;                // [batch]: each sequence's first row, read once
    int* lens = (int*)(offs + bpad);               // [bpad]
    int* by_rank = lens + bpad;                    // [batch]: sequence of each rank
    for (int i = threadIdx.x; i < bpad; i += kThreads) {
      const int64_t o0 = i < P.batch ? P.offsets[i] : 0;
      const int64_t o1 = i < P.batch ? P.offsets[i + 1] : 0;
      lens[i] = i < P.batch ? (int)(o1 - o0) : -1;
      if (i < P.batch) offs[i] = o0;
    }
    __syncthreads();
    // Equal lengths (every wave finds the same): the ranks are the sequence indices.
    const int len0 = lens[0];
    bool uniform = true;
    for (int i0 = 0; i0 < P.batch; i0 += 64) {
      const int i = i0 + (int)(threadIdx.x & 63);
      uniform = uniform && __all(i >= P.batch || lens[i] == len0);
    }
    if (!uniform) {
      for (int c = threadIdx.x; c < P.batch; c += kThreads) {
        const int lc = lens[c];
        int rank = 0;
        typedef int i32x4 __attribute__((ext_vector_type(4)));
        for (int i = 0; i < bpad; i += 16) {       // four reads in flight
          i32x4 v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = *(const i32x4*)(lens + i + 4 * q);
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) rank += (v[q][e] > lc || (v[q][e] == lc && i + 4 * q + e < c)) ? 1 : 0;
        }
        by_rank[rank] = c;                         // the ranks are a permutation of 0..batch-1
      }
      __syncthreads();
    }
    // this XCD's sequences in rank order, each with its non-empty splits: item j
    b = -1;
    s = 0;
    if (uniform) {
      int ns = P.split_rows > 0 ? (len0 + P.split_rows - 1) / P.split_rows : P.num_splits;
      ns = ns < 1 ? 1 : (ns > P.num_splits ? P.num_splits : ns);
      const int m = j / ns;
      const int p = 8 * m + ((m & 1) ? 7 - xcd : xcd);
      if (m < P.seqs_per_xcd && p < P.batch) {
        b = p;
        s = j - m * ns;
        used_splits = ns;
        row0_l = offs[p];
        len_l = len0;
      }
    } else if (P.seqs_per_xcd <= 64) {
      // longest first, as the bf16 decode: the full splits in rank order, then the last
      // splits, longest first; lane m holds this XCD's sequence m
      const int m = (int)(threadIdx.x & 63);
      const int pm = 8 * m + ((m & 1) ? 7 - xcd : xcd);
      const bool valid = m < P.seqs_per_xcd && pm < P.batch;
      const int bm = valid ? by_rank[pm] : 0;
      const int len = valid ? lens[bm] : 0;
      int ns = P.split_rows > 0 ? (len + P.split_rows - 1) / P.split_rows : P.num_splits;
      ns = ns < 1 ? 1 : (ns > P.num_splits ? P.num_splits : ns);
      const int nfull = valid ? ns - 1 : 0;
      const int tail = valid ? len - (ns - 1) * P.split_rows : -1;
      int before = 0, total = 0, rank = 0;
      for (int mm = 0; mm < P.seqs_per_xcd; ++mm) {
        const int f = __builtin_amdgcn_readlane(nfull, mm);
        const int tm = __builtin_amdgcn_readlane(tail, mm);
        before += mm < m ? f : 0;
        total += f;
        rank += (tm > tail || (tm == tail && mm < m)) ? 1 : 0;
      }
      const bool hit = valid && (j < total ? (j >= before && j < before + nfull) : rank == j - total);
      const unsigned long long hits = __ballot(hit);
      if (hits) {
        const int src = __ffsll((long long)hits) - 1;
        b = __builtin_amdgcn_readlane(bm, src);
        used_splits = __builtin_amdgcn_readlane(ns, src);
        s = j < total ? j - __builtin_amdgcn_readlane(before, src) : used_splits - 1;
        row0_l = offs[b];
        len_l = __builtin_amdgcn_readlane(len, src);
      }
    } else {
      int base = 0;
      for (int m = 0; m < P.seqs_per_xcd; ++m) {
        const int p = 8 * m + ((m & 1) ? 7 - xcd : xcd);
        if (p >= P.batch) break;                   // p grows with m
        const int bm = by_rank[p];
        const int len = lens[bm];
        int ns = P.split_rows > 0 ? (len + P.split_rows - 1) / P.split_rows : P.num_splits;
        ns = ns < 1 ? 1 : (ns > P.num_splits ? P.num_splits : ns);
        if (j < base + ns) {
          b = bm;
          s = j - base;
          used_splits = ns;
          row0_l = offs[bm];
          len_l = len;
          break;
        }
        base += ns;
      }
    }
    __syncthreads();                               // every wave has read LDS before it is reused
    if (b < 0) return;
  } else {
    const int stream = xcd * P.streams_per_xcd + j;
    if (stream >= P.streams) return;
    b = stream / P.num_splits;
    s = stream - b * P.num_splits;
  }
  const int hg = member % P.head_groups;
  // a stream's queries latest first: under a causal mask they see the most rows, so the
  // longest items start first
  const int r = P.q_per_seq - 1 - member / P.head_groups;
  const int n = b * P.q_per_seq + r;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int head = hg * kHeadsPerWg + wave * 32 + (lane & 31);
  const bool active = hg * kHeadsPerWg + wave * 32 < P.n_h;   // wave-uniform
  const int head_ld = active ? head : P.n_h - 1;

  const int64_t row0 = row0_l >= 0 ? row0_l : P.offsets[b];
  const int64_t len = row0_l >= 0 ? len_l : P.offsets[b + 1] - row0;
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
  // Queries: lane l's B operand of k-step ks is head l%32's components
  // 64 ks + 32 (l/32) .. +32.  Load them (bf16), find the head's largest magnitude (lanes l
  // and l^32 hold its two halves), scale by 2^e_h (largest in [128, 256)) and split into
  // E4M3 hi and lo parts.
  i32x8 qhi[kKSteps], qlo[kKSteps];
  float q_log2_scale;                          // scale_log2 * 2^-e_h: MFMA sums to log2 units
  {
    // The latent part (k-steps 0..7) comes through an LDS staging area after tile stage 0,
    // by direct-to-LDS loads of one head's contiguous 1 KiB per instruction (wave w: heads
    // 32w .. 32w+31 of the group, chunk c of head h stored at c ^ (h & 15), so the 16 heads
    // of a 16-lane read fall on distinct bank groups); the RoPE k-step loads straight into
    // registers.  Loaded per lane in the operand layout, every instruction touched 32 rows.
    i32x4 raw[kKSteps][4];
    {
      const char* qbase = (const char*)(P.q_abs + ((size_t)n * P.n_h + hg * kHeadsPerWg) * kDqk);
      const int hmax = P.n_h - 1 - hg * kHeadsPerWg;   // last head of the group that exists
      const uint32_t qlds = __builtin_amdgcn_readfirstlane(lds_addr(smem + kStageBytes + wave * kQStageWave));
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int hq = wave * 32 + j < hmax ? wave * 32 + j : hmax;
        global_to_lds16_sv(qbase, (uint32_t)(hq * (kDqk * 2) + ((lane ^ (j & 15)) * 16)), qlds + j * 1024);
      }
    }
    const bf16_bits* qh = P.q_abs + ((size_t)n * P.n_h + head_ld) * kDqk + 32 * (lane >> 5);
#pragma unroll
    for (int u = 0; u < 4; ++u) raw[kKSteps - 1][u] = *(const i32x4*)(qh + 64 * (kKSteps - 1) + 8 * u);
    wait_vmcnt<4>();                           // tile 0 and the staged queries
    {
      const int hl = lane & 31;
      const char* qrd = smem + kStageBytes + wave * kQStageWave + hl * 1024;
#pragma unroll
      for (int ks = 0; ks < kKSteps - 1; ++ks)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          raw[ks][u] = *(const i32x4*)(qrd + 16 * ((8 * ks + 4 * (lane >> 5) + u) ^ (hl & 15)));
    }
    wait_vmcnt<0>();                           // the RoPE k-step
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    uint32_t amax = 0;                         // largest |q| (bf16 magnitudes order as integers)
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = (uint32_t)raw[ks][u][e];
          const uint32_t lo16 = w & 0x7fffu, hi16 = (w >> 16) & 0x7fffu;
          const uint32_t a = lo16 > hi16 ? lo16 : hi16;
          amax = a > amax ? a : amax;
        }
    const float m = pair_max(__uint_as_float(amax << 16));
    // 2^e_h with m * 2^e_h in [128, 256); a zero query keeps scale 1
    const int ex = m > 0.f ? (int)((__float_as_uint(m) >> 23) & 0xff) - 127 : 7;
    const float up = __uint_as_float((uint32_t)(127 + 7 - ex) << 23);
    q_log2_scale = P.scale_log2 * __uint_as_float((uint32_t)(127 - 7 + ex) << 23);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const uint32_t w0 = (uint32_t)raw[ks][u][e], w1 = (uint32_t)raw[ks][u][e + 1];
          int h, l;
          split4(__uint_as_float(w0 << 16) * up, __uint_as_float(w0 & 0xffff0000u) * up,
                 __uint_as_float(w1 << 16) * up, __uint_as_float(w1 & 0xffff0000u) * up, h, l);
          qhi[ks][2 * u + e / 2] = h;
          qlo[ks][2 * u + e / 2] = l;
        }
  }

  f32x16 acc[kDvTiles];
#pragma unroll
  for (int t = 0; t < kDvTiles; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
  float m_ref = -INFINITY;
  float l_run = 0.f;

  // lane constants of the operand layouts
  const int a_row = lane & 31;
  // K operand of k-step ks: row a_row, logical chunks 4 ks + 2 (l/32) + {0, 1}
  const int kb0 = a_row * kRowBytes + 16 * ((2 * (lane >> 5)) ^ swz8(a_row));
  const int kb1 = a_row * kRowBytes + 16 * ((2 * (lane >> 5) + 1) ^ swz8(a_row));
  // V^T operand of dv tile m, rows 16 h .. +16: row 16 h + 8 (l/32) + (l%16)/2, logical
  // chunk 2m + (l/16)%2, byte 8 (l%2); at vb[m & 1] + 64 (m >> 1) + 16 h rows
  const int v_row = 8 * (lane >> 5) + ((lane & 15) >> 1);
  int vb[2];
#pragma unroll
  for (int pp = 0; pp < 2; ++pp)
    vb[pp] = v_row * kRowBytes + 16 * ((2 * pp + ((lane >> 4) & 1)) ^ swz8(v_row)) + 8 * (lane & 1);
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

    // ---- scores S^T = K . Q^T: hi and lo parts in two chains
    f32x16 st, st1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      st[i] = 0.f;
      st1[i] = 0.f;
    }
    i32x8 ka[kKSteps];
#pragma unroll
    for (int ks = 0; ks < kKSteps + kKAhead; ++ks) {
      if (ks < kKSteps) {
        const i32x4 a0 = *(const i32x4*)(tile + kb0 + 64 * ks);
        const i32x4 a1 = *(const i32x4*)(tile + kb1 + 64 * ks);
        ka[ks] = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      }
      const int kc = ks - kKAhead;
      if (kc >= 0) {
        if (kc == 0) {
          mfma8_acc_vgpr_first(st, ka[kc], qhi[kc]);
          mfma8_acc_vgpr_first(st1, ka[kc], qlo[kc]);
        } else {
          mfma8_acc_vgpr(st, ka[kc], qhi[kc]);
          mfma8_acc_vgpr(st1, ka[kc], qlo[kc]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    mfma8_drain2(st, st1);
    st += st1;

    // ---- row scales (wave 2's copy), then the online softmax (log2 domain)
    const char* scl = tile + kTileBytes;
    f32x4 sc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) sc[g] = *(const f32x4*)(scl + 4 * (8 * g + row_base));
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = st[i] * sc[i >> 2][i & 3] * q_log2_scale;
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
    // P^T operand rows in the V^T operand's order: lane l < 32 takes rows 0..7 (its 0-3
    // and lane l+32's 4-7), lane l >= 32 rows 8..15 (lane l-32's 8-11 and its 12-15); the
    // same for rows 16..31.  v_permlane32_swap exchanges the upper half of its first
    // operand with the lower half of its second.
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const auto r = __builtin_amdgcn_permlane32_swap(pw[4 * h + x], pw[4 * h + 2 + x], false, false);
        pw[4 * h + x] = r[0];
        pw[4 * h + 2 + x] = r[1];
      }
    const bf16x8 pb0 = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
    const bf16x8 pb1 = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});

    // ---- O^T += V^T . P^T: 2 row halves x 16 dv tiles, V^T operands kVAhead reads ahead
    i32x2 va[2 * kDvTiles];
#pragma unroll
    for (int u = 0; u < 2 * kDvTiles + kVAhead; ++u) {
      if (u < 2 * kDvTiles) {
        const int m = u % kDvTiles;
        va[u] = read_tr8(tile + vb[m & 1] + 64 * (m >> 1) + (16 * (u / kDvTiles)) * kRowBytes);
      }
      const int uc = u - kVAhead;
      if (uc >= 0) {
        acc[uc % kDvTiles] = mfma32x32x16(widen8(va[uc]), uc < kDvTiles ? pb0 : pb1, acc[uc % kDvTiles]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- finalize: o = acc / l, lse; two rounds of 256 dv through LDS, as the bf16 decode.
  lds_barrier();
  int lane_e = (int)threadIdx.x & 63;
  asm volatile("" : "+v"(lane_e));
  const int row_base_e = 4 * (lane_e >> 5);
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  constexpr int kRowB = out_row_bytes<OutT>();
  char* ost = smem + wave * 32 * kRowB;
  OutT* o = (OutT*)P.o_part + (out_row + hg * kHeadsPerWg + wave * 32) * kDc;
  // lse first: its inputs then die before the output rounds, which need every free VGPR
  // (stored last, they kept one accumulator spilled across the rounds of the fp32 form)
  if (active && lane_e < 32)
    P.lse_part[out_row + hg * kHeadsPerWg + wave * 32 + lane_e] = (m_ref + __log2f(l_tot)) * kLn2;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int mt2 = 0; mt2 < kDvTiles / 2; ++mt2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& a = acc[half * (kDvTiles / 2) + mt2];
        const int dv = 32 * mt2 + 8 * g + row_base_e;
        put4((OutT*)(ost + (lane_e & 31) * kRowB) + dv, a[4 * g] * inv, a[4 * g + 1] * inv,
             a[4 * g + 2] * inv, a[4 * g + 3] * inv);
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
  size_t smem = (size_t)kStageBytes + (size_t)kWaves * kQStageWave;   // tile 0 and the query staging
  smem = smem > (size_t)kStages * kStageBytes ? smem : (size_t)kStages * kStageBytes;
  const size_t out_stage = (size_t)kWaves * 32 * (f16_partials ? out_row_bytes<_Float16>() : out_row_bytes<float>());
  smem = smem > out_stage ? smem : out_stage;
  if (P.seqs_per_xcd > 0 && (size_t)((batch + 15) & ~15) * (sizeof(int64_t) + 2 * sizeof(int)) > smem) {
    P.seqs_per_xcd = 0;
    P.streams_per_xcd = (P.streams + 7) / 8;
  }
  const long long grid = P.streams < 8 ? (long long)P.streams * P.group_size
                                        : (long long)P.streams_per_xcd * 8 * P.group_size;
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
