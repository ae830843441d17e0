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
// wave w owns heads [32w, 32w+32) of the group, one wave per SIMD.  Per 32-row tile:
//   * the tile streams HBM -> LDS as 16-byte direct-to-LDS loads into a ring of three
//     stages: the nine loads of tile t+1 leave together right after the barrier that
//     opens tile t.  (A direct-to-LDS load stalls the issuing wave while the memory
//     pipeline is backed up, so the loads go out in one burst with the previous tile's
//     already landed, and only one tile is in flight.)
//   * S^T[32 rows x 32 heads] = K_tile[32 x 576] . Q^T (36 MFMA 32x32x16), with the
//     wave's queries resident in VGPRs as MFMA B operands and the scores accumulated in
//     VGPRs;
//   * online softmax in registers: lane l owns head l%32 (16 of the 32 rows; lane
//     l^32 owns the other 16), max exchanged across the pair;
//   * O^T[512 dv x 32 heads] += V_tile^T . P^T (32 MFMA), V^T operands read from the
//     row-major tile with the LDS transpose read, accumulators in AGPRs.
// The weighted sum of tile t-1 is interleaved with the scores of tile t (one MFMA of
// each in turn), so two tiles are read while the third stage fills.
// The softmax works in the log2 domain (scale folded with log2 e) and rescales the
// accumulators only when a head's running maximum grows by more than 8.
#include "mla_common.h"

namespace mla {
namespace {

constexpr int kDc = 512;                 // latent width (values)
constexpr int kDr = 64;                  // RoPE key width
constexpr int kDqk = kDc + kDr;          // 576: key width
constexpr int kTile = 32;                // rows per tile
constexpr int kChunks = kDqk / 8;        // 16-byte chunks per row (72)
constexpr int kRowBytes = kChunks * 16;  // 1152
constexpr int kTileBytes = kTile * kRowBytes;                 // 36864
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kHeadsPerWg = kWaves * 32;
constexpr int kLoads = kTile * kChunks / kThreads;            // 9 loads of 1 KiB per wave per tile
constexpr int kStages = 3;              // tile ring: scores of t, weighted sum of t-1, loads of t+1
constexpr int kKSteps = kDqk / 16;       // 36 MFMA k-steps for the scores
constexpr int kKReg = kDc / 16;          // 32 k-steps of the latent part (then 4 of the RoPE part)
constexpr int kQStaged = 30;             // latent k-steps of the queries staged through LDS
constexpr int kQChunks = 2 * kQStaged;   // 16-byte chunks per head in the staging area (60)
constexpr int kQStageWave = 32 * kQChunks * 16;               // 30 KiB per wave: 32 heads
constexpr int kQStageLoads = kQStageWave / 1024;              // 30 loads of 1 KiB per wave
constexpr int kDvTiles = kDc / 32;       // 16 output tiles of 32 dv
constexpr float kRescaleSlack = 8.0f;    // log2 units
constexpr int kKAhead = 6;               // K operand reads in flight
constexpr int kVAhead = 6;               // V^T operand reads in flight
constexpr int kOutHalf = kDc / 2;         // dv per epilogue round (256)
constexpr int kWaitVmcnt0 = 0x0F70;      // s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15) (gfx9 encoding)

static_assert(kTile * kChunks == kLoads * kThreads, "tile must split evenly into 1 KiB loads");
static_assert(kKSteps == 4 * kLoads, "one tile load per 4 score steps");
static_assert(kKSteps - kKReg == 4, "RoPE part: 4 k-steps of 16");
static_assert(kTileBytes + kWaves * kQStageWave <= 160 * 1024, "tile 0 and the query staging fit in LDS");

// Issue order of the score k-steps when they are interleaved with the weighted sum: the
// latent steps 0..31 in order (one accumulator chain), the 4 RoPE steps (a second chain)
// placed between the last latent ones, so that no two dependent MFMAs are adjacent.
__host__ __device__ constexpr int s_order(int p) {
  return p <= 28 ? p : (((p - 29) & 1) ? 29 + (p - 30) / 2 : 32 + (p - 29) / 2);
}

// First MFMA of a score chain: the accumulator source is the constant 0, so no zeroed
// registers are needed (the destination must not overlap the operands).
__device__ __forceinline__ void mfma_first_vgpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}

struct DecodeParams {
  const bf16_bits* q_abs;       // [n_q, n_h, 576]
  const bf16_bits* rows;        // packed rows [c_kv | k_r], stride `stride` elements
  const int64_t* offsets;       // [batch+1]
  void* o_part;                 // [S, n_q, n_h, 512] fp32 or fp16
  float* lse_part;              // [S, n_q, n_h]
  int64_t stride;
  int n_q, n_h, q_per_seq, num_splits, split_rows;
  int head_groups, group_size, streams, streams_per_xcd;
  int batch;
  int seqs_per_xcd;             // > 0: sequences dealt to XCDs by length (see the work item)
  float scale_log2;             // softmax scale * log2(e)
};

// LDS layout of a tile: row r at r * 1152 bytes; logical chunk c of the row (16 bytes)
// stored at physical chunk c ^ tile_swz(r), a swap inside the row's aligned groups of 8.
// LDS has 64 banks of 4 bytes; a 16-byte read serves 16 lanes per pass and an 8-byte
// read 32 lanes.  Consecutive rows start 128 bytes apart modulo the 256-byte bank
// space, so rows of equal parity share a bank alignment.  The swap gives:
//  - the K operand (16 rows at one logical chunk per pass) 16 distinct 16-byte slots:
//    among the 8 rows of each parity the swaps are distinct;
//  - the transposing V^T read (rows 4k..4k+3, 4 chunks of one half-group, per pass)
//    distinct slots: rows 4k and 4k+2 (and 4k+1, 4k+3) swap into opposite halves.
// Because LDS slot p of the tile holds a chunk of row p / 72, loading the tile is a
// contiguous copy with a small per-lane swap.
__host__ __device__ constexpr int tile_swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// Per-lane chunk swaps of the 9 loads: load i of lane l fills LDS slot
// p = 64 * (9w + i) + l with global chunk p + delta_i, delta_i in [-7, 7] (4-bit fields).
__device__ __forceinline__ void make_deltas(int wave, int lane, uint32_t& d0, uint32_t& d1) {
  d0 = 0;
  d1 = 0;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int p = 64 * (kLoads * wave + i) + lane;
    const int r = p / kChunks;
    const int pc = p - r * kChunks;
    const int delta = (pc ^ tile_swz(r)) - pc;
    if (i < 8) d0 |= (uint32_t)(delta & 15) << (4 * i);
    else d1 |= (uint32_t)(delta & 15) << (4 * (i - 8));
  }
}

// Load i of one tile: contiguous rows (stride 576), every row inside the cache.
__device__ __forceinline__ void load_fast(const char* tile_src, char* stage, int wave, int i,
                                          uint32_t d0, uint32_t d1, uint32_t lane16) {
  const int blk = kLoads * wave + i;
  const uint32_t bits = i < 8 ? d0 >> (4 * i) : d1 >> (4 * (i - 8));
  const int delta = ((int)(bits << 28)) >> 28;           // sign-extend the 4-bit field
  global_to_lds16_sv(tile_src + blk * 1024, lane16 + (uint32_t)(delta * 16),
                     __builtin_amdgcn_readfirstlane(lds_addr(stage + blk * 1024)));
}

// Load i of one tile, general form: any row stride, rows past `rmax` re-read row `rmax`.
__device__ __forceinline__ void load_clamped(const char* tile_src, int64_t stride_bytes, int rmax,
                                             char* stage, int wave, int i, int lane) {
  const int blk = kLoads * wave + i;
  const int p = 64 * blk + lane;
  const int r = p / kChunks;
  const int pc = p - r * kChunks;
  const int lc = pc ^ tile_swz(r);
  const int rr = r < rmax ? r : rmax;
  global_to_lds16_sv(tile_src, (uint32_t)(rr * stride_bytes + lc * 16),
                     __builtin_amdgcn_readfirstlane(lds_addr(stage + blk * 1024)));
}

// V^T operand for O^T step u (u < 16: rows 0-15, else rows 16-31; dv tile m = u % 16):
// lane l gets rows {0..3, 8..11} + 4(l/32) (+16) of dv column 32m + l%32.  `vb` holds the
// lane's addresses for dv tile pair parity m & 1: [0] rows 0..7, [1] rows 8..15 (their
// swaps differ; rows 16..31 repeat the swaps of rows 0..15).
__device__ __forceinline__ bf16x8 load_vt(const char* tile, const int (*vb)[2], int u) {
  const int m = u % kDvTiles;
  const int off = (16 * (u / kDvTiles)) * kRowBytes + 128 * (m >> 1);
  const i16x4 lo4 = lds_read_tr16(tile + vb[m & 1][0] + off);
  const i16x4 hi4 = lds_read_tr16(tile + vb[m & 1][1] + off);
  const i16x8 v8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
  return __builtin_bit_cast(bf16x8, v8);
}

// Wait until this wave's loads of all but the newest `pending` tiles have landed.
template <int kPending>
__device__ __forceinline__ void wait_tile() {
  wait_vmcnt<kPending * kLoads>();
}

// Epilogue staging: wave w's 32 heads x 256 dv of one round, in LDS at w * stage_bytes,
// one row of 256 outputs (+16 bytes of padding) per head; rows are then stored whole.
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
mla_decode_bf16_kernel(DecodeParams P) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  // ---- work item.  Workgroups are dealt round-robin over the 8 XCDs (workgroup L runs on
  // XCD L % 8), and the members of a stream (query tokens, head groups: same rows) run
  // side by side on one XCD, as do the splits of one sequence (one L2 fetch of its
  // queries).
  //  - Fewer than 8 streams (a long prefill, a few sequences): (stream, member) items are
  //    dealt round-robin over the XCDs, so that all eight work.
  //  - Otherwise, with fewer than 16 sequences: XCD x takes the contiguous stream range
  //    [x * streams_per_xcd, ...).
  //  - seqs_per_xcd > 0 (16 or more sequences): every workgroup ranks the sequences by
  //    length (longest first, ties by index) and XCD x takes ranks x, 15-x, 16+x, 31-x, ...
  //    (snake order), longest first.  Every XCD then gets the same number of sequences
  //    and nearly the same number of tiles, however ragged the lengths.  When every length
  //    is equal the ranks are the indices and the ranking is skipped; otherwise an XCD's
  //    items go longest first.  Only non-empty splits are enumerated (the split-0
  //    workgroup marks the empty ones): the dispatcher deals an XCD's workgroups to its
  //    shader engines in a fixed rotation, so empty workgroups interleaved with real ones
  //    would load the engines unevenly.
  const int L = blockIdx.x;
  const int xcd = L & 7;
  const int k = L >> 3;
  int member = k % P.group_size;
  const int j = k / P.group_size;
  if (P.streams >= 8 && j >= P.streams_per_xcd) return;
  int b, s;
  int used_splits = P.num_splits;                  // splits of sequence b that hold rows
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
      // Longest first: every split of split_rows rows (all but each sequence's last) in
      // rank order, then the last splits, longest first (ties in rank order).  A CU that
      // frees up late then takes a short item.  Lane m of every wave holds this XCD's
      // sequence m; the chosen item's values are read from its lane.
      const int m = (int)(threadIdx.x & 63);
      const int pm = 8 * m + ((m & 1) ? 7 - xcd : xcd);
      const bool valid = m < P.seqs_per_xcd && pm < P.batch;
      const int bm = valid ? by_rank[pm] : 0;
      const int len = valid ? lens[bm] : 0;
      int ns = P.split_rows > 0 ? (len + P.split_rows - 1) / P.split_rows : P.num_splits;
      ns = ns < 1 ? 1 : (ns > P.num_splits ? P.num_splits : ns);
      const int nfull = valid ? ns - 1 : 0;
      const int tail = valid ? len - (ns - 1) * P.split_rows : -1;
      int before = 0, total = 0, rank = 0;      // full splits before sequence m, all of them; rank of m's last
      for (int mm = 0; mm < P.seqs_per_xcd; ++mm) {
        const int f = __builtin_amdgcn_readlane(nfull, mm);
        const int tm = __builtin_amdgcn_readlane(tail, mm);
        before += mm < m ? f : 0;
        total += f;
        rank += (tm > tail || (tm == tail && mm < m)) ? 1 : 0;
      }
      const bool hit = valid && (j < total ? (j >= before && j < before + nfull) : rank == j - total);
      const unsigned long long hits = __ballot(hit);
      if (hits) {                                  // else past this XCD's items
        const int src = __ffsll((long long)hits) - 1;
        b = __builtin_amdgcn_readlane(bm, src);
        used_splits = __builtin_amdgcn_readlane(ns, src);
        s = j < total ? j - __builtin_amdgcn_readlane(before, src) : used_splits - 1;
        row0_l = offs[b];
        len_l = __builtin_amdgcn_readlane(len, src);
      }
    } else {
      // more than 64 sequences per XCD: sequence by sequence in rank order
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
    if (b < 0) return;                             // past this XCD's items (workgroup-uniform)
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
  // Waves past the last head (n_h not a multiple of 128) still load tiles and meet the
  // barriers; they read the last head's query and store nothing.
  const bool active = hg * kHeadsPerWg + wave * 32 < P.n_h;   // wave-uniform

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
  if (s == 0 && used_splits < P.num_splits && active && lane < 32) {   // splits with no workgroup
    for (int se = used_splits; se < P.num_splits; ++se) P.lse_part[((size_t)se * P.n_q + n) * P.n_h + head] = -INFINITY;
  }
  if (hi <= lo) {                      // empty split: lse = -inf marks it; o_part is not written
    if (active && lane < 32) P.lse_part[out_row + head] = -INFINITY;
    return;
  }

  const int ntiles = (int)((hi - lo + kTile - 1) / kTile);
  const int64_t stride_bytes = P.stride * 2;
  const char* first_row = (const char*)(P.rows + (row0 + lo) * P.stride);
  const int last_rel = (int)(hi - 1 - lo);        // last valid row, relative to lo
  const bool contiguous = P.stride == kDqk;
  const bool last_full = ((hi - lo) % kTile) == 0;

  uint32_t d0, d1;
  make_deltas(wave, lane, d0, d1);
  const uint32_t lane16 = (uint32_t)lane * 16;

  // ---- prologue.  Queries: all 36 k-steps (latent and RoPE parts) live in VGPRs as MFMA
  // B operands for the whole split.  Latent k-steps 0..29 come through an LDS staging area
  // by direct-to-LDS loads of contiguous 16-byte chunks (8 cache lines per instruction);
  // k-steps 30-31 and the 4 RoPE steps load straight into their registers in the MFMA
  // layout (32 rows per instruction).  The staging area follows tile stage 0 and takes
  // tile stages 1-2 (no loads before the barrier that opens tile 0) and the LDS beyond the
  // ring.  In it, wave w owns heads 32w .. 32w+31 at kQChunks chunks each, logical chunk c
  // of head h stored at c ^ ((h >> 2) & 3): the 16 heads of a 16-lane read then fall on
  // 16 distinct bank groups.
  bf16x8 qb[kKSteps];
  char* qstage = smem + kTileBytes + wave * kQStageWave;
  const char* qbase = (const char*)(P.q_abs + ((size_t)n * P.n_h + hg * kHeadsPerWg) * kDqk);

  // first tile: its loads go out first (they come from HBM, the queries mostly from L2)
  {
    const char* src = first_row;
    char* stage = smem;
    if (contiguous && (0 < ntiles - 1 || last_full)) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) load_fast(src, stage, wave, i, d0, d1, lane16);
    } else {
      const int rmax = last_rel < kTile - 1 ? last_rel : kTile - 1;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) load_clamped(src, stride_bytes, rmax, stage, wave, i, lane);
    }
  }
  {
    const uint32_t qstage_lds = __builtin_amdgcn_readfirstlane(lds_addr(qstage));
    const int hmax = P.n_h - 1 - hg * kHeadsPerWg;   // last head of the group that exists
#pragma unroll
    for (int j = 0; j < kQStageLoads; ++j) {
      const int g = 64 * j + lane;                 // slot of this lane's chunk
      const int h = g / kQChunks;                  // head of the wave
      const int c = (g - h * kQChunks) ^ ((h >> 2) & 3);
      int hq = wave * 32 + h;
      hq = hq < hmax ? hq : hmax;
      global_to_lds16_sv(qbase, (uint32_t)(hq * kRowBytes + c * 16), qstage_lds + j * 1024);
    }
  }
  // k-steps 30-31 and the RoPE part straight into their B-operand registers (lane l: head
  // l%32, 16 bytes per k-step)
  {
    int hq = wave * 32 + (lane & 31);
    hq = hg * kHeadsPerWg + hq < P.n_h ? hq : P.n_h - 1 - hg * kHeadsPerWg;
    const bf16_bits* qh = (const bf16_bits*)qbase + (size_t)hq * kDqk + 8 * (lane >> 5);
#pragma unroll
    for (int ks = kQStaged; ks < kKSteps; ++ks) qb[ks] = *(const bf16x8*)(qh + 16 * ks);
  }
  const int qh_l = lane & 31;                    // this lane's head in the staging area
  const char* qrd = qstage + qh_l * (kQChunks * 16);
  const int qx = (qh_l >> 2) & 3;                // its chunk swap
  wait_vmcnt<kKSteps - kQStaged>();              // tile 0 and the staged queries landed
#pragma unroll
  for (int ks = 0; ks < kQStaged; ++ks) qb[ks] = *(const bf16x8*)(qrd + 16 * ((2 * ks + (lane >> 5)) ^ qx));
  wait_vmcnt<0>();                               // the directly loaded steps landed
  // All queries (and the first tile) resident.  A builtin wait, so the compiler knows
  // the query loads have landed and places no vmcnt waits for them inside the tile loop,
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
  const int a_row = lane & 31;                 // K operand: tile row of this lane
  int kb[4];                                   // K operand address for k-steps 4q + j
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) kb[jj] = a_row * kRowBytes + 16 * ((2 * jj + (lane >> 5)) ^ tile_swz(a_row));
  const int v_row = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int v_cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  int vb[2][2];
#pragma unroll
  for (int pp = 0; pp < 2; ++pp)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int r = v_row + 8 * hh;
      vb[pp][hh] = r * kRowBytes + 16 * ((4 * pp + v_cl) ^ tile_swz(r)) + 8 * (lane & 1);
    }
  const int row_base = 4 * (lane >> 5);        // S^T rows held: 8(i/4) + row_base + i%4

  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  bf16x8 pb0, pb1;                     // P^T operands of the tile whose weighted sum is next
  // A growing maximum rescales acc just before the next weighted-sum MFMAs rather than in
  // the softmax: rescaling at the end of an iteration makes the compiler copy the whole
  // accumulator around the loop.
  float r_alpha = 1.f;
  bool r_pending = false;              // wave-uniform
  auto apply_rescale = [&]() {
    if (r_pending) {
      asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");   // MFMA results in acc settled
#pragma unroll
      for (int tt = 0; tt < kDvTiles; ++tt) scale_acc_agpr(acc[tt], r_alpha);
      r_pending = false;
    }
  };

  // Top of tile t: every wave's loads of tile t have landed; stage (t+1) % 3 held tile t-2,
  // read for the last time before this barrier, and takes tile t+1's loads now.
  auto open_tile = [&](int t) {
    wait_tile<0>();
    lds_barrier();
    // Hide the load-offset inputs from loop-invariant hoisting: recomputing an offset
    // costs two VALU ops, keeping nine of them live would cost nine VGPRs we do not have.
    uint32_t dd0 = d0, dd1 = d1, ln16 = lane16;
    int lane_v = lane;
    asm volatile("" : "+v"(dd0), "+v"(dd1), "+v"(ln16), "+v"(lane_v));
    const int tn = t + 1;
    if (tn < ntiles) {
      const char* next_src = first_row + (int64_t)tn * kTile * stride_bytes;
      char* next_stage = smem + (tn % kStages) * kTileBytes;
      if (contiguous && (tn < ntiles - 1 || last_full)) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) load_fast(next_src, next_stage, wave, i, dd0, dd1, ln16);
      } else {                                 // any stride or a partial tile
        const int rmax = last_rel - tn * kTile < kTile - 1 ? last_rel - tn * kTile : kTile - 1;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) load_clamped(next_src, stride_bytes, rmax, next_stage, wave, i, lane_v);
      }
    }
  };

  // ---- online softmax of tile t (log2 domain): scores -> pb0, pb1
  auto softmax = [&](int t, f32x16 st) {
    // No contraction: exp2(s - m) must be exactly 1 where s is the maximum, so the scaled
    // score and the maximum must be the same rounded product.
#pragma clang fp contract(off)
    const int rem = last_rel - t * kTile;      // rows of this tile with index <= rem count
    if (rem < kTile - 1) {                     // partial tile: drop the rows past the end
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + row_base + (i & 3);
        if (row > rem) st[i] = -INFINITY;
      }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      st[i] *= P.scale_log2;                   // -inf stays -inf (the scale is positive)
      mt = fmaxf(mt, st[i]);
    }
    mt = pair_max(mt);
    const bool grow = mt > m_ref + kRescaleSlack;
    if (t == 0) {
      m_ref = mt;                      // accumulators and l_run are still zero: nothing to rescale
    } else if (__any(grow)) {
      const float m_new = grow ? mt : m_ref;
      r_alpha = fast_exp2(m_ref - m_new);
      l_run *= r_alpha;
      r_pending = true;
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
    pb0 = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
    pb1 = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});
  };

  // ---- tile 0: scores alone, K operands kKAhead steps ahead, two accumulation chains
  // (even / odd k-steps): a dependent MFMA chain issues at about 60 cycles per step, two
  // interleaved chains at the MFMA rate.  The score accumulators stay in VGPRs
  // (inline-assembly MFMAs) so that the AGPRs hold all of acc.
  open_tile(0);
  {
    f32x16 st, st1;
    bf16x8 ka[kKSteps];
#pragma unroll
    for (int ks = 0; ks < kKAhead; ++ks) ka[ks] = *(const bf16x8*)(smem + kb[ks & 3] + 128 * (ks >> 2));
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      if (ks + kKAhead < kKSteps) {
        const int kn = ks + kKAhead;
        ka[kn] = *(const bf16x8*)(smem + kb[kn & 3] + 128 * (kn >> 2));
      }
      if (ks == 0) mfma_first_vgpr(st, ka[ks], qb[ks]);
      else if (ks == 1) mfma_first_vgpr(st1, ka[ks], qb[ks]);
      else if (ks & 1) mfma_acc_vgpr(st1, ka[ks], qb[ks]);
      else mfma_acc_vgpr(st, ka[ks], qb[ks]);
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_vgpr_drain2(st, st1);
    softmax(0, st + st1);
  }

  // ---- tiles 1..ntiles-1: scores of tile t interleaved with the weighted sum of tile t-1,
  // O^T += V^T . P^T over 2 row k-steps x 16 dv tiles: S step, O step, S step, ...
  for (int t = 1; t < ntiles; ++t) {
    open_tile(t);
    const char* tile = smem + (t % kStages) * kTileBytes;
    const char* otile = smem + ((t + kStages - 1) % kStages) * kTileBytes;
    // Fresh copies of the lane's operand addresses every tile: otherwise the compiler
    // hoists each (address + step offset) out of the loop, one register each.
    int kbl[4], vbl[2][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) kbl[j] = kb[j];
    vbl[0][0] = vb[0][0];
    vbl[0][1] = vb[0][1];
    vbl[1][0] = vb[1][0];
    vbl[1][1] = vb[1][1];
    asm volatile("" : "+v"(kbl[0]), "+v"(kbl[1]), "+v"(kbl[2]), "+v"(kbl[3]), "+v"(vbl[0][0]), "+v"(vbl[0][1]),
                 "+v"(vbl[1][0]), "+v"(vbl[1][1]));
    auto kread = [&](int ks) -> bf16x8 { return *(const bf16x8*)(tile + kbl[ks & 3] + 128 * (ks >> 2)); };
    apply_rescale();
    f32x16 st, st1;
    bf16x8 ka[kKSteps];
    bf16x8 va[2 * kDvTiles];
#pragma unroll
    for (int p = 0; p < kKAhead; ++p) ka[s_order(p)] = kread(s_order(p));
#pragma unroll
    for (int u = 0; u < kVAhead; ++u) va[u] = load_vt(otile, vbl, u);
#pragma unroll
    for (int p = 0; p < kKSteps; ++p) {
      if (p + kKAhead < kKSteps) ka[s_order(p + kKAhead)] = kread(s_order(p + kKAhead));
      const int ks = s_order(p);
      if (ks == 0) mfma_first_vgpr(st, ka[ks], qb[ks]);
      else if (ks == kKReg) mfma_first_vgpr(st1, ka[ks], qb[ks]);
      else if (ks < kKReg) mfma_acc_vgpr(st, ka[ks], qb[ks]);
      else mfma_acc_vgpr(st1, ka[ks], qb[ks]);
      __builtin_amdgcn_sched_barrier(0);
      if (ks < kKReg) {                        // O step u = ks
        const int u = ks;
        if (u + kVAhead < 2 * kDvTiles) va[u + kVAhead] = load_vt(otile, vbl, u + kVAhead);
        acc[u % kDvTiles] = mfma32x32x16(va[u], u < kDvTiles ? pb0 : pb1, acc[u % kDvTiles]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    mfma_vgpr_drain2(st, st1);
    softmax(t, st + st1);
  }

  // ---- the last tile's weighted sum
  {
    apply_rescale();
    const char* otile = smem + ((ntiles - 1) % kStages) * kTileBytes;
    bf16x8 va[2 * kDvTiles];
#pragma unroll
    for (int u = 0; u < kVAhead; ++u) va[u] = load_vt(otile, vb, u);
#pragma unroll
    for (int u = 0; u < 2 * kDvTiles; ++u) {
      if (u + kVAhead < 2 * kDvTiles) va[u + kVAhead] = load_vt(otile, vb, u + kVAhead);
      acc[u % kDvTiles] = mfma32x32x16(va[u], u < kDvTiles ? pb0 : pb1, acc[u % kDvTiles]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- finalize: o = acc / l, lse = ln(sum exp).  The outputs go through LDS in two
  // rounds of 256 dv so that every store writes whole rows (1 KiB per instruction).
  lds_barrier();                                 // every wave is done with the tiles
  // Lane-derived values of the epilogue come from a fresh copy of the lane id: sharing them
  // with the prologue's identical expressions would keep those live (spilled) across the loop.
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
    for (int mt2 = 0; mt2 < kDvTiles / 2; ++mt2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& a = acc[half * (kDvTiles / 2) + mt2];
        const int dv = 32 * mt2 + 8 * g + row_base_e;        // within the round
        put4((OutT*)(ost + (lane_e & 31) * kRowB) + dv, a[4 * g] * inv, a[4 * g + 1] * inv,
             a[4 * g + 2] * inv, a[4 * g + 3] * inv);
      }
    // read back whole rows: a row is kOutHalf * sizeof(OutT) bytes = 64 or 32 lanes x 16 bytes
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

// Host launcher (arguments already validated; rows are packed [c_kv | k_r]).
hipError_t launch_decode_bf16(const bf16_bits* q_abs, const bf16_bits* rows, int64_t stride,
                              const int64_t* offsets, void* o_part, bool f16_partials,
                              float* lse_part, int batch, int q_per_seq, int n_h, int num_splits,
                              int split_rows, float scale, hipStream_t stream) {
  DecodeParams P;
  P.q_abs = q_abs;
  P.rows = rows;
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
  // Sequences are dealt to XCDs by length once there are two per XCD; fewer sequences
  // keep contiguous stream ranges, so that a long sequence's splits spread over XCDs.
  P.seqs_per_xcd = batch >= 16 ? (batch + 7) / 8 : 0;
  P.streams_per_xcd = P.seqs_per_xcd > 0 ? P.seqs_per_xcd * num_splits : (P.streams + 7) / 8;
  P.scale_log2 = (float)((double)scale * 1.4426950408889634);
  size_t smem = (size_t)kTileBytes + (size_t)kWaves * kQStageWave;   // tile 0 and the query staging
  smem = smem > (size_t)kStages * kTileBytes ? smem : (size_t)kStages * kTileBytes;
  const size_t out_stage = (size_t)kWaves * 32 * (f16_partials ? out_row_bytes<_Float16>() : out_row_bytes<float>());
  smem = smem > out_stage ? smem : out_stage;
  if (P.seqs_per_xcd > 0 && (size_t)((batch + 15) & ~15) * (sizeof(int64_t) + 2 * sizeof(int)) > smem) {
    P.seqs_per_xcd = 0;
    P.streams_per_xcd = (P.streams + 7) / 8;
  }
  const long long grid = P.streams < 8 ? (long long)P.streams * P.group_size
                                        : (long long)P.streams_per_xcd * 8 * P.group_size;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // Dynamic LDS above 64 KiB must be allowed once per kernel (thread-safe static init).
  static const hipError_t attr32 = hipFuncSetAttribute(
      (const void*)mla_decode_bf16_kernel<float>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  static const hipError_t attr16 = hipFuncSetAttribute(
      (const void*)mla_decode_bf16_kernel<_Float16>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr32 != hipSuccess) return attr32;
  if (attr16 != hipSuccess) return attr16;
  if (f16_partials)
    hipLaunchKernelGGL(mla_decode_bf16_kernel<_Float16>, dim3((unsigned)grid), dim3(kThreads), smem, stream, P);
  else
    hipLaunchKernelGGL(mla_decode_bf16_kernel<float>, dim3((unsigned)grid), dim3(kThreads), smem, stream, P);
  return hipGetLastError();
}

}  // namespace mla
