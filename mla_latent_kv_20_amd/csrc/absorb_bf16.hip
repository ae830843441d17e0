// The two weight-absorption GEMMs of MLA decode, bf16 MFMA on gfx950.
//
// Pages cited: [notes] "MLA(Multi-head Latent Attention): DeepSeek-V2 논문정리";
// [report] "Техотчёт DeepSeek-V2 (2024): MLA и экономика инференса".
//
// absorb_q (key absorption, [notes] "Key에 대한 수식 전개"; [report] "Идея 1"):
//   q_abs[n, i, 0:d_c] = q_c[n, i, :] . W^UK_i        per head: [n_q x d_h] x [d_h x d_c]
//   q_abs[n, i, d_c:]  = q_r[n, i, :]                 ([notes] "Decoupled Rotary ...", item 4)
// out_proj (value absorption, [notes] "Value에 대한 수식 전개"):
//   o_c[n, i, :] = W^UV_i o_lat[n, i, :]              per head: [n_q x d_c] x [d_c x d_h]
//
// Both stream one weight matrix per head (128 x 512 bf16 = 128 KiB) and are bound by that
// weight traffic at decode batch sizes.  Each workgroup keeps its weight slice in MFMA B
// operands and sweeps all query rows over it, so every weight byte is read once.
#include "mla_common.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;

// ---------------------------------------------------------------------------
// absorb_q: workgroup = (head i, block of 128 latent columns); wave w owns 32 columns.
// W^UK rows are [d_h][d_c] with d_c contiguous, but the MFMA B operand needs 8
// consecutive d_h values per lane, so the slice is staged in LDS and read with the
// transposing LDS read.
// ---------------------------------------------------------------------------
constexpr int kAbsCols = 128;
constexpr int kAbsPitch = kAbsCols * 2 + 32;   // 288 B: 4 rows x 32 B of a transpose read hit distinct banks
constexpr int kAbsOutPitch = kAbsCols * 2 + 16; // output staging row (bf16): rows r and r+4 of a 2-byte write on distinct banks

struct AbsorbParams {
  const bf16_bits* q_c;   // [n_q, n_h, d_h]
  const bf16_bits* q_r;   // [n_q, n_h, d_r]
  const bf16_bits* w_uk;  // [n_h, d_h, d_c]
  bf16_bits* q_abs;       // [n_q, n_h, d_c + d_r]
  int n_q, n_h, d_h, d_c, d_r;
  const int64_t* pos;     // [n_q] token positions: rotate q_r there first; null: copy q_r as is
  RopeSpec rope;
};

// kDhT: d_h fixed at compile time (the loops then have no runtime bounds), or 0 for any d_h.
template <int kDhT>
__global__ void __launch_bounds__(kThreads)
absorb_q_bf16_kernel(AbsorbParams P) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int d_h = kDhT > 0 ? kDhT : P.d_h;
  // Workgroups are dealt round-robin over the 8 XCDs: workgroup L runs on XCD L % 8.  All
  // column blocks of head i go to XCD i % 8, so the head's queries are fetched into one
  // L2 once and shared by its blocks.
  const int nblk = P.d_c / kAbsCols;
  const int xcd = blockIdx.x & 7;
  const int kq = blockIdx.x >> 3;
  const int i = (kq / nblk) * 8 + xcd;            // head
  const int cbi = kq % nblk;
  const int cb = cbi * kAbsCols;                  // first latent column of this block
  if (i >= P.n_h) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int d_qk = P.d_c + P.d_r;

  char* ostage = smem + d_h * kAbsPitch;          // [32][kAbsOutPitch] output staging
  const int qpitch = d_h * 2 + 16;                // q_c staging row: 16 rows of a 16-byte read on distinct banks
  char* qstage = ostage + 32 * kAbsOutPitch;      // [32][qpitch] the first query block's q_c rows

  // The weight slice W^UK_i[:, cb:cb+128] goes out first (16-byte chunks, 16 per row), then
  // the first block's q_c rows (16-byte chunks, whole rows): the queries are shared by the
  // four waves, so one copy of them goes through LDS rather than each wave loading its A
  // operands itself (32 rows per instruction).
  const bf16_bits* w = P.w_uk + (size_t)i * d_h * P.d_c + cb;
  const int chunks = d_h * (kAbsCols / 8);        // <= 4096 (d_h <= 256)
  const int ksteps = d_h / 16;                    // <= 16 (d_h <= 256)
  const int qcpr = d_h / 8;                       // 16-byte chunks per q_c row
  const int qchunks = 32 * qcpr;                  // <= 1024
  for (int e0 = 0; e0 < chunks; e0 += 8 * kThreads) {
    bf16x8 v[8];
    // Every load is unconditional (an index past the end re-reads the last chunk, which is
    // not stored): a load under a branch leaves its register undefined on the other path,
    // and the compiler then waits for it in the middle of issuing the rest.
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      int e = e0 + u * kThreads + tid;
      e = e < chunks ? e : chunks - 1;
      v[u] = *(const bf16x8*)(w + (size_t)(e >> 4) * P.d_c + (e & 15) * 8);
    }
    bf16x8 qv[4];
    if (e0 == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        int e = u * kThreads + tid;
        e = e < qchunks ? e : qchunks - 1;
        int m = e / qcpr;
        m = m < P.n_q ? m : P.n_q - 1;
        qv[u] = *(const bf16x8*)(P.q_c + ((size_t)m * P.n_h + i) * d_h + (e % qcpr) * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * kThreads + tid;
      if (e < chunks) *(bf16x8*)(smem + (e >> 4) * kAbsPitch + (e & 15) * 16) = v[u];
    }
    if (e0 == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = u * kThreads + tid;
        const int m = e / qcpr;
        if (e < qchunks) *(bf16x8*)(qstage + m * qpitch + (e % qcpr) * 16) = m < P.n_q ? qv[u] : bf16x8{};
      }
    }
  }
  __syncthreads();

  // A operands of the first query block from the staged rows
  bf16x8 qa[16];
  {
    const char* qrow = qstage + (lane & 31) * qpitch + 16 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < 16; ++s)
      if (s < ksteps) qa[s] = *(const bf16x8*)(qrow + 32 * s);
  }

  // B operands for every k-step: lane l gets W[16s + 8(l/32) + j][32w + l%32], j = 0..7.
  bf16x8 wb[16];
  {
    const int g = lane >> 4;                      // 16-lane group
    const int col = 32 * wave + 16 * (g & 1) + 4 * (lane & 3);
    const int row = 8 * (g >> 1) + ((lane & 15) >> 2);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      if (s < ksteps) {
        const char* p = smem + (16 * s + row) * kAbsPitch + col * 2;
        const i16x4 lo4 = lds_read_tr16(p);
        const i16x4 hi4 = lds_read_tr16(p + 4 * kAbsPitch);
        const i16x8 v8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        wb[s] = __builtin_bit_cast(bf16x8, v8);
      }
    }
  }

  // Sweep the query rows 32 at a time.
  for (int mb = 0; mb < P.n_q; mb += 32) {
    const int m = mb + (lane & 31);
    const bool mrow = m < P.n_q;
    const bf16_bits* q = P.q_c + ((size_t)(mrow ? m : 0) * P.n_h + i) * d_h + 8 * (lane >> 5);
    if (mb > 0) {
#pragma unroll
      for (int s = 0; s < 16; ++s)
        if (s < ksteps) qa[s] = *(const bf16x8*)(q + 16 * s);
    }
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      if (s < ksteps) {
        const bf16x8 a = mrow ? qa[s] : bf16x8{};
        acc = mfma32x32x16(a, wb[s], acc);
      }
    }
    // D[m][n]: lane l, reg r -> row 8(r/4) + 4(l/32) + r%4, column l%32.  The 32 x 128
    // block goes through LDS so that every global store writes 16 contiguous bytes.
    if (mb > 0) __syncthreads();                  // the previous block's stores have read ostage
    const int col = 32 * wave + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      *(bf16_bits*)(ostage + row * kAbsOutPitch + col * 2) = f32_to_bf16(acc[r]);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 32 * (kAbsCols / 8) / kThreads; ++u) {
      const int e = u * kThreads + tid;
      const int row = e / (kAbsCols / 8), c8 = e % (kAbsCols / 8);
      if (mb + row < P.n_q)
        *(bf16x8*)(P.q_abs + ((size_t)(mb + row) * P.n_h + i) * d_qk + cb + 8 * c8) =
            *(const bf16x8*)(ostage + row * kAbsOutPitch + 16 * c8);
    }
  }

  // RoPE part, 16 bytes per thread with every load of a thread in flight before its stores.
  // It comes last, so that its memory latency does not delay the weight loads above.  With
  // token positions the pairs (k, k + d_r/2) are rotated on the way ([notes] "MLA 코드 구현":
  // q^R is rotated head by head at the new tokens' positions), and the head's query rows are
  // shared out over its nblk column blocks (block cbi takes rows cbi, cbi + nblk, ...); so
  // they are for a copy of more than one 16-byte chunk per thread.  A shorter copy is the
  // first block's alone.
  const bool spread = P.pos != nullptr || P.n_q * (P.d_r / 8) > kThreads;
  const int rfirst = spread ? cbi : 0;            // this block's rows: rfirst + rstep * r
  const int rstep = spread ? nblk : 1;
  const int rrows = spread ? (P.n_q > cbi ? (P.n_q - cbi + nblk - 1) / nblk : 0) : (cbi == 0 ? P.n_q : 0);
  if (P.pos == nullptr) {
    const int cpr = P.d_r / 8;                    // 16-byte chunks per query row (d_r % 8 == 0)
    const int total = rrows * cpr;
    for (int e0 = 0; e0 < total; e0 += 4 * kThreads) {
      bf16x8 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * kThreads + tid;
        if (e < total)
          v[u] = *(const bf16x8*)(P.q_r + ((size_t)(rfirst + rstep * (e / cpr)) * P.n_h + i) * P.d_r + (e % cpr) * 8);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * kThreads + tid;
        if (e < total)
          *(bf16x8*)(P.q_abs + ((size_t)(rfirst + rstep * (e / cpr)) * P.n_h + i) * d_qk + P.d_c + (e % cpr) * 8) = v[u];
      }
    }
  } else {
    // thread (k, query slot): one inverse frequency per thread, the block's rows strided
    const int half = P.d_r / 2;
    const int slots = kThreads / half;            // query slots per pair index (d_r <= 512)
    if (tid < half * slots) {
      const int k = tid % half;
      const double inv = rope_inv_freq(k, P.d_r, P.rope);
      for (int rr = tid / half; rr < rrows; rr += slots) {
        const int n = rfirst + rstep * rr;
        const bf16_bits* src = P.q_r + ((size_t)n * P.n_h + i) * P.d_r;
        double x = bf16_to_f32(src[k]);
        double y = bf16_to_f32(src[k + half]);
        rope_rotate(x, y, P.pos[n], inv);
        bf16_bits* dst = P.q_abs + ((size_t)n * P.n_h + i) * d_qk + P.d_c;
        dst[k] = f32_to_bf16((float)x);
        dst[k + half] = f32_to_bf16((float)y);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// absorb_q for many query rows (d_h = 128, d_c = 512, d_r = 64): workgroup = (head i, run
// of query rows), 4 waves, wave w computes latent columns 128w .. 128w+127.  W^UK_i is
// staged in LDS once (as in absorb_q_bf16_kernel, one 128-column slice per wave) and read
// with the transposing LDS read into the wave's B operands (4 column tiles x 8 k-steps,
// 128 VGPRs), which every 32-row block of the run reuses.  Per block, the q_c rows come in
// whole (256 bytes each) through LDS, the next block's rows are in flight during the
// MFMAs, and the whole 1152-byte q_abs rows (latent and RoPE parts) are staged in LDS and
// stored contiguously.  Every output element is the same MFMA chain over the same k-steps
// as in absorb_q_bf16_kernel, with the same RoPE arithmetic, so the two agree bit for bit.
// ---------------------------------------------------------------------------
constexpr int kArDh = 128, kArDc = 512, kArDr = 64;
constexpr int kArSlice = kArDh * kAbsPitch;          // one wave's staged W^UK slice (36 KiB)
constexpr int kArQPitch = kArDh * 2 + 16;            // q_c row in LDS (272 B)
constexpr int kArOPitch = (kArDc + kArDr) * 2 + 16;  // q_abs row in LDS (1168 B)
constexpr int kArQOff = 0;                           // block staging, after the slices are read
constexpr int kArOOff = 32 * kArQPitch;

struct AbsorbRowsParams {
  const bf16_bits* q_c;   // [n_q, n_h, 128]
  const bf16_bits* q_r;   // [n_q, n_h, 64]
  const bf16_bits* w_uk;  // [n_h, 128, 512]
  bf16_bits* q_abs;       // [n_q, n_h, 576]
  int n_q, n_h, chunks, chunk_rows;
  const int64_t* pos;     // [n_q] or null
  RopeSpec rope;
};

__global__ void __launch_bounds__(kThreads)
absorb_q_rows_kernel(AbsorbRowsParams P) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // Workgroup L runs on XCD L % 8; all row runs of head i go to XCD i % 8.
  const int xcd = blockIdx.x & 7;
  const int kc = blockIdx.x >> 3;
  const int i = (kc / P.chunks) * 8 + xcd;
  const int r0 = (kc % P.chunks) * P.chunk_rows;
  const int r1 = P.n_q < r0 + P.chunk_rows ? P.n_q : r0 + P.chunk_rows;
  if (i >= P.n_h || r0 >= r1) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  constexpr int kQk = kArDc + kArDr;

  // the q_c block of rows mb .. mb+31 (16-byte piece t + 256u: row (t + 256u) / 16)
  bf16x8 pf[2];
  auto load_q = [&](int mb) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + kThreads * u;
      const int m = mb + (e >> 4);
      pf[u] = m < r1 ? *(const bf16x8*)(P.q_c + ((size_t)m * P.n_h + i) * kArDh + 8 * (e & 15)) : bf16x8{};
    }
  };
  load_q(r0);

  // W^UK_i: slice w (columns 128w .. 128w+127) at w * kArSlice, rows at kAbsPitch
  {
    const bf16_bits* w = P.w_uk + (size_t)i * kArDh * kArDc;
    for (int e0 = 0; e0 < 4 * kArDh * 16; e0 += 8 * kThreads) {
      bf16x8 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * kThreads + tid;
        const int sl = e >> 11, row = (e >> 4) & 127, c = e & 15;
        v[u] = *(const bf16x8*)(w + (size_t)row * kArDc + 128 * sl + 8 * c);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * kThreads + tid;
        const int sl = e >> 11, row = (e >> 4) & 127, c = e & 15;
        *(bf16x8*)(smem + sl * kArSlice + row * kAbsPitch + c * 16) = v[u];
      }
    }
  }
  __syncthreads();
  // B operands: column tile t of the wave's slice, k-step s: lane l gets
  // W[16s + 8(l/32) + j][128w + 32t + l%32]
  bf16x8 wb[4][8];
  {
    const int g = lane >> 4;
    const int row = 8 * (g >> 1) + ((lane & 15) >> 2);
    const char* slice = smem + wave * kArSlice;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const char* p = slice + (16 * s + row) * kAbsPitch + (32 * t + 16 * (g & 1) + 4 * (lane & 3)) * 2;
        const i16x4 lo4 = lds_read_tr16(p);
        const i16x4 hi4 = lds_read_tr16(p + 4 * kAbsPitch);
        const i16x8 v8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        wb[t][s] = __builtin_bit_cast(bf16x8, v8);
      }
  }
  // RoPE pair indices of this thread: row t / 8 of a block, pairs k = 4 (t % 8) + j
  const int rrow = tid >> 3;
  double inv[4];
  if (P.pos) {
#pragma unroll
    for (int j = 0; j < 4; ++j) inv[j] = rope_inv_freq(4 * (tid & 7) + j, kArDr, P.rope);
  }
  char* qst = smem + kArQOff;
  char* ost = smem + kArOOff;
  __syncthreads();                                 // every wave has read its slice: LDS is free

  for (int mb = r0; mb < r1; mb += 32) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + kThreads * u;
      *(bf16x8*)(qst + (e >> 4) * kArQPitch + 16 * (e & 15)) = pf[u];
    }
    __syncthreads();
    bf16x8 qa[8];
    {
      const char* qr = qst + (lane & 31) * kArQPitch + 16 * (lane >> 5);
#pragma unroll
      for (int s = 0; s < 8; ++s) qa[s] = *(const bf16x8*)(qr + 32 * s);
    }
    if (mb + 32 < r1) load_q(mb + 32);
    // RoPE part of the block's rows: thread t, row t / 8, pairs (k, k + 32), k = 4 (t % 8) + j
    {
      const int m = mb + rrow;
      if (m < r1) {
        const bf16_bits* src = P.q_r + ((size_t)m * P.n_h + i) * kArDr;
        bf16_bits* dst = (bf16_bits*)(ost + rrow * kArOPitch) + kArDc;
        if (P.pos == nullptr) {
          typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
          *(u32x2*)(dst + 8 * (tid & 7)) = *(const u32x2*)(src + 8 * (tid & 7));
          *(u32x2*)(dst + 8 * (tid & 7) + 4) = *(const u32x2*)(src + 8 * (tid & 7) + 4);
        } else {
          const int64_t ps = P.pos[m];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int k = 4 * (tid & 7) + j;
            double x = bf16_to_f32(src[k]);
            double y = bf16_to_f32(src[k + kArDr / 2]);
            rope_rotate(x, y, ps, inv[j]);
            dst[k] = f32_to_bf16((float)x);
            dst[k + kArDr / 2] = f32_to_bf16((float)y);
          }
        }
      }
    }
    // the latent part: four 32 x 32 column tiles
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) acc = mfma32x32x16(qa[s], wb[t][s], acc);
      const int col = 128 * wave + 32 * t + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        *(bf16_bits*)(ost + row * kArOPitch + col * 2) = f32_to_bf16(acc[r]);
      }
    }
    __syncthreads();
    // whole q_abs rows: 72 pieces of 16 bytes per row
    for (int e = tid; e < 32 * 72; e += kThreads) {
      const int row = e / 72, c = e - row * 72;
      if (mb + row < r1)
        *(bf16x8*)(P.q_abs + ((size_t)(mb + row) * P.n_h + i) * kQk + 8 * c) =
            *(const bf16x8*)(ost + row * kArOPitch + 16 * c);
    }
    __syncthreads();                               // qst and ost are free for the next block
  }
}

// ---------------------------------------------------------------------------
// out_proj: workgroup = (head i, block of 32 output columns of d_h); wave w runs a quarter
// of the d_c reduction and the four partial 32 x 32 products are summed through LDS.
// W^UV_i rows are [d_h][d_c] with d_c (the reduction index) contiguous, so B operands load
// straight from global memory into VGPRs; the o_lat rows (fp32) are rounded to bf16 as A
// operands.  Every load of a query block is issued before its first MFMA.
// ---------------------------------------------------------------------------
struct OutProjParams {
  const float* o_lat;     // [n_q, n_h, d_c]
  const bf16_bits* w_uv;  // [n_h, d_h, d_c]
  bf16_bits* o_c;         // [n_q, n_h, d_h]
  int n_q, n_h, d_h, d_c;
};

constexpr int kOutMaxSteps = 8;    // k-steps of 16 per wave: d_c <= 4 * 8 * 16 = 512

// kStepsT: the k-steps per wave (d_c / 64) fixed at compile time, so that every load is
// unconditional and all of them issue before the first wait, or 0 for any d_c.
template <int kStepsT>
__global__ void __launch_bounds__(kThreads)
out_proj_bf16_kernel(OutProjParams P) {
  __shared__ f32x16 red[kWaves][64];
  // Workgroups are dealt round-robin over the 8 XCDs: workgroup L runs on XCD L % 8.  All
  // column blocks of head i go to XCD i % 8, so the head's o_lat rows are fetched into one
  // L2 once and shared by its blocks.
  const int nblk = P.d_h / 32;
  const int xcd = blockIdx.x & 7;
  const int kq = blockIdx.x >> 3;
  const int i = (kq / nblk) * 8 + xcd;
  const int nb = (kq % nblk) * 32;
  if (i >= P.n_h) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int steps = kStepsT > 0 ? kStepsT : P.d_c / 64;   // k-steps of this wave
  const int k0 = wave * steps * 16 + 8 * (lane >> 5);

  // B operands: lane l holds W^UV_i[nb + l%32][k0 + 16s .. +7]
  bf16x8 wb[kOutMaxSteps];
  const bf16_bits* w = P.w_uv + ((size_t)i * P.d_h + nb + (lane & 31)) * P.d_c + k0;
#pragma unroll
  for (int s = 0; s < kOutMaxSteps; ++s)
    if (s < steps) wb[s] = *(const bf16x8*)(w + 16 * s);

  for (int mb = 0; mb < P.n_q; mb += 32) {
    const int m = mb + (lane & 31);
    const float* a = P.o_lat + ((size_t)(m < P.n_q ? m : P.n_q - 1) * P.n_h + i) * P.d_c + k0;
    f32x4 av[kOutMaxSteps][2];
#pragma unroll
    for (int s = 0; s < kOutMaxSteps; ++s) {
      if (s < steps) {
        av[s][0] = *(const f32x4*)(a + 16 * s);
        av[s][1] = *(const f32x4*)(a + 16 * s + 4);
      }
    }
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < kOutMaxSteps; ++s) {
      if (s < steps) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 pk = {pack_bf16x2(av[s][0][0], av[s][0][1]), pack_bf16x2(av[s][0][2], av[s][0][3]),
                          pack_bf16x2(av[s][1][0], av[s][1][1]), pack_bf16x2(av[s][1][2], av[s][1][3])};
        acc = mfma32x32x16(__builtin_bit_cast(bf16x8, pk), wb[s], acc);
      }
    }
    if (mb > 0) __syncthreads();                  // the previous block's sums are read
    red[wave][lane] = acc;
    __syncthreads();
    // wave w sums accumulator registers 4w .. 4w+3 of the four waves.
    // D[m][n]: lane l, reg r -> query mb + 8(r/4) + 4(l/32) + r%4, column nb + l%32
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 4 * wave + q;
      const float v = red[0][lane][r] + red[1][lane][r] + red[2][lane][r] + red[3][lane][r];
      const int mm = mb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (mm < P.n_q) P.o_c[((size_t)mm * P.n_h + i) * P.d_h + nb + (lane & 31)] = f32_to_bf16(v);
    }
  }
}

// ---------------------------------------------------------------------------
// out_proj for many query rows (d_h = 128, d_c = 512): workgroup = (head i, run of query
// rows), 4 waves, wave w computes output columns 32w .. 32w+31 over the whole reduction.
// The wave's B operands (its 32 rows of W^UV_i, 128 VGPRs) are loaded once and reused by
// every 32-row block of the run.  Each block of o_lat rows (fp32, 2 KiB per row of head i)
// is loaded with whole contiguous rows, rounded to bf16 and staged in LDS, where all four
// waves read their A operands.  The reduction runs as the four quarters of 8 MFMA steps of
// out_proj_bf16_kernel, summed in the same order, so the two kernels agree bit for bit.
// ---------------------------------------------------------------------------
constexpr int kRowsDh = 128;
constexpr int kRowsDc = 512;
constexpr int kRowsPitch = kRowsDc * 2 + 16;    // bf16 o_lat row in LDS, padded against conflicts
constexpr int kRowsBlock = 32;

struct OutProjRowsParams {
  const float* o_lat;     // [n_q, n_h, 512]
  const bf16_bits* w_uv;  // [n_h, 128, 512]
  bf16_bits* o_c;         // [n_q, n_h, 128]
  int n_q, n_h, chunks, chunk_rows;
};

__global__ void __launch_bounds__(kThreads)
out_proj_rows_kernel(OutProjRowsParams P) {
  __shared__ __attribute__((aligned(16))) char a_lds[kRowsBlock * kRowsPitch];
  // Workgroup L runs on XCD L % 8; all row runs of head i go to XCD i % 8, so W^UV_i is
  // fetched into one L2.
  const int xcd = blockIdx.x & 7;
  const int kc = blockIdx.x >> 3;
  const int i = (kc / P.chunks) * 8 + xcd;
  const int r0 = (kc % P.chunks) * P.chunk_rows;
  const int r1 = P.n_q < r0 + P.chunk_rows ? P.n_q : r0 + P.chunk_rows;
  if (i >= P.n_h || r0 >= r1) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  // B operands: lane l holds W^UV_i[32w + l%32][16s + 8(l/32) .. +7] for the 32 k-steps s
  bf16x8 wb[kRowsDc / 16];
  {
    const bf16_bits* w = P.w_uv + ((size_t)i * kRowsDh + 32 * wave + (lane & 31)) * kRowsDc + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < kRowsDc / 16; ++s) wb[s] = *(const bf16x8*)(w + 16 * s);
  }

  for (int mb = r0; mb < r1; mb += kRowsBlock) {
    // o_lat rows mb .. mb+31 of head i -> bf16 in LDS: thread t takes 16-byte pieces
    // t + 256u (row = piece / 128, 4 floats each); rows past r1 repeat row r1 - 1
    if (mb > r0) __syncthreads();                 // every wave has read the previous block
    {
      f32x4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int c = tid + kThreads * u;
        const int row = c >> 7;
        const int m = mb + row < r1 ? mb + row : r1 - 1;
        v[u] = *(const f32x4*)(P.o_lat + ((size_t)m * P.n_h + i) * kRowsDc + 4 * (c & 127));
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int c = tid + kThreads * u;
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        *(u32x2*)(a_lds + (c >> 7) * kRowsPitch + 8 * (c & 127)) =
            u32x2{pack_bf16x2(v[u][0], v[u][1]), pack_bf16x2(v[u][2], v[u][3])};
      }
    }
    __syncthreads();
    // A operands: lane l reads row l%32, k = 16s + 8(l/32) .. +7
    const char* arow = a_lds + (lane & 31) * kRowsPitch + 16 * (lane >> 5);
    f32x16 accq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int r = 0; r < 16; ++r) accq[q][r] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        accq[q] = mfma32x32x16(*(const bf16x8*)(arow + 32 * (8 * q + s)), wb[8 * q + s], accq[q]);
    }
    // D[m][n]: lane l, reg r -> row mb + 8(r/4) + 4(l/32) + r%4, column 32w + l%32
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float v = accq[0][r] + accq[1][r] + accq[2][r] + accq[3][r];
      const int mm = mb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (mm < r1) P.o_c[((size_t)mm * P.n_h + i) * kRowsDh + 32 * wave + (lane & 31)] = f32_to_bf16(v);
    }
  }
}

}  // namespace

bool absorb_bf16_supported(int d_h, int d_c) {
  return d_h % 16 == 0 && d_h <= 256 && d_c % kAbsCols == 0;
}
bool out_proj_bf16_supported(int d_h, int d_c) {
  return d_h % 32 == 0 && d_c % 64 == 0 && d_c <= 4 * 16 * kOutMaxSteps;
}

hipError_t launch_absorb_q_bf16(const bf16_bits* q_c, const bf16_bits* q_r, const bf16_bits* w_uk,
                                bf16_bits* q_abs, int n_q, int n_h, int d_h, int d_c, int d_r,
                                const int64_t* positions, const RopeSpec& rope, hipStream_t stream) {
  // Many rows: runs of up to 512 rows (whole 32-row blocks), at least 2 per head.  Measured
  // against the (head, 128 columns) workgroups with 128 heads: without positions from 128
  // rows (15.2 against 15.4 us; 11.4 against 9.9 at 64, 14.6 against 12.8 at 96), with
  // positions from 64 (12.3 against 13.1 us), where the column form's per-head RoPE loop is
  // the slower part.
  const int rows_from = positions ? 64 : 128;
  if (n_q >= rows_from && d_h == kArDh && d_c == kArDc && d_r == kArDr) {
    AbsorbRowsParams R{q_c, q_r, w_uk, q_abs, n_q, n_h, 0, 0, positions, rope};
    R.chunks = (n_q + 511) / 512;
    if (R.chunks < 2) R.chunks = 2;
    R.chunk_rows = ((n_q + R.chunks - 1) / R.chunks + 31) / 32 * 32;
    R.chunks = (n_q + R.chunk_rows - 1) / R.chunk_rows;
    const size_t smem_rows = (size_t)4 * kArSlice;
    static const hipError_t attr = hipFuncSetAttribute((const void*)absorb_q_rows_kernel,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem_rows);
    if (attr != hipSuccess) return attr;
    const long long grid = 8LL * ((n_h + 7) / 8) * R.chunks;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(absorb_q_rows_kernel, dim3((unsigned)grid), dim3(kThreads), smem_rows, stream, R);
    return hipGetLastError();
  }
  AbsorbParams P{q_c, q_r, w_uk, q_abs, n_q, n_h, d_h, d_c, d_r, positions, rope};
  const size_t smem = (size_t)d_h * kAbsPitch + 32 * kAbsOutPitch + (size_t)32 * (d_h * 2 + 16);
  static const hipError_t attr = hipFuncSetAttribute((const void*)absorb_q_bf16_kernel<0>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)(256 * kAbsPitch + 32 * kAbsOutPitch + 32 * (256 * 2 + 16)));
  if (attr != hipSuccess) return attr;
  static const hipError_t attr128 = hipFuncSetAttribute((const void*)absorb_q_bf16_kernel<128>,
                                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                                        (int)(128 * kAbsPitch + 32 * kAbsOutPitch + 32 * (128 * 2 + 16)));
  if (attr128 != hipSuccess) return attr128;
  const int grid = 8 * ((n_h + 7) / 8) * (d_c / kAbsCols);
  if (d_h == 128)
    hipLaunchKernelGGL(absorb_q_bf16_kernel<128>, dim3(grid), dim3(kThreads), smem, stream, P);
  else
    hipLaunchKernelGGL(absorb_q_bf16_kernel<0>, dim3(grid), dim3(kThreads), smem, stream, P);
  return hipGetLastError();
}

hipError_t launch_out_proj_bf16(const float* o_lat, const bf16_bits* w_uv, bf16_bits* o_c, int n_q,
                                int n_h, int d_h, int d_c, hipStream_t stream) {
  if (n_q >= 128 && d_h == kRowsDh && d_c == kRowsDc) {
    // many rows: runs of 128 rows (whole 32-row blocks), at most 64 per head
    OutProjRowsParams R{o_lat, w_uv, o_c, n_q, n_h, 0, 0};
    R.chunks = (n_q + 127) / 128;
    if (R.chunks > 64) R.chunks = 64;
    R.chunk_rows = ((n_q + R.chunks - 1) / R.chunks + kRowsBlock - 1) / kRowsBlock * kRowsBlock;
    R.chunks = (n_q + R.chunk_rows - 1) / R.chunk_rows;
    const long long grid = 8LL * ((n_h + 7) / 8) * R.chunks;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(out_proj_rows_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, R);
    return hipGetLastError();
  }
  OutProjParams P{o_lat, w_uv, o_c, n_q, n_h, d_h, d_c};
  const int grid = 8 * ((n_h + 7) / 8) * (d_h / 32);
  if (d_c == 64 * kOutMaxSteps)
    hipLaunchKernelGGL(out_proj_bf16_kernel<kOutMaxSteps>, dim3(grid), dim3(kThreads), 0, stream, P);
  else
    hipLaunchKernelGGL(out_proj_bf16_kernel<0>, dim3(grid), dim3(kThreads), 0, stream, P);
  return hipGetLastError();
}

}  // namespace mla
