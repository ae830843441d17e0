// Split planner for mla_decode: picks num_splits and split_rows for a batch of sequence
// lengths by simulating how the decode deals its work items to the GPU.
//
// Split-KV decoding splits each sequence's rows so that one query's attention spreads over
// several workgroups; the splits are merged afterwards by their log-sum-exp ([notes]
// "MLA(Multi-head Latent Attention): DeepSeek-V2 논문정리", "Key에 대한 수식 전개": the
// softmax is over all of a query's visible rows, so any partition of them merges exactly).
// Which partition is fastest depends on the lengths: too few splits leave CUs idle, too many
// pay every workgroup's fixed start and write more split results to merge.
//
// The model mirrors the decode kernel's work-item mapping (the same dealing of workgroups to
// the 8 XCDs, the same orders within an XCD) and the hardware's dispatch: every CU of an XCD
// takes the XCD's next workgroup when it frees up.  A workgroup costs a fixed start plus a
// time per 32-row tile; the merge costs the split results' bytes, written and read back, at
// the streaming rate.  The constants were measured on MI355X (fixed start about 10 us, a tile
// about 2.05 us at the decode's sustained clock, about 5 TB/s); only the plans' order
// matters, not the absolute times.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <functional>
#include <queue>
#include <vector>

#include "../../include/mla_kv.h"

namespace mla {
namespace {

constexpr int kXcds = 8;
constexpr int kCusPerXcd = 32;
constexpr int kTileRows = 32;
constexpr int kHeadsPerWg = 128;
constexpr double kFixedUs = 10.0;        // a workgroup's start: work item, queries, epilogue
constexpr double kTileUs = 2.05;         // one 32-row tile
constexpr double kEmptyUs = 1.0;         // a workgroup whose split holds no row
constexpr double kBytesPerUs = 5.0e6;    // split results written and read back
constexpr int64_t kMaxWorkgroups = 1 << 20;

struct Batch {
  std::vector<int64_t> len;  // rows of each sequence
  int q_per_seq, head_groups, n_h, d_h, d_c;
  int64_t max_len;
  bool uniform;
  std::vector<int> by_rank;  // sequences longest first, ties by index
};

// Rows of split s of query r (0 = oldest) of a sequence of len rows, as mla_decode splits them.
int64_t split_rows_of(const Batch& B, int64_t len, int r, int S, int R, int s) {
  const int64_t vis = len - B.q_per_seq + r + 1;
  if (S == 1) return vis > 0 ? vis : 0;
  int64_t lo = (int64_t)s * R;
  int64_t hi = s == S - 1 ? vis : lo + R;
  lo = std::min(lo, vis);
  hi = std::min(hi, vis);
  return hi > lo ? hi - lo : 0;
}

// Cost of one workgroup: (sequence b, split s, member) with members query-major, latest
// query first, as the decode enumerates them.
double wg_cost(const Batch& B, int b, int S, int R, int s, int member) {
  const int r = B.q_per_seq - 1 - member / B.head_groups;
  const int64_t rows = split_rows_of(B, B.len[b], r, S, R, s);
  return rows > 0 ? kFixedUs + kTileUs * (double)((rows + kTileRows - 1) / kTileRows) : kEmptyUs;
}

// Makespan of one XCD taking its workgroups in order on kCusPerXcd CUs.
double xcd_makespan(const std::vector<double>& costs) {
  std::priority_queue<double, std::vector<double>, std::greater<double>> cu;
  for (int i = 0; i < kCusPerXcd; ++i) cu.push(0.0);
  double end = 0.0;
  for (double c : costs) {
    const double t = cu.top() + c;
    cu.pop();
    cu.push(t);
    end = std::max(end, t);
  }
  return end;
}

// Modeled time of the decode and the merge of its split results for plan (S, R); negative
// when the plan has too many workgroups to simulate.
double plan_cost(const Batch& B, int S, int R) {
  const int batch = (int)B.len.size();
  const int gs = B.head_groups * B.q_per_seq;
  const int64_t streams = (int64_t)batch * S;
  if (streams * gs > kMaxWorkgroups) return -1.0;
  std::vector<std::vector<double>> per_xcd(kXcds);
  auto ns_of = [&](int64_t len) {
    int ns = R > 0 ? (int)((len + R - 1) / R) : S;
    return std::max(1, std::min(S, ns));
  };
  if (streams < kXcds) {
    for (int64_t L = 0; L < streams * gs; ++L) {
      const int64_t stream = L / gs;
      per_xcd[L % kXcds].push_back(wg_cost(B, (int)(stream / S), S, R, (int)(stream % S), (int)(L % gs)));
    }
  } else if (batch < 16) {
    const int64_t spx = (streams + kXcds - 1) / kXcds;
    for (int x = 0; x < kXcds; ++x)
      for (int64_t j = 0; j < spx && x * spx + j < streams; ++j) {
        const int64_t stream = x * spx + j;
        for (int mb = 0; mb < gs; ++mb)
          per_xcd[x].push_back(wg_cost(B, (int)(stream / S), S, R, (int)(stream % S), mb));
      }
  } else {
    const int spx = (batch + kXcds - 1) / kXcds;
    for (int x = 0; x < kXcds; ++x) {
      std::vector<std::pair<int, int>> items;   // (sequence, split)
      std::vector<std::pair<int64_t, int>> tails;
      for (int m = 0; m < spx; ++m) {
        const int p = 8 * m + ((m & 1) ? 7 - x : x);
        if (p >= batch) break;
        const int b = B.uniform ? p : B.by_rank[p];
        const int ns = ns_of(B.len[b]);
        const bool longest_first = !B.uniform && spx <= 64;
        for (int s = 0; s < ns - (longest_first ? 1 : 0); ++s) items.push_back({b, s});
        if (longest_first) tails.push_back({B.len[b] - (int64_t)(ns - 1) * R, b});
      }
      // the last splits, longest first, ties in the order they were met
      std::stable_sort(tails.begin(), tails.end(),
                       [](const std::pair<int64_t, int>& a, const std::pair<int64_t, int>& c) { return a.first > c.first; });
      for (const auto& t : tails) items.push_back({t.second, ns_of(B.len[t.second]) - 1});
      for (const auto& it : items)
        for (int mb = 0; mb < gs; ++mb) per_xcd[x].push_back(wg_cost(B, it.first, S, R, it.second, mb));
    }
  }
  double decode = 0.0;
  for (const auto& c : per_xcd) decode = std::max(decode, xcd_makespan(c));
  // What the decode leaves behind: with one split, fp32 o_lat rows, written and read back by
  // the projection.  With several, fp16 split results and an lse per (query, head, non-empty
  // split), written and read back by the fused merge and projection, which also reads W^UV_i
  // again for every block of 16 queries.
  const int64_t n_q = (int64_t)batch * B.q_per_seq;
  double bytes = 0.0;
  if (S == 1) {
    bytes = 2.0 * (double)n_q * B.n_h * (B.d_c * 4 + 4);
  } else {
    const double row16 = (double)B.n_h * (B.d_c * 2 + 4);
    for (int b = 0; b < batch; ++b)
      for (int r = 0; r < B.q_per_seq; ++r)
        for (int s = 0; s < S; ++s)
          if (split_rows_of(B, B.len[b], r, S, R, s) > 0) bytes += 2.0 * row16;
    bytes += (double)((n_q + 15) / 16) * B.n_h * B.d_h * B.d_c * 2;
  }
  return decode + bytes / kBytesPerUs;
}

}  // namespace
}  // namespace mla

extern "C" mla_status_t mla_plan_splits(const mla_dims_t* dims, const int64_t* host_offsets, int32_t batch,
                                        int32_t q_per_seq, int32_t max_splits, int32_t* num_splits,
                                        int32_t* split_rows) {
  if (!dims || !num_splits || !split_rows) return MLA_ERR_NULL;
  if (batch < 0 || q_per_seq < 1 || max_splits < 1 || dims->n_h < 1 || dims->d_h < 1 || dims->d_c < 1)
    return MLA_ERR_SHAPE;
  *num_splits = 1;
  *split_rows = 0;
  if (batch == 0) return MLA_OK;
  if (!host_offsets) return MLA_ERR_NULL;
  mla::Batch B;
  B.q_per_seq = q_per_seq;
  B.n_h = dims->n_h;
  B.d_h = dims->d_h;
  B.d_c = dims->d_c;
  B.head_groups = (dims->n_h + mla::kHeadsPerWg - 1) / mla::kHeadsPerWg;
  B.len.resize(batch);
  B.max_len = 0;
  for (int b = 0; b < batch; ++b) {
    const int64_t len = host_offsets[b + 1] - host_offsets[b];
    if (host_offsets[b] < 0 || len < q_per_seq) return MLA_ERR_SHAPE;
    B.len[b] = len;
    B.max_len = std::max(B.max_len, len);
  }
  B.uniform = std::all_of(B.len.begin(), B.len.end(), [&](int64_t l) { return l == B.len[0]; });
  B.by_rank.resize(batch);
  for (int b = 0; b < batch; ++b) B.by_rank[b] = b;
  std::stable_sort(B.by_rank.begin(), B.by_rank.end(), [&](int a, int c) { return B.len[a] > B.len[c]; });

  // candidates: one split, and split_rows in whole tiles, at most about 256 of them
  const int64_t tiles = (B.max_len + mla::kTileRows - 1) / mla::kTileRows;
  const int64_t step = std::max<int64_t>(1, (tiles + 255) / 256);
  double best = mla::plan_cost(B, 1, 0);
  int best_s = 1, best_r = 0;
  for (int64_t t = step; t < tiles; t += step) {
    if (t * mla::kTileRows > INT32_MAX) break;
    const int R = (int)(t * mla::kTileRows);
    const int64_t need = (B.max_len + R - 1) / R;
    const int S = (int)std::min<int64_t>(max_splits, need);
    if (S < 2) continue;
    const double c = mla::plan_cost(B, S, R);
    if (c >= 0.0 && (best < 0.0 || c < best)) {
      best = c;
      best_s = S;
      best_r = R;
    }
  }
  if (best < 0.0) return MLA_ERR_SHAPE;     // too many workgroups even for one split
  *num_splits = best_s;
  *split_rows = best_r;
  return MLA_OK;
}
