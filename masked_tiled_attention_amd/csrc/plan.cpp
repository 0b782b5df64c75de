// Chunk -> rank assignment for context parallelism (host code).
//
// "FlashMask-3" page (iitog.ru), contributions paragraph and "Key facts": the
// distributed extension has a sparsity-aware load balancer (HCC-IPO); the
// pages give its name only. The algorithm here is this library's own: with
// C chunks of the global query axis, each with a known amount of work (open
// pairs, from chunk_work_kernel), give every one of R ranks exactly C / R
// chunks so that the largest rank load is as small as we can find:
//   - two chunks per rank: pair the largest with the smallest, the second
//     largest with the second smallest, and so on (optimal for pairs: an
//     exchange argument shows any crossing pair can be uncrossed without
//     raising the maximum);
//   - otherwise: longest first, each chunk to the least loaded rank that
//     still has room, then exchanges of one chunk between the most loaded
//     rank and another while that lowers the larger of the two loads.
// The snake order (round k of R chunks assigned left to right for even k and
// right to left for odd k; with two chunks per rank this is the dual-chunk
// assignment) is improved by the same exchanges, and the plan with the
// smaller maximum wins (the snake one on ties), so the result is never worse
// than dual-chunk. Deterministic.
#include <algorithm>
#include <cstdint>
#include <numeric>
#include <vector>

#include "fm_internal.hpp"

namespace fm {
namespace {

int64_t max_load(const std::vector<int64_t>& w, const std::vector<int32_t>& rank, int R,
                 std::vector<int64_t>* loads_out = nullptr) {
  std::vector<int64_t> loads(R, 0);
  for (size_t c = 0; c < w.size(); ++c) loads[rank[c]] += w[c];
  if (loads_out) *loads_out = loads;
  return *std::max_element(loads.begin(), loads.end());
}

// Exchanges of one chunk between the most loaded rank and another while that
// lowers the larger of the two loads (each accepted exchange lowers the
// maximum or the number of ranks at the maximum, so it ends).
void improve(const std::vector<int64_t>& w, std::vector<int32_t>& rank, int R) {
  const int C = (int)w.size();
  std::vector<int64_t> loads;
  for (int iter = 0; iter < 64 * C * C; ++iter) {
    max_load(w, rank, R, &loads);
    const int top = (int)(std::max_element(loads.begin(), loads.end()) - loads.begin());
    int best_x = -1, best_y = -1;
    int64_t best = loads[top];
    for (int x = 0; x < C; ++x) {
      if (rank[x] != top) continue;
      for (int y = 0; y < C; ++y) {
        if (rank[y] == top) continue;
        const int64_t d = w[x] - w[y];
        if (d <= 0) continue;
        const int64_t m = std::max(loads[top] - d, loads[rank[y]] + d);
        if (m < best) {
          best = m;
          best_x = x;
          best_y = y;
        }
      }
    }
    if (best_x < 0) return;
    std::swap(rank[best_x], rank[best_y]);
  }
}

}  // namespace

int64_t plan_chunks(const int64_t* work, int C, int R, int32_t* rank_of_chunk) {
  const int per = C / R;
  std::vector<int64_t> w(work, work + C);
  std::vector<int> idx(C);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return w[a] > w[b]; });

  // snake (dual-chunk for two per rank), then exchanges
  std::vector<int32_t> snake(C);
  for (int c = 0; c < C; ++c) {
    const int k = c / R, p = c % R;
    snake[c] = (k % 2 == 0) ? p : R - 1 - p;
  }
  improve(w, snake, R);

  // sorted pairing or longest-first with capacities, then exchanges
  std::vector<int32_t> greedy(C);
  if (per == 2) {
    for (int r = 0; r < R; ++r) {
      greedy[idx[r]] = r;
      greedy[idx[C - 1 - r]] = r;
    }
  } else {
    std::vector<int64_t> loads(R, 0);
    std::vector<int> count(R, 0);
    for (int c : idx) {
      int best = -1;
      for (int r = 0; r < R; ++r)
        if (count[r] < per && (best < 0 || loads[r] < loads[best])) best = r;
      greedy[c] = best;
      loads[best] += w[c];
      ++count[best];
    }
  }
  improve(w, greedy, R);

  const int64_t ms = max_load(w, snake, R), mg = max_load(w, greedy, R);
  const std::vector<int32_t>& pick = mg < ms ? greedy : snake;
  std::copy(pick.begin(), pick.end(), rank_of_chunk);
  return std::min(ms, mg);
}

}  // namespace fm
