// Correlated expert placement search (host code).
//
// Source: "Expert Coupling in MoE Pretraining" (summary), "Method 1: Correlated
// Expert Placement + Deduplicating Dispatcher": a Kernighan-Lin-style local
// search starts from the contiguous placement and swaps experts between ranks
// to raise the co-selection weight of the pairs that share a rank, every rank
// keeping E/R experts.  The page names the search without printing it; this
// library takes the plainest reading: repeatedly apply the swap with the
// largest gain (ties to the lowest expert pair), until no swap gains.
//
// Objective: O = sum over ordered pairs x != y on one rank of W[x][y].
// With S(x, y) = W[x][y] + W[y][x] and A[x][r] = sum of S(x, y) over the
// experts y != x on rank r, swapping e (rank a) with f (rank b) changes O by
//   A[e][b] + A[f][a] - A[e][a] - A[f][b] - 2 S(e, f).
// A is kept up to date in O(E) per swap, so a pass over all pairs is O(E^2).
// Runs on the host: E <= 1024, and the search is sequential by nature.
//
// Also the token-shuffle planner's assignment ("Expert Coupling in MoE
// Pretraining" (summary), "Method 2: Token Shuffling": greedy in decreasing
// confidence under a per-rank capacity): tokens sorted by confidence = largest
// score / sum of scores (ties to the lower token), each to its highest-scoring
// rank with room left of T/R (ties to the lower rank).  Sequential, host.
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

namespace moe {

int placement_search(const int32_t* W, int E, int R, const int32_t* initial, int max_swaps,
                     int32_t* place, int64_t* objective, int* swaps) {
  const int m = E / R;
  for (int e = 0; e < E; ++e) place[e] = initial ? initial[e] : e / m;
  auto S = [&](int x, int y) -> int64_t {
    return int64_t(W[int64_t(x) * E + y]) + int64_t(W[int64_t(y) * E + x]);
  };
  std::vector<int64_t> A(size_t(E) * R, 0);
  for (int x = 0; x < E; ++x)
    for (int y = 0; y < E; ++y)
      if (y != x) A[size_t(x) * R + place[y]] += S(x, y);
  int done = 0;
  while (done < max_swaps) {
    int64_t best = 0;
    int be = -1, bf = -1;
    for (int e = 0; e < E; ++e) {
      const int a = place[e];
      const int64_t* Ae = &A[size_t(e) * R];
      for (int f = e + 1; f < E; ++f) {
        const int b = place[f];
        if (a == b) continue;
        const int64_t* Af = &A[size_t(f) * R];
        const int64_t g = Ae[b] + Af[a] - Ae[a] - Af[b] - 2 * S(e, f);
        if (g > best) {
          best = g;
          be = e;
          bf = f;
        }
      }
    }
    if (be < 0) break;
    const int a = place[be], b = place[bf];
    const int64_t sef = S(be, bf);
    for (int x = 0; x < E; ++x) {
      if (x == be || x == bf) continue;
      const int64_t d = S(x, bf) - S(x, be);
      A[size_t(x) * R + a] += d;
      A[size_t(x) * R + b] -= d;
    }
    A[size_t(be) * R + a] += sef;
    A[size_t(be) * R + b] -= sef;
    A[size_t(bf) * R + b] += sef;
    A[size_t(bf) * R + a] -= sef;
    place[be] = b;
    place[bf] = a;
    ++done;
  }
  if (objective) {
    int64_t o2 = 0;
    for (int x = 0; x < E; ++x) o2 += A[size_t(x) * R + place[x]];
    *objective = o2 / 2;
  }
  if (swaps) *swaps = done;
  return 0;
}

// Host: confidence order, then each token to its best rank with room.
int shuffle_assign(const float* scores, int64_t T, int R, int32_t* owner) {
  std::vector<double> conf(static_cast<size_t>(T));
  for (int64_t t = 0; t < T; ++t) {
    double mx = 0.0, sum = 0.0;
    for (int r = 0; r < R; ++r) {
      const double v = double(scores[t * R + r]);
      sum += v;
      if (v > mx) mx = v;
    }
    conf[size_t(t)] = sum > 0.0 ? mx / sum : 0.0;
  }
  std::vector<int64_t> order(static_cast<size_t>(T));
  for (int64_t t = 0; t < T; ++t) order[size_t(t)] = t;
  std::sort(order.begin(), order.end(), [&](int64_t x, int64_t y) {
    if (conf[size_t(x)] != conf[size_t(y)]) return conf[size_t(x)] > conf[size_t(y)];
    return x < y;
  });
  std::vector<int64_t> room(static_cast<size_t>(R), T / R);
  for (int64_t t : order) {
    const float* s = scores + t * R;
    int best = -1;
    for (int r = 0; r < R; ++r) {
      if (room[size_t(r)] == 0) continue;
      if (best < 0 || s[r] > s[best]) best = r;
    }
    owner[t] = best;
    --room[size_t(best)];
  }
  return 0;
}

}  // namespace moe
