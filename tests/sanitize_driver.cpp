// Host-only driver run under AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_sanitizers.py: exercises every oracle entry point and the
// library's host planners (placement search, token-shuffle assignment) on
// small and edge-case shapes, and checks the planners against the oracle.  Exits 0
// when the sanitizers report nothing (they abort otherwise).
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <random>
#include <vector>

extern "C" {
int oracle_route_topk(const float*, int64_t, int, int, int32_t*, float*);
int oracle_route_topk_softmax_all(const float*, int64_t, int, int, int32_t*, float*);
int oracle_send_counts(const int32_t*, int64_t, int, int, int, const int32_t*, int, int32_t*,
                       int32_t*, int32_t*, int32_t*);
int oracle_dispatch(const uint8_t*, const int32_t*, const float*, int64_t, int, int, int,
                    const int32_t*, uint8_t*, int32_t*, int32_t*, float*, int32_t*);
int oracle_dispatch_dedup(const uint8_t*, const int32_t*, const float*, int64_t, int, int, int,
                          int, const int32_t*, const int32_t*, uint8_t*, int32_t*, int32_t*,
                          float*, float*, int32_t*, int32_t*);
int oracle_expand_dedup(const uint8_t*, const int32_t*, const float*, int64_t, int64_t, int, int,
                        int, int, const int32_t*, int32_t*, int32_t*, int32_t*, int32_t*,
                        uint8_t*, int32_t*, int32_t*, float*, int32_t*);
int oracle_combine(const uint16_t*, const float*, const int32_t*, int64_t, int, int, uint16_t*);
int oracle_combine_fp8(const uint8_t*, const float*, const int32_t*, int64_t, int, int,
                       uint16_t*);
int oracle_coselect(const int32_t*, int64_t, int, int, int32_t*);
int oracle_placement_search(const int32_t*, int, int, const int32_t*, int, int32_t*, int64_t*,
                            int*);
int oracle_shuffle_fit(const int32_t*, const int32_t*, const int32_t*, int64_t, int, int, int,
                       const int32_t*, int32_t*, int32_t*);
int oracle_shuffle_predict(const int32_t*, const int32_t*, int64_t, int, int, int,
                           const int32_t*, const int32_t*, int, float*);
int oracle_shuffle_assign(const float*, int64_t, int, int32_t*);
}
namespace moe {
int placement_search(const int32_t*, int, int, const int32_t*, int, int32_t*, int64_t*, int*);
int shuffle_assign(const float*, int64_t, int, int32_t*);
}

static int run(int T, int E, int k, int R, int H, unsigned seed) {
  std::mt19937 g(seed);
  std::normal_distribution<float> nd;
  const int N = T * k;
  std::vector<float> logits(size_t(T) * E);
  for (auto& v : logits) v = nd(g);
  std::vector<int32_t> idx(N), place(E);
  std::vector<float> gate(N);
  for (int e = 0; e < E; ++e) place[e] = e / (E / R);
  if (oracle_route_topk(logits.data(), T, E, k, idx.data(), gate.data())) return 1;
  if (oracle_route_topk_softmax_all(logits.data(), T, E, k, idx.data(), gate.data())) return 1;
  std::vector<int32_t> ec(E), rc(R), ro(R + 1), eo(E);
  for (int dedup = 0; dedup < 2; ++dedup)
    if (oracle_send_counts(idx.data(), T, E, k, R, place.data(), dedup, ec.data(), rc.data(),
                           ro.data(), eo.data()))
      return 1;
  std::vector<uint16_t> x(size_t(T) * H);
  for (auto& v : x) v = uint16_t(g() & 0x3FFF);
  std::vector<uint16_t> send(size_t(N) * H), out(size_t(T) * H);
  std::vector<int32_t> rt(N), re(N), sr(N), rx(size_t(N) * k), nr(1);
  std::vector<float> rw(N), rg(size_t(N) * k);
  oracle_send_counts(idx.data(), T, E, k, R, place.data(), 0, ec.data(), rc.data(), ro.data(),
                     eo.data());
  if (oracle_dispatch(reinterpret_cast<const uint8_t*>(x.data()), idx.data(), gate.data(), T,
                      H * 2, E, k, eo.data(), reinterpret_cast<uint8_t*>(send.data()), rt.data(),
                      re.data(), rw.data(), sr.data()))
    return 1;
  if (oracle_combine(send.data(), rw.data(), sr.data(), T, H, k, out.data())) return 1;
  oracle_send_counts(idx.data(), T, E, k, R, place.data(), 1, ec.data(), rc.data(), ro.data(),
                     nullptr);
  if (oracle_dispatch_dedup(reinterpret_cast<const uint8_t*>(x.data()), idx.data(), gate.data(),
                            T, H * 2, E, k, R, place.data(), ro.data(),
                            reinterpret_cast<uint8_t*>(send.data()), rt.data(), rx.data(),
                            rg.data(), rw.data(), sr.data(), nr.data()))
    return 1;
  std::vector<uint16_t> expd(size_t(N) * H);
  std::vector<int32_t> er(N), ee(N), rs(size_t(N) * k);
  std::vector<float> eg(N);
  if (oracle_expand_dedup(reinterpret_cast<const uint8_t*>(send.data()), rx.data(), rg.data(),
                          nr[0], N, H * 2, E, k, R, place.data(), ec.data(), rc.data(),
                          ro.data(), eo.data(), reinterpret_cast<uint8_t*>(expd.data()),
                          er.data(), ee.data(), eg.data(), rs.data()))
    return 1;
  std::vector<uint16_t> red(size_t(N) * H);
  if (oracle_combine(expd.data(), eg.data(), rs.data(), nr[0], H, k, red.data())) return 1;
  std::vector<uint8_t> f8(size_t(N) * H);
  for (auto& v : f8) v = uint8_t(g() & 0x7E);
  if (oracle_combine_fp8(f8.data(), rw.data(), sr.data(), T, H, k, out.data())) return 1;
  std::vector<int32_t> W(size_t(E) * E, 0);
  if (oracle_coselect(idx.data(), T, E, k, W.data())) return 1;
  std::vector<int32_t> p1(E), p2(E);
  int64_t o1 = 0, o2 = 0;
  int s1 = 0, s2 = 0;
  if (oracle_placement_search(W.data(), E, R, nullptr, E * E, p1.data(), &o1, &s1)) return 1;
  if (moe::placement_search(W.data(), E, R, nullptr, E * E, p2.data(), &o2, &s2)) return 1;
  if (p1 != p2 || o1 != o2 || s1 != s2) return 2;
  // token-shuffle planner: the three layers are the routing above and two
  // shuffled copies of it; T rounded down to a multiple of R for the assignment
  std::vector<int32_t> prev(idx), next(idx);
  std::shuffle(prev.begin(), prev.end(), g);
  std::shuffle(next.begin(), next.end(), g);
  std::vector<int32_t> pair(size_t(E) * E * R, 0), single(size_t(E) * R, 0);
  if (oracle_shuffle_fit(prev.data(), idx.data(), next.data(), T, E, k, R, place.data(),
                         pair.data(), single.data()))
    return 1;
  std::vector<float> sc(size_t(T) * R);
  for (int min_obs : {0, 1, 3, 1 << 30})
    if (oracle_shuffle_predict(prev.data(), idx.data(), T, E, k, R, pair.data(), single.data(),
                               min_obs, sc.data()))
      return 1;
  const int Ta = T / R * R;
  std::vector<int32_t> o_or(size_t(Ta) + 1), o_lib(size_t(Ta) + 1);
  if (oracle_shuffle_assign(sc.data(), Ta, R, o_or.data())) return 1;
  if (moe::shuffle_assign(sc.data(), Ta, R, o_lib.data())) return 1;
  if (o_or != o_lib) return 3;
  return 0;
}

int main() {
  const int cases[][5] = {{1, 1, 1, 1, 8},  {7, 8, 3, 4, 8},   {65, 16, 16, 8, 16},
                          {33, 12, 2, 3, 8}, {200, 64, 6, 16, 8}, {5, 64, 64, 64, 8}};
  unsigned seed = 1;
  for (auto& c : cases) {
    const int rc = run(c[0], c[1], c[2], c[3], c[4], seed++);
    if (rc) {
      printf("case T=%d E=%d k=%d R=%d failed (%d)\n", c[0], c[1], c[2], c[3], rc);
      return rc;
    }
  }
  printf("ok\n");
  return 0;
}
