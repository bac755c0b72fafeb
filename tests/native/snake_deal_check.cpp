// Host check of the prefill's snake deal of units to XCDs (duo_internal.h,
// prefill.hip): for seeded sequence sets, every (unit, query tile) is dealt
// to exactly one work item, items past an XCD's units return false, the
// work-group count is 8 x the largest XCD's tile count, and a deal is
// offered only when the XCDs' work is within 10% of even.  Links the built
// library for snake_deal_items and finish_seqs; runs no GPU code.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "duo_internal.h"

static int check(const duo::Seqs& q, int ups, int tq) {
  const int units = q.nact * ups;
  const int64_t items = duo::snake_deal_items(q, ups, tq);
  // the host's own sums, for the balance and count rules
  std::vector<int64_t> slots(8, 0), work(8, 0);
  for (int j = 0; 8 * j < units; ++j)
    for (int x = 0; x < 8; ++x) {
      const int u = duo::snake_unit(j, x);
      if (u >= units) continue;
      const int b = q.act[u / ups];
      const int64_t tiles = (q.n[b] + tq - 1) / tq;
      slots[x] += tiles;
      work[x] += tiles * (2 * (int64_t)q.len[b] + q.n[b]);
    }
  int64_t max_slots = 0, max_work = 0, sum_work = 0;
  for (int x = 0; x < 8; ++x) {
    if (slots[x] > max_slots) max_slots = slots[x];
    if (work[x] > max_work) max_work = work[x];
    sum_work += work[x];
  }
  const bool balanced = units >= 16 && 80 * max_work <= 11 * sum_work;
  if (items != (balanced ? 8 * max_slots : 0)) {
    std::printf("items %lld, expected %lld\n", (long long)items, (long long)(balanced ? 8 * max_slots : 0));
    return 1;
  }
  if (items == 0) return 0;
  std::vector<std::vector<int>> seen(units);
  for (int u = 0; u < units; ++u) seen[u].assign((q.n[q.act[u / ups]] + tq - 1) / tq, 0);
  for (int64_t id = 0; id < items; ++id) {
    int t = -1, u = -1;
    if (!duo::snake_deal_item(q, (int)id, units, ups, tq, t, u)) continue;
    if (u < 0 || u >= units || t < 0 || t >= (int)seen[u].size()) {
      std::printf("item %lld -> unit %d tile %d out of range\n", (long long)id, u, t);
      return 1;
    }
    if (seen[u][t]++) {
      std::printf("unit %d tile %d dealt twice\n", u, t);
      return 1;
    }
  }
  for (int u = 0; u < units; ++u)
    for (size_t t = 0; t < seen[u].size(); ++t)
      if (seen[u][t] != 1) {
        std::printf("unit %d tile %zu not dealt\n", u, t);
        return 1;
      }
  return 0;
}

int main() {
  std::mt19937 rng(1234);
  int offered = 0, declined = 0;
  for (int trial = 0; trial < 400; ++trial) {
    duo::Seqs q{};
    const int batch = 1 + (int)(rng() % 64);
    const bool chunked = trial % 3 == 0;
    for (int b = 0; b < batch; ++b) {
      q.len[b] = chunked ? (int)(rng() % 65536) : (trial % 5 == 0 ? 0 : (int)(rng() % 4096));
      q.n[b] = (rng() % 9 == 0) ? 0 : (chunked ? 4096 : 1 + (int)(rng() % 5000));
      q.off[b] = 0;
    }
    duo::finish_seqs(q, batch);
    for (int ups : {1, 2, 4, 8})
      for (int tq : {32, 64, 128}) {
        if (check(q, ups, tq)) {
          std::printf("FAIL trial %d batch %d ups %d tq %d\n", trial, batch, ups, tq);
          return 1;
        }
        (duo::snake_deal_items(q, ups, tq) > 0 ? offered : declined)++;
      }
  }
  std::printf("ok offered=%d declined=%d\n", offered, declined);
  return offered > 0 && declined > 0 ? 0 : 2;
}
