// Host build of the work-decomposition formulas the library's host sizing and its planner
// kernel share (pa_internal.h), checked for calls sized for a capacity M (graph_max_seq_len):
// the host counts every request at seq_len M, the planner kernel recounts it at its device
// length, clamped to M.  For every head-group size, window and pool kind, every query-row
// count such a call admits (rows x g <= 64) and every device length from 0 (a padding row of
// a pad_to batch, "Flattened ragged batches") to past M, no list may get more items on the
// device than the host sized it for.  A batch-level pass then lays out whole batches the way
// the planner does (exclusive scans) and checks every item index against the host's list
// sizes.  Prints one line per failure and "checked N" at the end; exits non-zero on failure.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "pa_internal.h"

using pa::Plan;

namespace {

struct Counts {
  int64_t small = 0, merge = 0, pf = 0, g1 = 0, g3 = 0, stage = 0;
};

Counts counts(const Plan& p, int32_t t, int32_t L) {
  Counts c;
  int32_t a, b, d, e;
  pa::request_counts(p, t, L, &a, &b, &d, &e);
  c.small = a;
  c.merge = b;
  c.pf = d;
  pa::small_groups(p, t, L, &a, &b);
  c.g1 = a;
  c.g3 = b;
  c.stage = pa::staged_blocks(p, t, L);
  return c;
}

int failures = 0;
int64_t checked = 0;

void expect_le(int64_t dev, int64_t host, const char* what, const Plan& p, int32_t t, int32_t M, int32_t L) {
  ++checked;
  if (dev <= host) return;
  if (++failures <= 20)
    std::printf("FAIL %s: device %lld > host %lld (g=%d window=%d f8=%d split=%d t=%d M=%d L=%d)\n", what,
                (long long)dev, (long long)host, p.g, p.window, p.f8, p.split_keys, t, M, L);
}

Plan make_plan(int32_t g, int32_t window, int32_t f8, int32_t split, int32_t M) {
  Plan p{};
  p.R = 1;
  p.H = g;
  p.Hkv = 1;
  p.g = g;
  p.D = 128;
  p.bs = 16;
  pa::set_tile_shape(p);
  p.split_keys = split;
  // the prefill path is on (bf16 pools, head_dim 128) where its tile divides the group;
  // a capacity-sized call never routes a request there (rows x g <= 64)
  p.pf_tokens = (256 % g == 0) ? 256 / g : 0;
  p.decode_kind = 1;
  p.window = window;
  p.f8 = f8;
  p.v16 = p.pf_tokens > 0 ? 1 : 0;
  p.graph_max = M;
  return p;
}

}  // namespace

int main() {
  const int32_t groups[] = {1, 2, 4, 8, 16, 32, 64};
  const int32_t windows[] = {0, 100};
  const int32_t splits[] = {64, 512, 2048};
  const int32_t caps[] = {1, 15, 16, 17, 64, 65, 100, 777, 2048, 5000};
  for (int32_t g : groups)
    for (int32_t window : windows)
      for (int32_t f8 = 0; f8 < 2; ++f8)
        for (int32_t split : splits)
          for (int32_t M : caps) {
            const Plan p = make_plan(g, window, f8, split, M);
            for (int32_t t = 1; t * g <= pa::kPrefillMinCols; ++t) {
              const Counts host = counts(p, t, M);
              for (int32_t L = 0; L <= M + 70; ++L) {
                const int32_t Ld = L < M ? L : M;   // the planner kernel's clamp
                const Counts dev = counts(p, t, Ld);
                expect_le(dev.small, host.small, "small-tile splits", p, t, M, L);
                expect_le(dev.merge, host.merge, "merge items", p, t, M, L);
                expect_le(dev.pf, host.pf, "prefill items", p, t, M, L);
                expect_le(dev.g1, host.g1, "single-tile items", p, t, M, L);
                expect_le(dev.g3, host.g3, "grouped items", p, t, M, L);
                expect_le(dev.stage, host.stage, "staged blocks", p, t, M, L);
                // a list with items on the device had room on the host (the partials and the
                // grids exist only where the host counted some)
                expect_le(dev.merge > 0, host.merge > 0, "merge partials present", p, t, M, L);
              }
            }
          }

  // whole batches: requests of random rows and device lengths, laid out by exclusive scans
  // as the planner kernel lays them out; every item index lies inside the host's list
  std::srand(12345);
  for (int trial = 0; trial < 4000; ++trial) {
    const int32_t g = groups[std::rand() % 7];
    const int32_t M = 1 + std::rand() % 6000;
    const Plan p = make_plan(g, (trial & 1) ? 100 : 0, (trial >> 1) & 1, splits[std::rand() % 3], M);
    const int32_t R = 1 + std::rand() % 40;
    Counts host_tot, dev_tot;
    for (int32_t r = 0; r < R; ++r) {
      const int32_t tmax = pa::kPrefillMinCols / g;
      const int32_t t = 1 + std::rand() % tmax;
      // padding rows (length 0), lengths below, at and past the capacity
      const int kind = std::rand() % 4;
      int32_t L = kind == 0 ? 0 : kind == 1 ? M : kind == 2 ? t + std::rand() % (M + 1) : M + 1 + std::rand() % 99;
      const int32_t Ld = L < M ? L : M;
      const Counts h = counts(p, t, M), d = counts(p, t, Ld);
      host_tot.small += h.small; host_tot.merge += h.merge; host_tot.g1 += h.g1; host_tot.g3 += h.g3;
      // the request's items sit at [its exclusive-scan offset, + its count) on the device
      const int64_t last_small = dev_tot.small + d.small - 1, last_merge = dev_tot.merge + d.merge - 1;
      const int64_t last_g1 = dev_tot.g1 + d.g1 - 1, last_g3 = dev_tot.g3 + d.g3 - 1;
      dev_tot.small += d.small; dev_tot.merge += d.merge; dev_tot.g1 += d.g1; dev_tot.g3 += d.g3;
      expect_le(last_small + 1, host_tot.small, "batch small-tile index", p, t, M, L);
      expect_le(last_merge + 1, host_tot.merge, "batch merge index", p, t, M, L);
      expect_le(last_g1 + 1, host_tot.g1, "batch single-tile index", p, t, M, L);
      expect_le(last_g3 + 1, host_tot.g3, "batch grouped index", p, t, M, L);
    }
  }
  std::printf("checked %lld\n", (long long)checked);
  if (failures) std::printf("%d failures\n", failures);
  return failures ? 1 : 0;
}
