// Host check of the M = 1 step kernel's row plan (verify_gemm_amd/csrc/
// step_plan.h), built with the host compiler by test_step_plan.py.  Prints
// the plan of a 64-layer pass's first layer and checks, over seeded random
// stage sets and grids, that every row of every job goes to exactly one
// workgroup, that each stage's signal count is the number of workgroups
// holding its rows, and that no workgroup holds more than 33/32 of the
// largest share an even split could give it (the sum over the stage of
// ceil(n / G) * k).  Exit status 0: all checks held.
#include <cstdio>
#include <cstdint>
#include <vector>

#include "step_plan.h"

using vg::StreamJob;

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static int rnd(int n) {  // xorshift64*, uniform enough for shapes
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (int)(((rng * 0x2545F4914F6CDD1Dull) >> 33) % (uint64_t)n);
}

static bool check(std::vector<StreamJob>& jobs, int G, int nstages) {
  std::vector<unsigned> totals((size_t)nstages, 0);
  vg::plan_step_rows(jobs, G, totals);
  size_t b = 0;
  for (int s = 0; s < nstages; ++s) {
    size_t e = b;
    while (e < jobs.size() && jobs[e].stage == s) ++e;
    std::vector<long long> load((size_t)G, 0);
    long long bound = 0;
    for (size_t q = b; q < e; ++q) {
      const StreamJob& j = jobs[q];
      std::vector<int> seen((size_t)j.n, 0);
      for (int w = 0; w < G; ++w) {
        int pos;
        const int r = vg::step_rows(j, w, G, pos);
        if (r < 0 || pos < 0 || pos + r > j.n) {
          printf("job %zu: workgroup %d rows [%d, %d) outside [0, %d)\n", q, w, pos, pos + r, j.n);
          return false;
        }
        for (int i = 0; i < r; ++i) ++seen[(size_t)(pos + i)];
        load[(size_t)w] += (long long)r * j.k;
      }
      for (int i = 0; i < j.n; ++i)
        if (seen[(size_t)i] != 1) {
          printf("job %zu: row %d held by %d workgroups\n", q, i, seen[(size_t)i]);
          return false;
        }
      bound += (long long)((j.n + G - 1) / G) * j.k;
    }
    unsigned holders = 0;
    long long mx = 0;
    for (int w = 0; w < G; ++w) {
      holders += load[(size_t)w] > 0 ? 1u : 0u;
      mx = load[(size_t)w] > mx ? load[(size_t)w] : mx;
    }
    if (holders != totals[(size_t)s]) {
      printf("stage %d: %u workgroups hold rows, signal count %u\n", s, holders, totals[(size_t)s]);
      return false;
    }
    if (32 * mx > 33 * bound) {
      printf("stage %d: largest workgroup share %lld above 33/32 of %lld\n", s, mx, bound);
      return false;
    }
    b = e;
  }
  return true;
}

int main() {
  // one layer of the 64-layer pass, then the lm_head, on 256 workgroups
  const int n[7] = {5120, 5120, 5120, 5120, 17408, 17408, 5120};
  const int k[7] = {5120, 5120, 5120, 5120, 5120, 5120, 17408};
  const int st[7] = {0, 0, 0, 1, 2, 2, 3};
  std::vector<StreamJob> jobs;
  for (int i = 0; i < 7; ++i) {
    StreamJob j{};
    j.n = n[i];
    j.k = k[i];
    j.stage = st[i];
    jobs.push_back(j);
  }
  StreamJob lm{};
  lm.n = 248320;
  lm.k = 5120;
  lm.kind = 1;
  lm.stage = 4;
  jobs.push_back(lm);
  if (!check(jobs, 256, 5)) return 1;
  for (const StreamJob& j : jobs) printf("layer job n=%d k=%d stage=%d wg0=%d wgn=%d\n", j.n, j.k, j.stage, j.wg0, j.wgn);
  // a stage that keeps the even split on 256 workgroups (a partition's
  // largest share would be above 33/32 of it), its extra rows rotated
  std::vector<StreamJob> spread;
  const int sn[3] = {491, 768, 300}, sk[3] = {1024, 1024, 64};
  for (int i = 0; i < 3; ++i) {
    StreamJob j{};
    j.n = sn[i];
    j.k = sk[i];
    j.stage = 0;
    spread.push_back(j);
  }
  if (!check(spread, 256, 1)) return 1;
  for (const StreamJob& j : spread) printf("spread job n=%d k=%d wg0=%d wgn=%d rr=%d\n", j.n, j.k, j.wg0, j.wgn, j.rr);
  int cases = 0;
  for (int it = 0; it < 3000; ++it) {
    const int G = 1 + rnd(320);
    std::vector<StreamJob> js;
    const int nst = 1 + rnd(4);
    for (int s = 0; s < nst; ++s) {
      const int c = 1 + rnd(6);
      for (int q = 0; q < c; ++q) {
        StreamJob j{};
        j.n = 1 + rnd(rnd(2) ? 48 : 4000);
        j.k = 64 * (1 + rnd(288));
        j.stage = s;
        js.push_back(j);
      }
    }
    if (!check(js, G, nst)) {
      printf("failed: case %d, grid %d\n", it, G);
      return 1;
    }
    ++cases;
  }
  printf("random cases ok: %d\n", cases);
  return 0;
}
