// Host-side plan of the M = 1 step kernel's rows per workgroup (header
// only, no device code: the library and a host check both include it).
#pragma once

#include <algorithm>
#include <vector>

#include "launch.h"

namespace vg {

// The M = 1 step kernel's rows per workgroup, stage by stage (the step
// fields of each job; the stream-kernel item fields they overlay are not
// used by a step plan).  A stage of one matrix is split evenly over the
// grid.  A stage of several GEMMs is split either way:
//   * even: every matrix over the whole grid, each matrix's extra rows
//     starting where the previous matrix's ended, so that no workgroup
//     collects more than one of them beyond its share;
//   * partitioned: each matrix over its own run of workgroups, the runs
//     sized to the matrices' bytes (n * k) to minimise the largest
//     workgroup's bytes.  Measured on the 64-layer pass (256 workgroups):
//     q, k, v on 85, 85 and 86 workgroups (60 or 61 rows of one matrix, two
//     chunks of ~30) instead of 20 rows of each on every workgroup (three
//     chunks of 20 in three regions) took the step from 4.07 to 3.96 ms
//     with the same output bits; small, scattered chunks keep fewer weight
//     bytes in flight per CU.
// The partition is taken when its largest workgroup holds at most 1/32 more
// bytes than the even split's (q, k, v: 61 rows against 60).
inline void plan_step_rows(std::vector<StreamJob>& jobs, int G, std::vector<unsigned>& totals) {
  std::vector<long long> load((size_t)G);
  std::vector<unsigned char> has((size_t)G);
  size_t b = 0;
  for (size_t s = 0; s < totals.size(); ++s) {
    size_t e = b;
    while (e < jobs.size() && jobs[e].stage == (int)s) ++e;
    const int cnt = (int)(e - b);
    // even split, rotated by the extra rows already dealt
    int start = 0;
    std::fill(load.begin(), load.end(), 0);
    for (size_t q = b; q < e; ++q) {
      set_step_rows(jobs[q], start, G);
      start = (start + jobs[q].rr) % G;
      for (int w = 0; w < G; ++w) {
        int pos;
        load[(size_t)w] += (long long)step_rows(jobs[q], w, G, pos) * jobs[q].k;
      }
    }
    const long long even_max = cnt ? *std::max_element(load.begin(), load.end()) : 0;
    bool gemms = true;
    for (size_t q = b; q < e; ++q) gemms = gemms && jobs[q].kind == 0;
    if (cnt >= 2 && cnt <= G && gemms) {
      // one workgroup each, then every further workgroup to the matrix
      // whose largest share is largest (ties: the largest mean share)
      std::vector<int> g((size_t)cnt, 1);
      auto share = [&](int i) {
        const StreamJob& j = jobs[b + (size_t)i];
        return (long long)((j.n + g[(size_t)i] - 1) / g[(size_t)i]) * j.k;
      };
      auto mean = [&](int i) {
        const StreamJob& j = jobs[b + (size_t)i];
        return (double)j.n * j.k / g[(size_t)i];
      };
      for (int left = G - cnt; left > 0; --left) {
        int best = 0;
        for (int i = 1; i < cnt; ++i)
          if (share(i) > share(best) || (share(i) == share(best) && mean(i) > mean(best))) best = i;
        ++g[(size_t)best];
      }
      long long part_max = 0;
      for (int i = 0; i < cnt; ++i) part_max = std::max(part_max, share(i));
      if (32 * part_max <= 33 * even_max) {
        int w0 = 0;
        for (int i = 0; i < cnt; ++i) {
          set_step_rows(jobs[b + (size_t)i], w0, g[(size_t)i]);
          w0 += g[(size_t)i];
        }
      }
    }
    std::fill(has.begin(), has.end(), 0);
    for (size_t q = b; q < e; ++q)
      for (int w = 0; w < G; ++w) {
        int pos;
        if (step_rows(jobs[q], w, G, pos) > 0) has[(size_t)w] = 1;
      }
    totals[s] = (unsigned)std::count(has.begin(), has.end(), 1);
    b = e;
  }
}

}  // namespace vg
