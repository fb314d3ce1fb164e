// Job order of the attention grids (host and device: the kernels call it
// with their workgroup index; a host test enumerates whole grids).
//
// A grid has nroles * nblk * npairs workgroups: nroles kinds of work (the
// fused backward has two, dQ and dK/dV; the forward one), nblk 128-row
// blocks along the sequence and npairs (sequence, head) pairs. Workgroup j
// runs on XCD j % 8 (round-robin dispatch) and takes the (j / 8)-th entry of
// that XCD's list. Under the causal mask a block's work depends on its rank
// (its distance from the long end of the sequence), so each list is in rank
// order, roles alternating: an XCD starts its longest jobs first and its
// short ones fill the compute units that free up. A list holds whole pairs
// where the pairs divide evenly over the 8 XCDs, so the workgroups that
// stream one pair's tiles share that XCD's L2. Otherwise each pair is cut
// into m parts by rank modulo m (m = 8 / gcd(npairs, 8)) and every XCD takes
// the same number of whole parts, which keeps the work of the XCDs even, not
// only their job counts. When nblk does not divide by m there is one list,
// the whole grid in rank order, without L2 grouping. A role's block is its
// rank, or nblk - 1 - rank where that role's rev flag is set.
#pragma once

#include <hip/hip_runtime.h>

namespace tpl {

struct AttnJob {
  int blk, pair, role;  // blk < 0: j is past the grid
};

__host__ __device__ inline AttnJob attn_job(int j, int nblk, int npairs, int nroles, bool rev0,
                                            bool rev1) {
  const int low = npairs & -npairs;  // largest power of two dividing npairs
  int m = 8 / (low < 8 ? low : 8);
  int u0, u1, t;  // parts [u0, u1): part u = the ranks r of pair u / m with r % m == u % m
  if (nblk % m == 0) {
    const int Q = npairs * m / 8;
    u0 = (j % 8) * Q;
    u1 = u0 + Q;
    t = j / 8;
  } else {
    m = 1;
    u0 = 0;
    u1 = npairs;
    t = j;
  }
  for (int r = 0; r < nblk; ++r) {
    const int k = r & (m - 1);
    const int plo = (u0 - k + m - 1) / m, pend = (u1 - 1 - k + m) / m;  // pairs with a part in range
    const int cnt = pend > plo ? pend - plo : 0;
    if (t < nroles * cnt) {
      const int role = t % nroles;
      const bool rev = role ? rev1 : rev0;
      return AttnJob{rev ? nblk - 1 - r : r, plo + t / nroles, role};
    }
    t -= nroles * cnt;
  }
  return AttnJob{-1, 0, 0};
}

}  // namespace tpl
