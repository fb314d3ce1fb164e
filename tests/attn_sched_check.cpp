// Host check of the attention grids' job lists (attn_sched.hpp), built and
// run by test_attn_sched.py. For every grid shape in the sweep: each
// workgroup index maps to a distinct (role, block, pair) inside the grid, so
// every output block is written exactly once; every XCD list is in rank
// order (longest causal jobs first); all 8 lists have the same length when
// the grid is grouped by XCD. Prints "ok" and exits 0, or names the first
// failing shape and exits 1.
#include <cstdio>
#include <set>
#include <tuple>
#include <vector>

#include "attn_sched.hpp"

using tpl::attn_job;
using tpl::AttnJob;

static int fail(const char* what, int nblk, int npairs, int nroles, int j) {
  std::printf("FAIL %s: nblk %d npairs %d nroles %d j %d\n", what, nblk, npairs, nroles, j);
  return 1;
}

int main() {
  for (int nblk = 1; nblk <= 40; ++nblk)
    for (int npairs = 1; npairs <= 48; ++npairs)
      for (int nroles = 1; nroles <= 2; ++nroles)
        for (int rv = 0; rv < 4; ++rv) {
          const bool rev0 = rv & 1, rev1 = rv & 2;
          const int n = nroles * nblk * npairs;
          // grouped by XCD when nblk divides by m = 8 / gcd(npairs, 8)
          int g = 1;
          while (g < 8 && npairs % (2 * g) == 0) g *= 2;
          const bool grouped = nblk % (8 / g) == 0;
          if (grouped && n % 8 != 0) return fail("list lengths", nblk, npairs, nroles, n);
          std::set<std::tuple<int, int, int>> seen;
          std::vector<int> rank_of(n, -1);
          for (int j = 0; j < n; ++j) {
            const AttnJob a = attn_job(j, nblk, npairs, nroles, rev0, rev1);
            if (a.blk < 0 || a.blk >= nblk || a.pair < 0 || a.pair >= npairs || a.role < 0 ||
                a.role >= nroles)
              return fail("out of range", nblk, npairs, nroles, j);
            if (!seen.insert({a.role, a.blk, a.pair}).second)
              return fail("duplicate job", nblk, npairs, nroles, j);
            const bool rev = a.role ? rev1 : rev0;
            rank_of[j] = rev ? nblk - 1 - a.blk : a.blk;
            const int prev = grouped ? j - 8 : j - 1;  // previous entry of the same list
            if (prev >= 0 && rank_of[prev] > rank_of[j])
              return fail("rank order", nblk, npairs, nroles, j);
          }
          if ((int)seen.size() != n) return fail("coverage", nblk, npairs, nroles, n);
          if (attn_job(n, nblk, npairs, nroles, rev0, rev1).blk >= 0)
            return fail("past the grid", nblk, npairs, nroles, n);
        }
  std::printf("ok\n");
  return 0;
}
