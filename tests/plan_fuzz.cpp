// The planner (pure host code) over random shapes and options: built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_plan_sanitized.py, so an
// out-of-bounds access, a signed overflow or another undefined operation in the grid and
// workspace arithmetic stops the run.  Shapes reach N = 2^31 - 1 and M * N up to 2^62.
#include <cstdio>
#include <cstdlib>
#include <random>
#include "plan.h"
using namespace rownorm;
int main(int argc, char** argv) {
  const long iters = argc > 1 ? std::atol(argv[1]) : 200000;
  std::mt19937_64 g(12345);
  long ok = 0, bad = 0;
  auto rnd = [&](int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(g); };
  const int lprs[] = {0, 8, 16, 32, 64, 128, 256, 512, 1024};
  for (long it = 0; it < iters; ++it) {
    const bool bwd = g() & 1, ln = g() & 1;
    const int dt = int(rnd(0, 2));
    int64_t N;
    switch (rnd(0, 3)) {
      case 0: N = rnd(1, 64); break;
      case 1: N = rnd(1, 1 << 17); break;
      case 2: N = rnd(1, (int64_t(1) << 31) - 1); break;
      default: N = int64_t(1) << rnd(0, 30); break;
    }
    int64_t M;
    switch (rnd(0, 3)) {
      case 0: M = rnd(0, 4); break;
      case 1: M = rnd(0, 1 << 20); break;
      case 2: M = rnd(0, (int64_t(1) << 40) / (N > 0 ? N : 1)); break;
      default: M = (int64_t(1) << 62) / N; break;
    }
    if (N > 0 && M > INT64_MAX / N) continue;
    norm_options_t o = {};
    const bool use_opt = g() & 1;
    if (use_opt) {
      o.path = int(rnd(0, 4));
      o.lanes_per_row = lprs[rnd(0, 8)];
      o.vecs_per_lane = int(rnd(0, 16));
      o.grid = int(rnd(0, 3)) ? int(rnd(0, 70000)) : 0;
      o.cluster_size = int(rnd(0, 3)) ? (1 << rnd(0, 6)) : 0;
      o.cluster_rows = int(rnd(0, 3));
      o.pipeline = int(rnd(0, 3));
      o.dgamma_mode = int(rnd(0, 3));
    }
    Plan p;
    const norm_status_t st = make_plan(bwd, ln, M, N, dt, g() & 1, use_opt ? &o : nullptr, &p);
    if (st == NORM_OK) {
      ++ok;
      volatile size_t w = workspace_bytes(bwd, M, N, ln, dt, use_opt ? &o : nullptr);
      (void)w;
      if (!bwd) { Plan q; make_fwd_plan_without_workspace(ln, M, N, dt, g() & 1, use_opt ? &o : nullptr, &q); }
      if (p.path == NORM_PATH_CLUSTER) { Plan f; make_fallback_plan(bwd, ln, M, N, dt, &f); }
    } else {
      ++bad;
    }
  }
  std::printf("ok %ld refused %ld\n", ok, bad);
  return 0;
}
