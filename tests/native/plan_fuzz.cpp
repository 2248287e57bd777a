// Randomised host checks of the argument validation and workspace layout
// (csrc/gdn_plan.cpp), built with g++ and the address / undefined-behaviour
// sanitizers by tests/test_plan_sanitized.py.  Exits non-zero on the first
// broken invariant; a sanitizer report aborts on its own.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "gdn_plan.h"

static int fail(const char* what, int iter) {
  std::fprintf(stderr, "plan_fuzz: %s (iteration %d)\n", what, iter);
  return 1;
}

int main() {
  std::mt19937_64 rng(12345);
  auto pick = [&](int lo, int hi) { return static_cast<int>(lo + rng() % (hi - lo + 1)); };
  const int ds[] = {16, 64, 128, 17, 0, -1};
  const int Cs[] = {16, 64, 32, 0, -4};
  for (int it = 0; it < 20000; ++it) {
    gdn_shape_t s{};
    s.H_qk = pick(-1, 8);
    s.H_v = s.H_qk > 0 ? s.H_qk * pick(0, 9) : pick(-1, 8);
    s.d_k = ds[pick(0, 5)];
    s.d_v = pick(0, 7) == 0 ? ds[pick(0, 5)] : s.d_k;
    s.C = Cs[pick(0, 4)];
    s.in_dtype = pick(0, 2);
    s.qk_l2norm = pick(0, 2);
    s.scale = 1.0f;
    const int shape_rc = gdn::check_shape(&s);
    const int N = pick(0, 40);
    std::vector<int32_t> cu(static_cast<size_t>(N) + 1, 0);
    const bool bad = pick(0, 9) == 0;
    for (int n = 0; n < N; ++n) cu[n + 1] = cu[n] + pick(0, 3000);
    if (bad && N > 0) cu[pick(1, N)] -= pick(1, 5000);
    if (bad && pick(0, 1)) cu[0] = pick(1, 3);
    gdn::Counts cnt;
    const int C = s.C > 0 ? s.C : 64;
    const int crc = gdn::count_chunks(cu.data(), N, C, &cnt);
    bool mono = cu[0] == 0;
    for (int n = 0; n < N; ++n) mono = mono && cu[n + 1] >= cu[n];
    if ((crc == GDN_OK) != mono) return fail("count_chunks accepts exactly the monotone prefixes from 0", it);
    if (crc == GDN_OK) {
      int64_t chunks = 0, full = 0;
      for (int n = 0; n < N; ++n) {
        const int64_t L = cu[n + 1] - cu[n];
        chunks += (L + C - 1) / C;
        full += L / C;
      }
      if (cnt.T != cu[N] || cnt.chunks != chunks || cnt.full != full) return fail("counts", it);
    }
    for (int op = -1; op <= 5; ++op) {
      const int64_t T = crc == GDN_OK ? cnt.T : pick(0, 100000);
      const gdn::Layout L = gdn::layout(&s, N, T, op);
      if (shape_rc != GDN_OK && L.total != 0) return fail("a rejected shape gets no layout", it);
      if (L.total == 0) continue;
      // in the order layout() hands them out
      const size_t regions[] = {L.cu_chunks, L.cu_full, L.qk,  L.W,      L.U,    L.G,     L.states,
                                L.order,     L.Dl,      L.E,   L.dstates, L.dD,  L.SdO,   L.DsD,
                                L.SdD,       L.dqv,     L.dkv, L.cu_ext, L.v_ext, L.b_ext,
                                L.g_ext,     L.o_ext};
      // offsets are aligned, inside the workspace (an empty region may sit at
      // its end) and never decrease (empty regions share an offset)
      size_t prev = 0;
      for (size_t r : regions) {
        if (r == 0) continue;
        if (r % gdn::kAlign != 0) return fail("region alignment", it);
        if (r > L.total) return fail("region inside the workspace", it);
        if (r < prev) return fail("regions in allocation order", it);
        prev = r;
      }
      if (L.total % gdn::kAlign != 0) return fail("total size alignment", it);
      if (op == GDN_OP_PREFILL || op == GDN_OP_FWD_BWD) {
        if (L.state_slots < T / C + N || L.full_slots < T / C) return fail("slot bounds", it);
      }
    }
  }
  std::printf("plan_fuzz: ok\n");
  return 0;
}
