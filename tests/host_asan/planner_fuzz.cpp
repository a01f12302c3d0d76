// Host-only fuzz of the planners under AddressSanitizer: random lengths, exact
// and tight capacities, padding on and off.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>
#include "kvc.h"
int main(int argc, char** argv) {
  std::mt19937_64 g(1);
  long checks = 0;
  const int iters = argc > 1 ? atoi(argv[1]) : 5000;
  for (int it = 0; it < iters; ++it) {
    int B = 1 + g() % 8;
    std::vector<int64_t> sl(B), el(B);
    int64_t N = 0;
    for (int b = 0; b < B; ++b) { el[b] = 1 + g() % 700; sl[b] = el[b] + g() % 700; N += el[b]; }
    // two-list planner, exact-size buffers
    std::vector<kvc_online_plan> cp(N), wp(N);
    uint32_t nc, nw;
    int rc = kvc_c128_plan_prefill(sl.data(), el.data(), B, N, cp.data(), wp.data(), (int)(g() & 1), &nc, &nw);
    if (rc) { printf("plan rc %d: %s\n", rc, kvc_last_error()); return 1; }
    // fused planner with the bound capacity and with a deliberately tight one
    int64_t cap = kvc_c128_fused_capacity(N, B);
    std::vector<kvc_online_item> items(cap);
    uint32_t ni;
    rc = kvc_c128_plan_prefill_fused(sl.data(), el.data(), B, N, items.data(), cap, 0, &ni);
    if (rc) { printf("fused rc %d: %s\n", rc, kvc_last_error()); return 1; }
    uint32_t np;
    rc = kvc_c128_plan_prefill_fused(sl.data(), el.data(), B, N, items.data(), cap, 1, &np);
    if (rc || np != cap) { printf("fused pad rc %d\n", rc); return 1; }
    int64_t tight = (int64_t)ni > 0 ? (int64_t)ni - (int64_t)(g() % 2) : 0;
    std::vector<kvc_online_item> small(tight > 0 ? tight : 1);
    uint32_t ns;
    rc = kvc_c128_plan_prefill_fused(sl.data(), el.data(), B, N, small.data(), tight, (int)(g() & 1), &ns);
    if (tight < (int64_t)ni ? rc != KVC_ERR_PLAN : rc != KVC_OK) { printf("tight rc %d\n", rc); return 1; }
    // pool planner with capacity below and at the need
    std::vector<int64_t> lens(B);
    for (int b = 0; b < B; ++b) lens[b] = g() % 900;
    int64_t need;
    kvc_plan_pool_prefill(lens.data(), B, 16, nullptr, 0, &need);
    std::vector<int32_t> rows(need > 0 ? need : 1);
    rc = kvc_plan_pool_prefill(lens.data(), B, 16, rows.data(), need, &need);
    if (rc) { printf("pool rc %d\n", rc); return 1; }
    checks += 4;
  }
  printf("asan planner fuzz ok: %ld calls\n", checks);
  return 0;
}
