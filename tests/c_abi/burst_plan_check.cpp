// Prints the burst launch plan (combine_ep_dispatch_amd/csrc/burst_plan.h)
// for the shapes given on the command line, so that a CPU test can check
// that every launch fits its workgroup's registers and LDS.
//   burst_plan_check T vpt items threads cus lds_per_token lds_limit ...
// (seven numbers per shape); per shape one line "plan launches slice
// tpb_max", then one line "slice Ts tpb grid lds" per launch.
#include <cstdio>
#include <cstdlib>

#include "../../combine_ep_dispatch_amd/csrc/burst_plan.h"

int main(int argc, char** argv) {
  for (int i = 1; i + 6 < argc; i += 7) {
    const long long T = atoll(argv[i]);
    const long long vpt = atoll(argv[i + 1]);
    const int items = atoi(argv[i + 2]), threads = atoi(argv[i + 3]), cus = atoi(argv[i + 4]);
    const size_t lds_per_token = static_cast<size_t>(atoll(argv[i + 5]));
    const size_t lds_limit = static_cast<size_t>(atoll(argv[i + 6]));
    const ep::BurstPlan p = ep::burst_plan(T, vpt, items, threads, cus, lds_per_token, lds_limit);
    printf("plan %d %d %d\n", p.launches, p.slice, p.tpb_max);
    if (p.launches == 0) continue;
    for (long long t0 = 0; t0 < T; t0 += p.slice) {
      const int Ts = static_cast<int>(T - t0 < p.slice ? T - t0 : p.slice);
      const int tpb = ep::burst_tpb(Ts, cus);
      printf("slice %d %d %d %zu\n", Ts, tpb, (Ts + tpb - 1) / tpb, static_cast<size_t>(tpb) * lds_per_token);
    }
  }
  return 0;
}
