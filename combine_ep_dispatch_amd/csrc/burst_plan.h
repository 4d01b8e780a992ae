// Sizing of the burst launches (internal; pure host code, no HIP): the
// burst combine and the burst fan-out of BF16 rows run one workgroup per CU,
// each holding its tokens' work items in registers, and a batch larger than
// one such wave of workgroups goes as equal token slices, one launch each.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace ep {

// T tokens of vpt work items each, over `cus` workgroups of `threads` lanes
// that hold at most `items` work items per lane; each token also takes
// lds_per_token bytes of the workgroup's LDS (at most lds_limit).  The batch
// goes in `launches` slices of at most `slice` tokens; a slice of Ts tokens
// runs ceil(Ts / tpb) workgroups of tpb = ceil(Ts / cus) <= tpb_max tokens
// (burst_tpb).  launches == 0: no plan (no tokens, an unknown CU count, or
// not even one token fits a workgroup); the caller then takes another path.
struct BurstPlan {
  int launches;
  int slice;
  int tpb_max;
};

inline BurstPlan burst_plan(int64_t T, int64_t vpt, int items, int threads, int cus, size_t lds_per_token,
                            size_t lds_limit) {
  const BurstPlan none{0, 0, 0};
  if (T <= 0 || vpt <= 0 || items <= 0 || threads <= 0 || cus <= 0) return none;
  int64_t tpb_max = static_cast<int64_t>(items) * threads / vpt;
  if (lds_per_token > 0) {
    const int64_t by_lds = static_cast<int64_t>(lds_limit / lds_per_token);
    if (by_lds < tpb_max) tpb_max = by_lds;
  }
  if (tpb_max <= 0) return none;
  const int64_t per_launch = static_cast<int64_t>(cus) * tpb_max;
  const int64_t launches = (T + per_launch - 1) / per_launch;
  const int64_t slice = (T + launches - 1) / launches;
  return BurstPlan{static_cast<int>(launches), static_cast<int>(slice), static_cast<int>(tpb_max)};
}

// Tokens per workgroup for a slice of Ts tokens.
inline int burst_tpb(int Ts, int cus) { return (Ts + cus - 1) / cus; }

}  // namespace ep
