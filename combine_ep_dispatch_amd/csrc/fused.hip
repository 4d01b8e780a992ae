// Layout and dispatch in one launch, for small batches (decode).
//
// The pages' dispatch call takes the tokens with their routing and returns
// the received rows together with the handle ([P4 "使用示例 › MoE 训练中的
// 应用"]); its low-latency form fills per-expert buffers of a fixed number
// of rows and reports per-expert counts ([P4 "使用示例 › 推理解码阶段的应用"]).
// At decode sizes a launch costs a few microseconds of mostly fixed latency,
// so this kernel writes everything the layout kernels and the dispatch
// kernel would, bit for bit, in a single launch.
//
// A token's receive rows have a closed form as counts over all n = T*K
// entries.  With key = expert for a valid entry and E for a masked one, and
// entry position p = t*K + k:
//   packed layout: row  = #{p' : (key', p') < (key, p)} (lexicographic), the
//                  stable counting sort by expert;
//   padded layout: rank = #{p' < p : key' == key}, row = key*capacity + rank,
//                  dropped when rank >= capacity.
// Encoding an entry as key*n + p turns either count into one integer range
// test per entry: the packed row counts codes below the entry's own, the
// padded rank the codes from key*n up to it (entries with a code below
// key*n are exactly those of a smaller key).  Each wavefront compares 64
// entries per step against its token's K codes and counts the matches with
// a ballot and a popcount, so the counts stay wave-uniform and only the
// per-wave totals meet, in LDS.
// Integer counting is exact and order-free: the result is a pure function
// of topk_idx.
//
// Work split: workgroup 0 histograms all entries with LDS atomic adds and
// writes counts (and, packed, the exclusive-scan offsets).  Every other
// workgroup owns the work items of one token (16 channels each for FP8, 8
// for BF16, as in the dispatch kernel; a token wider than 1024 items is
// split over several workgroups).  It issues the token loads first, so
// they overlap the counting, then finds the token's K rows.  The first
// workgroup of a token writes the token's slot, src and receive-weight
// entries.  Then every workgroup writes its part of the K receive rows.
// Every workgroup reads all n ids (4n bytes, from L2 after the first) and
// compares them with its token's K codes, so the counting grows as n*K per
// workgroup.  The path is used up to 3072 entries: against the layout
// kernels plus the dispatch kernel it broke even at 4096.  Larger batches
// run the chunked kernel (layout_dispatch.hip), or, past its limits, the
// layout kernels and the dispatch kernel.
//
// At decode sizes the kernel is latency-bound with one wave per SIMD, so a
// wave's serial instruction chain sets its time, and the code keeps that
// chain short: every id step is counted (codes past n match nothing, so no
// step count is needed), each wave turns the per-wave counts into rows
// itself (one barrier, not two), and the quantiser divides by one shared
// reciprocal (div_by_recip).  Measured on MI355X at 128 tokens of hidden
// 7168, top-8 of 256 experts, GPU time per launch in a graph: 4.5 us
// against 5.25 us with two barriers and a full division per channel; an
// empty launch of the same grid takes 1.7 us and one that only loads the
// token and ids and stores the 7.3 MB of rows 2.9 us.

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kMinThreads = 256;   // a workgroup has 256..1024 lanes, a multiple of 64
constexpr int kMaxThreads = 1024;
constexpr int kMaxWaves = kMaxThreads / kWave;
constexpr int kMaxK = 32;
static_assert(static_cast<int64_t>(1025) * kFusedMaxEntries < (int64_t(1) << 31), "entry codes fit int32");

// LDS: workgroup 0 needs E+1 histogram bins; the token workgroups need the
// per-wave counts, the K rows and the K keys.
constexpr int kTokenLdsInts = kMaxWaves * kMaxK + 2 * kMaxK;
constexpr int kLdsInts = 1025 > kTokenLdsInts ? 1025 : kTokenLdsInts;

// This lane's keys: entries u*bs + tid for u < NS (bs: the workgroup's
// lanes), with the address clamped to the last entry (n >= 1) so that all
// NS loads are issued back to back, free of branches; lanes past n get a
// copy of the last key, which callers mask by position.
template <int NS, typename Idx>
__device__ __forceinline__ void load_ids(const Idx* __restrict__ idx, int n, int bs, Idx (&raw)[NS]) {
#pragma unroll
  for (int u = 0; u < NS; ++u) raw[u] = idx[min(u * bs + static_cast<int>(threadIdx.x), n - 1)];
}

template <int NS, typename Idx>
__device__ __forceinline__ void load_keys(const Idx* __restrict__ idx, int n, int E, int bs, int (&e)[NS]) {
  Idx raw[NS];
  load_ids<NS>(idx, n, bs, raw);
#pragma unroll
  for (int u = 0; u < NS; ++u) e[u] = expert_key(raw[u], E);
}

// Workgroup 0: per-expert counts (clamped to the capacity in the padded
// layout) and, for the packed layout, the exclusive-scan offsets.
template <int NS, typename Idx>
__device__ void write_counts_block(const Idx* __restrict__ idx, int n, int E, int cap, int bs, int* lds,
                                   int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  const int tid = threadIdx.x, nk = E + 1;
  int* hist = lds;
  int e[NS];  // keys
  if (n > 0) load_keys<NS>(idx, n, E, bs, e);  // block-uniform; nothing to read for an empty batch
  for (int i = tid; i < nk; i += bs) hist[i] = 0;
  __syncthreads();
  if (n > 0) {
#pragma unroll
    for (int u = 0; u < NS; ++u)
      if (u * bs + tid < n) atomicAdd(&hist[e[u]], 1);
  }
  __syncthreads();
  for (int j = tid; j < E; j += bs) counts[j] = cap == 0 ? hist[j] : min(hist[j], cap);
  if (cap == 0) {  // block-uniform
    block_exclusive_scan(hist, nk);
    for (int j = tid; j <= E; j += bs) offsets[j] = hist[j];
  }
}

// Per-wave counts for targets k0 .. k0+KC-1 (keys te) of the token
// whose entries start at p0, as one unsigned comparison per entry:
//   packed: c_j = #{entries with lo_j <= code < code_j}, lo_j = 0: the row;
//   padded: the same with lo_j = key_j * n: the rank among entries with the
//           same key (codes from key*n up are those of that key or later).
// (uint)(code - lo) < (uint)(code_j - lo) holds exactly when
// lo <= code < code_j, because code - lo < 0 wraps to a large value.  `code`
// holds this lane's entry codes (INT_MAX past n); the wave's entries are
// lane + 64*w + bs*u.  Lane 0 of each wave leaves its counts in LDS,
// and wave 0 the targets' keys.
template <int KC, int NS>
__device__ __forceinline__ void count_targets(const int (&te)[KC], int p0, int k0, int K, int n, int E, bool padded,
                                              const int (&code)[NS], int nsteps, int* wc, int* tkey) {
  int tk[KC], lo[KC], span[KC], c[KC];
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    tk[j] = k0 + j < K ? te[j] : E;
    lo[j] = padded ? tk[j] * n : 0;
    span[j] = tk[j] * n + p0 + k0 + j - lo[j];
    c[j] = 0;
  }
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    if (u < nsteps) {  // wave-uniform
#pragma unroll
      for (int j = 0; j < KC; ++j)
        c[j] += __popcll(wave_ballot(static_cast<uint32_t>(code[u] - lo[j]) < static_cast<uint32_t>(span[j])));
    }
  }
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      if (k0 + j >= K) break;
      wc[w * kMaxK + k0 + j] = c[j];
      if (w == 0) tkey[k0 + j] = tk[j];
    }
  }
}

// NS: steps of bs entries per lane (n <= NS * bs).  MAXT: the largest
// workgroup the instantiation is launched with (256, or 1024 for
// token-wide workgroups); the tighter bound measured 0.25-0.45 us faster.
// Idx: int32_t or int64_t expert ids.  The workgroup size comes as an
// argument (a constant where MAXT fixes it), not from blockDim: reading
// blockDim makes the launch carry the runtime's implicit arguments, 256
// bytes more that the host writes for every launch (measured host cost of
// a launch: 2.6 us with 8 bytes of arguments, 3.5 us with 128).
template <int KT, bool FP8, int NS, int MAXT, typename Idx>
__global__ __launch_bounds__(MAXT) void layout_dispatch_kernel(
    const Idx* __restrict__ idx, const uint16_t* __restrict__ x, const float* __restrict__ w, int32_t T,
    int32_t H, int32_t Krt, int32_t E, int32_t cap, uint32_t nchunk, int32_t bs_arg, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot, int32_t* __restrict__ src, void* __restrict__ recv,
    float* __restrict__ recv_scale, float* __restrict__ recv_weight) {
  __shared__ int lds[kLdsInts];
  constexpr int KC = KT > 0 ? KT : 8;  // targets counted per pass over the ids
  const int K = KT > 0 ? KT : Krt;
  const int n = T * K;
  const int bs = MAXT == kMinThreads ? kMinThreads : bs_arg;
  if (blockIdx.x == 0) {
    write_counts_block<NS>(idx, n, E, cap, bs, lds, counts, offsets);
    return;
  }
  const uint32_t b = blockIdx.x - 1;
  const int t = static_cast<int>(b / nchunk);
  const uint32_t chunk = b - static_cast<uint32_t>(t) * nchunk;
  const int tid = threadIdx.x, nw = bs / kWave;
  const uint32_t vpt = static_cast<uint32_t>(H) / (FP8 ? 16 : 8);
  const uint32_t v = chunk * bs + tid;  // vector within the token
  const bool active = v < vpt;
  const int p0 = t * K;

  // every load up front: the token's expert ids, the token itself (its
  // latency overlaps the counting), then all ids.  The token is read with
  // plain loads: at these sizes it is usually still in the caches (measured
  // 5.7 against 6.0 us with streaming loads at 128 tokens)
  int te[KC];  // the token's keys
#pragma unroll
  for (int j = 0; j < KC; ++j) te[j] = expert_key(idx[p0 + min(j, K - 1)], E);
  // lane j < K carries the weight of target j (recv_weight implies w)
  float wj = 0.0f;
  if (recv_weight != nullptr) wj = w[p0 + min(static_cast<int>(tid & (kWave - 1)), K - 1)];
  u32x4 a = {0, 0, 0, 0}, a2 = {0, 0, 0, 0};
  if (active) {
    const u32x4* px = reinterpret_cast<const u32x4*>(x + static_cast<size_t>(t) * H);
    if (FP8) {
      a = px[2 * v];
      a2 = px[2 * v + 1];
    } else {
      a = px[v];
    }
  }
  Idx raw[NS];
  load_ids<NS>(idx, n, bs, raw);
  // keep every load above this point: the compiler would otherwise sink
  // some of them next to their first use, one memory latency after another
  asm volatile("" ::: "memory");
  int code[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int p = u * bs + tid;
    code[u] = p < n ? expert_key(raw[u], E) * n + p : 0x7FFFFFFF;
  }

  // every step is counted: codes past n are INT_MAX and match no target
  const int nsteps = NS;
  int* wc = lds;                        // [kMaxWaves][kMaxK]
  int* rows = lds + kMaxWaves * kMaxK;  // [kMaxK]
  int* tkey = rows + kMaxK;             // [kMaxK]
  const bool padded = cap > 0;
  count_targets<KC, NS>(te, p0, 0, K, n, E, padded, code, nsteps, wc, tkey);
  for (int k0 = KC; k0 < K; k0 += KC) {  // top-k beyond one pass (generic K only)
#pragma unroll
    for (int j = 0; j < KC; ++j) te[j] = expert_key(idx[p0 + min(k0 + j, K - 1)], E);
    count_targets<KC, NS>(te, p0, k0, K, n, E, padded, code, nsteps, wc, tkey);
  }
  __syncthreads();

  // every wave turns the per-wave counts into the K rows itself: lane j < K
  // sums target j's counts over the waves, and the rows become wave-uniform
  // by readlane, so no second barrier is needed
  const int lane = tid & (kWave - 1);
  const int j = lane < K ? lane : 0;
  int c = 0;  // packed: the entry's row; padded: its rank within the expert
#pragma unroll
  for (int ww = 0; ww < MAXT / kWave; ++ww) {
    const int cw = wc[ww * kMaxK + j];  // read for every wave slot (in the array), so the reads go out together
    c += ww < nw ? cw : 0;
  }
  const int key = tkey[j];
  float s = 1.0f;
  u32x4 q = a;
  if (FP8) q = quantize16_e4m3(a, a2, s);
  const bool valid = key < E;
  const int row = !padded ? (valid ? c : -1) : ((valid && c < cap) ? key * cap + c : -1);
  if (chunk == 0 && tid < K) {  // wave 0 of the token's first workgroup
    slot[p0 + tid] = row;
    if (!padded) src[c] = valid ? t : -1;  // masked entries take the rows after the valid ones
    else if (row >= 0) src[row] = t;
    if (recv_weight != nullptr && row >= 0) recv_weight[row] = wj;
  }
  constexpr int KR = KT > 0 ? KT : kMaxK;
  int rk[KR];
#pragma unroll
  for (int k = 0; k < KR; ++k) rk[k] = k < K ? __builtin_amdgcn_readlane(row, k) : -1;
  if (!active) return;

  const uint32_t G = static_cast<uint32_t>(H) / kGroup;
  const bool lead = (v & 7) == 0;  // one lane per group writes the scale
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    if (k >= K) break;
    const int r = rk[k];
    if (r < 0) continue;
    if (FP8) {
      reinterpret_cast<u32x4*>(static_cast<uint8_t*>(recv) + static_cast<size_t>(r) * H)[v] = q;
      if (lead) recv_scale[static_cast<size_t>(r) * G + (v >> 3)] = s;
    } else {
      reinterpret_cast<u32x4*>(static_cast<uint16_t*>(recv) + static_cast<size_t>(r) * H)[v] = q;
    }
  }
}

// Workgroup size.  Up to 2048 entries: 256 lanes, so even 128 tokens fill
// the chip (FP8 at hidden 7168: two workgroups per token, 257 in all).
// Beyond, the counting (n*K per workgroup) dominates, and a workgroup
// takes the whole token (its vectors rounded up to whole waves, at most
// 1024 lanes) so the ids are read and counted once per token.  Measured on
// MI355X, top-8, hidden 7168: token-sized workgroups take 7.2 against
// 6.4 us at 128 tokens, the same 9.0 us at 256, and 11.2 against 12.8 us
// at 384.
constexpr int kWideFromEntries = 2048;

int fused_threads(uint32_t vpt, int n) {
  if (n <= kWideFromEntries) return kMinThreads;
  const uint32_t lanes = (vpt + kWave - 1) / kWave * kWave;
  return static_cast<int>(lanes < kMinThreads ? kMinThreads : lanes > kMaxThreads ? kMaxThreads : lanes);
}

template <bool FP8, int NS, int MAXT, typename Idx>
void launch_fused(const Idx* idx, const uint16_t* x, const float* w, int32_t T, int32_t H, int32_t K,
                  int32_t E, int32_t cap, int bs, int32_t* counts, int32_t* offsets, int32_t* slot, int32_t* src,
                  void* recv, float* recv_scale, float* recv_weight, hipStream_t stream) {
  const uint32_t vpt = static_cast<uint32_t>(H) / (FP8 ? 16 : 8);
  const uint32_t nchunk = (vpt + bs - 1) / bs;
  const dim3 grid(1 + static_cast<uint32_t>(T) * nchunk), block(bs);
#define EP_FUSED(KV)                                                                                            \
  hipLaunchKernelGGL((layout_dispatch_kernel<KV, FP8, NS, MAXT, Idx>), grid, block, 0, stream, idx, x, w, T, H, K, E, cap, \
                     nchunk, bs, counts, offsets, slot, src, recv, recv_scale, recv_weight)
  switch (K) {
    case 1: EP_FUSED(1); break;
    case 2: EP_FUSED(2); break;
    case 4: EP_FUSED(4); break;
    case 6: EP_FUSED(6); break;
    case 8: EP_FUSED(8); break;
    default: EP_FUSED(0); break;
  }
#undef EP_FUSED
}

template <bool FP8, typename Idx>
void launch_fused_ns(const Idx* idx, const uint16_t* x, const float* w, int32_t T, int32_t H, int32_t K,
                     int32_t E, int32_t cap, int32_t* counts, int32_t* offsets, int32_t* slot, int32_t* src,
                     void* recv, float* recv_scale, float* recv_weight, hipStream_t stream) {
  static_assert(kFusedMaxEntries <= 12 * kMinThreads, "steps per lane");
  const int n = T * K;
  const int bs = fused_threads(static_cast<uint32_t>(H) / (FP8 ? 16 : 8), n);
  // steps per lane: n <= 3072 and bs >= 256, so at most 12
  const int steps = (n + bs - 1) / bs;
  if (bs == kMinThreads) {
    if (steps <= 4)
      launch_fused<FP8, 4, kMinThreads>(idx, x, w, T, H, K, E, cap, bs, counts, offsets, slot, src, recv, recv_scale,
                                        recv_weight, stream);
    else if (steps <= 8)
      launch_fused<FP8, 8, kMinThreads>(idx, x, w, T, H, K, E, cap, bs, counts, offsets, slot, src, recv, recv_scale,
                                        recv_weight, stream);
    else
      launch_fused<FP8, 12, kMinThreads>(idx, x, w, T, H, K, E, cap, bs, counts, offsets, slot, src, recv,
                                         recv_scale, recv_weight, stream);
  } else if (steps <= 4) {
    launch_fused<FP8, 4, kMaxThreads>(idx, x, w, T, H, K, E, cap, bs, counts, offsets, slot, src, recv, recv_scale,
                                      recv_weight, stream);
  } else if (steps <= 8) {
    launch_fused<FP8, 8, kMaxThreads>(idx, x, w, T, H, K, E, cap, bs, counts, offsets, slot, src, recv, recv_scale,
                                      recv_weight, stream);
  } else {
    launch_fused<FP8, 12, kMaxThreads>(idx, x, w, T, H, K, E, cap, bs, counts, offsets, slot, src, recv,
                                       recv_scale, recv_weight, stream);
  }
}

}  // namespace

template <typename Idx>
hipError_t launch_layout_dispatch(const Idx* topk_idx, const uint16_t* x, const float* topk_weights,
                                  int32_t num_tokens, int32_t hidden, int32_t top_k, int32_t num_experts,
                                  int32_t capacity, bool fp8, int32_t* counts, int32_t* offsets, int32_t* slot,
                                  int32_t* src, void* recv, float* recv_scale, float* recv_weight,
                                  void* workspace, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(num_tokens) * top_k;
  if (n > kFusedMaxEntries) {
    hipError_t e = hipSuccess;
    if (launch_layout_dispatch_chunked(topk_idx, x, topk_weights, num_tokens, hidden, top_k, num_experts, capacity,
                                       fp8, counts, offsets, slot, src, recv, recv_scale, recv_weight, stream, &e))
      return e;
    e = launch_layout(topk_idx, static_cast<int32_t>(n), top_k, num_experts, capacity, counts, offsets,
                                 slot, src, workspace, stream);
    if (e != hipSuccess) return e;
    return fp8 ? launch_dispatch_fp8(x, num_tokens, hidden, top_k, slot, topk_weights, static_cast<uint8_t*>(recv),
                                     recv_scale, recv_weight, stream)
               : launch_dispatch_bf16(x, num_tokens, hidden, top_k, slot, topk_weights,
                                      static_cast<uint16_t*>(recv), recv_weight, stream);
  }
  if (fp8)
    launch_fused_ns<true>(topk_idx, x, topk_weights, num_tokens, hidden, top_k, num_experts, capacity, counts,
                          offsets, slot, src, recv, recv_scale, recv_weight, stream);
  else
    launch_fused_ns<false>(topk_idx, x, topk_weights, num_tokens, hidden, top_k, num_experts, capacity, counts,
                           offsets, slot, src, recv, recv_scale, recv_weight, stream);
  return hipGetLastError();
}

template hipError_t launch_layout_dispatch<int32_t>(const int32_t*, const uint16_t*, const float*, int32_t, int32_t,
                                                    int32_t, int32_t, int32_t, bool, int32_t*, int32_t*, int32_t*,
                                                    int32_t*, void*, float*, float*, void*, hipStream_t);
template hipError_t launch_layout_dispatch<int64_t>(const int64_t*, const uint16_t*, const float*, int32_t, int32_t,
                                                    int32_t, int32_t, int32_t, bool, int32_t*, int32_t*, int32_t*,
                                                    int32_t*, void*, float*, float*, void*, hipStream_t);

}  // namespace ep
