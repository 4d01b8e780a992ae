// Layout and dispatch in one launch for mid-size batches (more entries than
// the decode kernel in fused.hip takes, up to the one-launch layout's
// limit; e.g. 4096 tokens x top-8).
//
// The pages' dispatch call takes the tokens with their routing and returns
// the received rows together with the handle ([P4 "使用示例 › MoE 训练中的
// 应用"]).  This kernel writes everything the layout kernels and the
// dispatch kernel write, bit for bit, in one launch.
//
// gfx950 design.  The one-launch layout (layout_chunk) already has every
// workgroup histogram all T*K ids, so a workgroup can find the rows of any
// chunk of consecutive entries on its own.  Here workgroup b owns the
// tokens b*tpb .. b*tpb+tpb-1: their K*tpb entries are its layout chunk,
// and it also dispatches those tokens.  The tokens' loads are spread over
// the steps of the histogram (which is bound by on-chip work), and once
// the chunk's rows are known (staged in LDS) the workgroup quantises (FP8)
// or copies (BF16) the tokens into its receive rows.  tpb is chosen so
// that there is one workgroup per CU: the histogram is then paid once per
// CU, and the dispatch stores still come from every CU.  Against the
// layout kernel followed by the dispatch kernel this saves the second
// launch and hides the layout's on-chip work under the token reads.

#include "ep_internal.h"
#include "layout_device.h"

namespace ep {
namespace {

// work items per thread, their token loads held in registers (two 16-byte
// loads per FP8 item, one per BF16 item: 64 and 56 VGPRs; 14 BF16 items
// hold 16 tokens of hidden 7168, and 16 would spill)
constexpr int max_items(bool fp8) { return fp8 ? 8 : 14; }
constexpr int kChunkMaxK = 64;  // one lane per row for the wavefront scale stores

// FP8: work item = (token, 16 channels) as in the dispatch kernel; BF16:
// (token, 8 channels).  NT: non-temporal token loads and scale stores; WS:
// wavefront scale stores (store_wave_scales).  Each thread holds the work
// items i*kThreads + tid, i < max_items(FP8), of its workgroup's tokens.
template <int NW, bool V4, typename Idx, bool FP8, bool NT, bool WS>
__global__ __launch_bounds__(NW * kWave) void layout_dispatch_chunked(
    const Idx* __restrict__ idx, const uint16_t* __restrict__ x, const float* __restrict__ w, int32_t T,
    int32_t H, int32_t K, int32_t E, int32_t cap, int32_t tpb, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot, int32_t* __restrict__ src, void* __restrict__ recv,
    float* __restrict__ recv_scale, float* __restrict__ recv_weight) {
  extern __shared__ uint64_t lds64[];
  constexpr int kThreads = NW * kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int tok0 = blockIdx.x * tpb;
  const int ntok = min(T - tok0, tpb);
  const int c0 = tok0 * K, c1 = c0 + ntok * K;
  const uint32_t vpt = static_cast<uint32_t>(H) / (FP8 ? 16 : 8);  // work items per token
  const uint32_t nitems = static_cast<uint32_t>(ntok) * vpt;
  const int nit = static_cast<int>((nitems + kThreads - 1) / kThreads);  // workgroup-uniform

  // Token loads: the item slots up to the workgroup's last item are
  // loaded, with no per-lane branch (slots past a lane's last item load a
  // copy of the workgroup's last item, from the cache, and store nothing).  Item 0 goes out once the ids are in, the others spread over
  // the steps of the histogram (one FP8 item or two BF16 items per step):
  // HBM takes the tokens no faster than it reads them, so loads issued all
  // at once stall their waves for the whole read, while loads spread over
  // the histogram keep HBM busy under the counting.
  constexpr int kItems = max_items(FP8);
  constexpr int kPerStep = FP8 ? 1 : 2;
  static_assert(kItems <= 1 + kPerStep * kChunkSteps, "every item load has a hook");
  u32x4 a[kItems], b[FP8 ? kItems : 1];
  auto load_item = [&](int i) {
    if (i >= nit) return;  // workgroup-uniform: no slot of this one holds an item
    const uint32_t item = min(static_cast<uint32_t>(i * kThreads + tid), nitems - 1);
    const uint32_t tl = item / vpt, v = item - tl * vpt;
    const u32x4* p = reinterpret_cast<const u32x4*>(x + static_cast<size_t>(tok0 + tl) * H) + (FP8 ? 2 * v : v);
    a[i] = load_token<NT>(p);
    if constexpr (FP8) b[i] = load_token<NT>(p + 1);
  };
  // 16 ids per thread at a time with int64 ids (8 loads, as with int32): the
  // token registers and 16 id loads would not fit in 128 VGPRs
  const int row = layout_chunk<NW, V4, Idx, true, sizeof(Idx) == 8 ? 16 : 32>(
      idx, T * K, K, E, cap, c0, c1, lds64, counts, offsets, slot, src, [&] { load_item(0); },
      [&](int u) {
#pragma unroll
        for (int j = 0; j < kPerStep; ++j)
          if (1 + kPerStep * u + j < kItems) load_item(1 + kPerStep * u + j);
      });

  int* rows = reinterpret_cast<int*>(reinterpret_cast<char*>(lds64) + chunk_lds_bytes(NW, E));  // [tpb*K]
  if (tid < c1 - c0) rows[tid] = row;
  __syncthreads();

  const uint32_t G = static_cast<uint32_t>(H) / kGroup;
  static_for<0, kItems>([&](auto ic_) {
    constexpr int i = decltype(ic_)::value;
    if (i >= nit) return;
    const uint32_t item = static_cast<uint32_t>(i * kThreads + tid);
    const bool active = item < nitems;  // with WS whole wavefronts only
    const uint32_t ic = active ? item : nitems - 1;
    const uint32_t tl = ic / vpt, v = ic - tl * vpt;
    const int* trow = rows + tl * K;
    const float* wrow = w != nullptr ? w + static_cast<size_t>(tok0 + tl) * K : nullptr;
    const bool want_w = recv_weight != nullptr && v == 0;
    if constexpr (FP8) {
      float s;
      const u32x4 q = quantize16_e4m3(a[i], b[i], s);
      int32_t rj = -1;  // WS: this lane's row for the scale stores
      if (WS && active && lane < K) rj = trow[lane];
      if (active) {
        const bool lead = (v & 7) == 0;  // one lane per group writes the scale
        uint8_t* out = static_cast<uint8_t*>(recv);
        for (int k = 0; k < K; ++k) {
          const int r = trow[k];
          if (r < 0) continue;
          reinterpret_cast<u32x4*>(out + static_cast<size_t>(r) * H)[v] = q;
          if (!WS && lead) {
            float* ps = recv_scale + static_cast<size_t>(r) * G + (v >> 3);
            if (NT) __builtin_nontemporal_store(s, ps); else *ps = s;
          }
          if (want_w) recv_weight[r] = wrow[k];
        }
      }
      if (WS) store_wave_scales<NT>(rj, s, v, G, recv_scale);
    } else {
      if (!active) return;
      uint16_t* out = static_cast<uint16_t*>(recv);
      for (int k = 0; k < K; ++k) {
        const int r = trow[k];
        if (r < 0) continue;
        reinterpret_cast<u32x4*>(out + static_cast<size_t>(r) * H)[v] = a[i];
        if (want_w) recv_weight[r] = wrow[k];
      }
    }
  });
}

// ---- the split form ---------------------------------------------------------
//
// The chunked kernel above spreads its token loads over the histogram, and
// every wavefront both counts and loads: a wave that issues more loads than
// the memory system takes at once stalls, and with it its share of the
// counting, so the layout outlasts the token read and HBM idles before the
// first store.  Here the roles are split inside each workgroup of 16 waves:
//  1. all waves load the T*K ids once and leave their keys in LDS as 16-bit
//     values (padded to a multiple of 8 with a key no entry has): the ids
//     go through the CU's load path before any token load queues in it;
//  2. every wave issues all of its token loads;
//  3. waves 0..3 (one per SIMD) do the whole layout from LDS, with no
//     global load left to wait for: the before/after histogram of every
//     key, the rank of the workgroup's own entries, the per-key merge, the
//     scan and the slot/src writes; they synchronise among themselves
//     through an LDS counter (the other waves take no part), with a bounded
//     spin;
//  4. the other waves, stalled at issue while HBM takes their loads, reach
//     a workgroup barrier once their loads are all issued;
//  5. every wave then quantises (FP8) or copies (BF16) its items into the
//     rows staged in LDS: the token reads come first, the receive-row
//     writes after, with the layout hidden under the reads.
// On MI355X at 4096 tokens x 7168, top-8, FP8: 51.9-52.2 us against
// 53.1-53.7 us for the chunked kernel (A/B in one process, bit-equal).
// Issuing the loads a few items ahead of the stores instead (so that reads
// and writes overlap after the layout) measured 53.2-53.9 us: HBM streams
// a run of reads followed by a run of writes faster than a mix of them.
// Outputs are bit-identical to the chunked kernel's (the same counts, the
// same ranks, the same stores).

constexpr int kSplitWaves = 16;
constexpr int kSplitThreads = kSplitWaves * kWave;                         // 1024
constexpr int kLayoutWaves = 4;                                            // one per SIMD
constexpr int kLayoutLanes = kLayoutWaves * kWave;                         // 256
constexpr int kSplitRankSteps = 4;                                         // own entries: up to 1024
constexpr int kSyncSpinLimit = 1 << 22;                                    // bounded wait, ~0.1 s

// LDS of the split kernel (bytes, 16-byte aligned pieces): lane masks and
// running counts of the layout waves, two histograms of kHistCopies copies
// of E+2 bins (bin E+1 takes the padding keys), the sync counter, the rows
// of the workgroup's entries, then the keys.
struct SplitLds {
  size_t lmask, cnt, before, after, ctr, rows, keys, total;
};

__host__ __device__ inline SplitLds split_lds(int R, int E, int nrows) {
  auto up16 = [](size_t v) { return (v + 15) / 16 * 16; };
  const size_t nk = static_cast<size_t>(E) + 1, nb = nk + 1;
  SplitLds l;
  l.lmask = 0;
  l.cnt = up16(l.lmask + kLayoutWaves * nk * 8);
  l.before = up16(l.cnt + kLayoutWaves * nk * 4);
  l.after = up16(l.before + kHistCopies * nb * 4);
  l.ctr = up16(l.after + kHistCopies * nb * 4);
  l.rows = up16(l.ctr + 4);
  l.keys = up16(l.rows + static_cast<size_t>(nrows) * 4);
  l.total = up16(l.keys + static_cast<size_t>((R + 7) / 8 * 8) * 2);
  return l;
}

// A barrier among the layout waves only: each arrives on an LDS counter
// and waits until all kLayoutWaves have arrived for the `target`-th time.
// The wait is bounded so that it always ends.
__device__ __forceinline__ void layout_waves_sync(int* ctr, int& target) {
  target += kLayoutWaves;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if ((threadIdx.x & (kWave - 1)) == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  for (int it = 0; it < kSyncSpinLimit; ++it) {
    if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Exclusive prefix sum of data[0..n) in LDS by wave 0 (as
// block_exclusive_scan, without the workgroup barrier).
template <int MAXPER>
__device__ inline void wave0_exclusive_scan(int* data, int n) {
  if (threadIdx.x >= kWave) return;
  const int lane = threadIdx.x;
  const int per = (n + kWave - 1) / kWave;
  const int beg = lane * per;
  int v[MAXPER];
  int local = 0;
#pragma unroll
  for (int i = 0; i < MAXPER; ++i) {
    v[i] = (i < per && beg + i < n) ? data[beg + i] : 0;
    local += v[i];
  }
  int run = wave_inclusive_scan(local) - local;
#pragma unroll
  for (int i = 0; i < MAXPER; ++i) {
    if (i < per && beg + i < n) data[beg + i] = run;
    run += v[i];
  }
}

// One work item: quantise (FP8) or copy (BF16) and store to the token's K
// rows (the chunked kernel's store step).  `active`: the item exists (with
// WS, whole wavefronts only).
template <bool FP8, bool NT, bool WS>
__device__ __forceinline__ void store_item(u32x4 a, u32x4 b, bool active, uint32_t tl, uint32_t v, int tok0,
                                           const int* rows, const float* __restrict__ w, int32_t H, int32_t K,
                                           void* __restrict__ recv, float* __restrict__ recv_scale,
                                           float* __restrict__ recv_weight) {
  const int lane = threadIdx.x & (kWave - 1);
  const int* trow = rows + tl * K;
  const float* wrow = w != nullptr ? w + static_cast<size_t>(tok0 + tl) * K : nullptr;
  const bool want_w = recv_weight != nullptr && v == 0;
  if constexpr (FP8) {
    const uint32_t G = static_cast<uint32_t>(H) / kGroup;
    float s;
    const u32x4 q = quantize16_e4m3(a, b, s);
    int32_t rj = -1;
    if (WS && active && lane < K) rj = trow[lane];
    if (active) {
      const bool lead = (v & 7) == 0;
      uint8_t* out = static_cast<uint8_t*>(recv);
      for (int k = 0; k < K; ++k) {
        const int r = trow[k];
        if (r < 0) continue;
        reinterpret_cast<u32x4*>(out + static_cast<size_t>(r) * H)[v] = q;
        if (!WS && lead) {
          float* ps = recv_scale + static_cast<size_t>(r) * G + (v >> 3);
          if (NT) __builtin_nontemporal_store(s, ps); else *ps = s;
        }
        if (want_w) recv_weight[r] = wrow[k];
      }
    }
    if (WS) store_wave_scales<NT>(rj, s, v, G, recv_scale);
  } else {
    if (!active) return;
    uint16_t* out = static_cast<uint16_t*>(recv);
    for (int k = 0; k < K; ++k) {
      const int r = trow[k];
      if (r < 0) continue;
      reinterpret_cast<u32x4*>(out + static_cast<size_t>(r) * H)[v] = a;
      if (want_w) recv_weight[r] = wrow[k];
    }
  }
}

// V4: ids aligned to 16 bytes.  Workgroup b owns tokens b*tpb ..; tpb*K is
// a multiple of 8, so a group of 8 keys lies wholly before or at/after the
// workgroup's entries.  NI: work items per lane (item i*1024 + tid); every
// lane issues exactly NI token loads, none under a condition (a slot past
// the last item reloads that item and stores nothing), and the layout
// waves' loads and the others' come from one place: loads under a
// condition, or in two branches, make the compiler wait for them before
// the layout.
template <bool V4, typename Idx, bool FP8, bool NT, bool WS, int NI>
__global__ __launch_bounds__(kSplitThreads) void layout_dispatch_split(
    const Idx* __restrict__ idx, const uint16_t* __restrict__ x, const float* __restrict__ w, int32_t T,
    int32_t H, int32_t K, int32_t E, int32_t cap, int32_t tpb, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot, int32_t* __restrict__ src, void* __restrict__ recv,
    float* __restrict__ recv_scale, float* __restrict__ recv_weight) {
  extern __shared__ uint64_t lds64[];
  constexpr int kThreads = kSplitThreads;
  const int tid = threadIdx.x, wv = tid / kWave, lane = tid & (kWave - 1);
  const int R = T * K;
  const int nk = E + 1, nb = E + 2;
  const int tok0 = blockIdx.x * tpb;
  const int ntok = min(T - tok0, tpb);
  const int c0 = tok0 * K, c1 = c0 + ntok * K;
  const SplitLds L = split_lds(R, E, tpb * K);
  char* base = reinterpret_cast<char*>(lds64);
  uint64_t* lmask = reinterpret_cast<uint64_t*>(base + L.lmask);
  int* cnt = reinterpret_cast<int*>(base + L.cnt);
  int* before = reinterpret_cast<int*>(base + L.before);
  int* after = reinterpret_cast<int*>(base + L.after);
  int* ctr = reinterpret_cast<int*>(base + L.ctr);
  int* rows = reinterpret_cast<int*>(base + L.rows);
  uint16_t* keys = reinterpret_cast<uint16_t*>(base + L.keys);
  const int Rpad = (R + 7) / 8 * 8;

  // 1. every id -> its key in LDS; clear the layout's LDS
  for (int i = tid; i < kLayoutWaves * nk; i += kThreads) {
    lmask[i] = 0;
    cnt[i] = 0;
  }
  for (int i = tid; i < kHistCopies * nb; i += kThreads) {
    before[i] = 0;
    after[i] = 0;
  }
  if (tid == 0) *ctr = 0;
  int done = 0;  // ids converted by the vector loads
  if constexpr (V4) {
    constexpr int kPer = 16 / static_cast<int>(sizeof(Idx));
    constexpr int kBatch = 8;
    const int n4 = R / kPer;
    const int4* idx4 = reinterpret_cast<const int4*>(idx);
    for (int q0 = 0; q0 < n4; q0 += kThreads * kBatch) {
      int4 e[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) e[u] = idx4[min(q0 + u * kThreads + tid, n4 - 1)];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int q = q0 + u * kThreads + tid;
        if (q >= n4) continue;
        int k4[kPer];
        expert_keys16<Idx>(e[u], E, k4);
        if constexpr (kPer == 4) {
          reinterpret_cast<uint2*>(keys)[q] = make_uint2(static_cast<uint32_t>(k4[0]) | (static_cast<uint32_t>(k4[1]) << 16),
                                                         static_cast<uint32_t>(k4[2]) | (static_cast<uint32_t>(k4[3]) << 16));
        } else {
          reinterpret_cast<uint32_t*>(keys)[q] = static_cast<uint32_t>(k4[0]) | (static_cast<uint32_t>(k4[1]) << 16);
        }
      }
    }
    done = n4 * kPer;
  }
  for (int p = done + tid; p < Rpad; p += kThreads) keys[p] = static_cast<uint16_t>(p < R ? expert_key(idx[p], E) : E + 1);
  __syncthreads();

  const uint32_t vpt = static_cast<uint32_t>(H) / (FP8 ? 16 : 8);
  const uint32_t nitems = static_cast<uint32_t>(ntok) * vpt;
  const bool is_layout = wv < kLayoutWaves;
  u32x4 a[NI], b[FP8 ? NI : 1];
  auto load_item = [&](int i) {
    const uint32_t item = min(static_cast<uint32_t>(i * kThreads + tid), nitems - 1);
    const uint32_t tl = item / vpt, v = item - tl * vpt;
    const u32x4* px = reinterpret_cast<const u32x4*>(x + static_cast<size_t>(tok0 + tl) * H) + (FP8 ? 2 * v : v);
    a[i] = load_token<NT>(px);
    if constexpr (FP8) b[i] = load_token<NT>(px + 1);
  };
  // 2. every token load of this lane
  static_for<0, NI>([&](auto ic) { load_item(decltype(ic)::value); });
  if (is_layout) {
    // 3. the layout, by the layout waves alone
    int target = 0;
    const int copy = (lane & (kHistCopies - 1)) * nb;
    int* const hb = before + copy;
    int* const ha = after + copy;
    const int ng = Rpad / 8;
    for (int g = tid; g < ng; g += kLayoutLanes) {
      const uint4 kk = reinterpret_cast<const uint4*>(keys)[g];
      int* const h = 8 * g < c0 ? hb : ha;
      atomicAdd(&h[kk.x & 0xFFFF], 1);
      atomicAdd(&h[kk.x >> 16], 1);
      atomicAdd(&h[kk.y & 0xFFFF], 1);
      atomicAdd(&h[kk.y >> 16], 1);
      atomicAdd(&h[kk.z & 0xFFFF], 1);
      atomicAdd(&h[kk.z >> 16], 1);
      atomicAdd(&h[kk.w & 0xFFFF], 1);
      atomicAdd(&h[kk.w >> 16], 1);
    }
    // rank the workgroup's own entries: wave wv takes entries c0 + 256*wv ..
    const int p_begin = c0 + wv * kWave * kSplitRankSteps;
    const int p_end = min(c1, p_begin + kWave * kSplitRankSteps);
    int e[kSplitRankSteps], key[kSplitRankSteps], rank[kSplitRankSteps];
#pragma unroll
    for (int i = 0; i < kSplitRankSteps; ++i) {
      const int p = p_begin + i * kWave + lane;
      e[i] = p < p_end ? static_cast<int>(keys[p]) : E;
    }
    rank_wave_keys<kSplitRankSteps>(e, p_begin, p_end, lmask + wv * nk, cnt + wv * nk, key, rank);
    layout_waves_sync(ctr, target);
    for (int j = tid; j < nk; j += kLayoutLanes) {
      int run = 0;
#pragma unroll
      for (int ww = 0; ww < kLayoutWaves; ++ww) {
        const int c = cnt[ww * nk + j];
        cnt[ww * nk + j] = run;
        run += c;
      }
      int bs = 0, as = 0;
#pragma unroll
      for (int cp = 0; cp < kHistCopies; ++cp) {
        bs += before[cp * nb + j];
        as += after[cp * nb + j];
      }
      before[j] = bs;
      after[j] = bs + as;  // total
    }
    layout_waves_sync(ctr, target);
    if (nk <= 5 * kWave) wave0_exclusive_scan<5>(after, nk);
    else if (nk <= 9 * kWave) wave0_exclusive_scan<9>(after, nk);
    else wave0_exclusive_scan<17>(after, nk);
    layout_waves_sync(ctr, target);
    if (blockIdx.x == 0) {
      for (int j = tid; j < E; j += kLayoutLanes) {
        const int total = after[j + 1] - after[j];
        counts[j] = cap == 0 ? total : min(total, cap);
      }
      if (cap == 0)
        for (int j = tid; j <= E; j += kLayoutLanes) offsets[j] = after[j];
    }
#pragma unroll
    for (int i = 0; i < kSplitRankSteps; ++i) {
      const int k = key[i];
      if (k < 0) continue;
      const int p = p_begin + i * kWave + lane;
      rows[p - c0] = write_entry(p, k, before[k] + cnt[wv * nk + k] + rank[i], after, E, K, cap, slot, src);
    }
  }
  // 4. the other waves wait here once their loads are all issued
  __syncthreads();

  // 5. quantise / copy and store
  static_for<0, NI>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const uint32_t item = static_cast<uint32_t>(i * kThreads + tid);
    const bool active = item < nitems;  // with WS whole wavefronts only
    const uint32_t ic2 = active ? item : nitems - 1;
    const uint32_t tl = ic2 / vpt, v = ic2 - tl * vpt;
    store_item<FP8, NT, WS>(a[i], FP8 ? b[FP8 ? i : 0] : a[i], active, tl, v, tok0, rows, w, H, K, recv, recv_scale,
                            recv_weight);
  });
}

// The split kernel where its limits hold: 16-byte aligned ids, tpb*K a
// multiple of 8 and at most 1024, every lane's item slots filled but its
// last (7 or 8 FP8, 13 or 14 BF16 items per lane: the large batches, e.g.
// 4096 tokens of hidden 7168, where the layout would otherwise hold up the
// token stream), and the keys plus the layout within the LDS.  Returns
// false, launching nothing, otherwise.
template <typename Idx>
bool launch_layout_dispatch_split(const Idx* topk_idx, const uint16_t* x, const float* topk_weights, int32_t T,
                                  int32_t H, int32_t K, int32_t E, int32_t capacity, bool fp8, int32_t* counts,
                                  int32_t* offsets, int32_t* slot, int32_t* src, void* recv, float* recv_scale,
                                  float* recv_weight, hipStream_t stream, hipError_t* err) {
  if ((reinterpret_cast<uintptr_t>(topk_idx) & 15) != 0) return false;
  const int cus = device_cu_count();
  if (cus <= 0) return false;
  int step = 1;
  while ((step * K) % 8 != 0) ++step;
  int tpb = (T + cus - 1) / cus;
  tpb = (tpb + step - 1) / step * step;
  if (tpb * K > kLayoutLanes * kSplitRankSteps) return false;
  const int vpt = H / (fp8 ? 16 : 8);
  const int64_t nslots = (static_cast<int64_t>(tpb) * vpt + kSplitThreads - 1) / kSplitThreads;
  const int ni_max = fp8 ? 8 : 14;
  if (nslots < ni_max - 1 || nslots > ni_max) return false;
  const SplitLds L = split_lds(T * K, E, tpb * K);
  if (L.total > kLdsLimit) return false;
  const bool nt = static_cast<size_t>(T) * H * 2 >= kStreamingTokenBytes;
  const bool ws = fp8 && vpt % kWave == 0 && (H / kGroup) % 4 == 0 &&
                  (reinterpret_cast<uintptr_t>(recv_scale) & 15) == 0;
  const dim3 grid((T + tpb - 1) / tpb), block(kSplitThreads);
#define EP_SPLIT(F, NTV, WSV, NIV)                                                                                 \
  hipLaunchKernelGGL((layout_dispatch_split<true, Idx, F, NTV, WSV, NIV>), grid, block, L.total, stream, topk_idx, \
                     x, topk_weights, T, H, K, E, capacity, tpb, counts, offsets, slot, src, recv, recv_scale,     \
                     recv_weight)
#define EP_SPLIT_NI(F, NTV, WSV, NIMAX) \
  if (nslots == NIMAX) EP_SPLIT(F, NTV, WSV, NIMAX); else EP_SPLIT(F, NTV, WSV, NIMAX - 1)
  if (fp8) {
    if (nt) {
      if (ws) EP_SPLIT_NI(true, true, true, 8); else EP_SPLIT_NI(true, true, false, 8);
    } else {
      if (ws) EP_SPLIT_NI(true, false, true, 8); else EP_SPLIT_NI(true, false, false, 8);
    }
  } else {
    if (nt) EP_SPLIT_NI(false, true, false, 14); else EP_SPLIT_NI(false, false, false, 14);
  }
#undef EP_SPLIT_NI
#undef EP_SPLIT
  *err = hipGetLastError();
  return true;
}

}  // namespace

template <typename Idx>
bool launch_layout_dispatch_chunked(const Idx* topk_idx, const uint16_t* x, const float* topk_weights,
                                    int32_t T, int32_t H, int32_t K, int32_t E, int32_t capacity, bool fp8,
                                    int32_t* counts, int32_t* offsets, int32_t* slot, int32_t* src, void* recv,
                                    float* recv_scale, float* recv_weight, hipStream_t stream, hipError_t* err) {
  const int64_t n = static_cast<int64_t>(T) * K;
  if (n <= kFusedMaxEntries || n > kOneLaunchMaxEntries || K > kChunkMaxK) return false;
  if (launch_layout_dispatch_split(topk_idx, x, topk_weights, T, H, K, E, capacity, fp8, counts, offsets, slot, src,
                                   recv, recv_scale, recv_weight, stream, err))
    return true;
  const int nw = chunk_waves(E);
  if (nw < 8) return false;
  const int threads = nw * kWave;
  const int vpt = H / (fp8 ? 16 : 8);
  // 16-byte id loads need chunk starts on 16 bytes: tpb*K a multiple of 4 ids
  // (int32) or 2 (int64)
  const bool v4 = (reinterpret_cast<uintptr_t>(topk_idx) & 15) == 0;
  const int per16 = 16 / static_cast<int>(sizeof(Idx));
  int step = 1;
  while (v4 && (step * K) % per16 != 0) ++step;
  const int cus = device_cu_count();  // one workgroup per CU
  if (cus <= 0) return false;
  int tpb = (T + cus - 1) / cus;
  tpb = (tpb + step - 1) / step * step;
  if (tpb * K > threads || static_cast<int64_t>(tpb) * vpt > static_cast<int64_t>(max_items(fp8)) * threads)
    return false;
  const size_t lds = chunk_lds_bytes(nw, E) + static_cast<size_t>(tpb) * K * sizeof(int);
  if (lds > kLdsLimit) return false;
  const bool nt = static_cast<size_t>(T) * H * 2 >= kStreamingTokenBytes;
  // wavefront scale stores: wavefronts inside one token, 16-byte pieces
  const bool ws = fp8 && vpt % kWave == 0 && (H / kGroup) % 4 == 0 &&
                  (reinterpret_cast<uintptr_t>(recv_scale) & 15) == 0;
  const dim3 grid((T + tpb - 1) / tpb), block(threads);
#define EP_CHUNKED(NW, V, F, NTV, WSV)                                                                          \
  hipLaunchKernelGGL((layout_dispatch_chunked<NW, V, Idx, F, NTV, WSV>), grid, block, lds, stream, topk_idx, x, \
                     topk_weights, T, H, K, E, capacity, tpb, counts, offsets, slot, src, recv, recv_scale,     \
                     recv_weight)
#define EP_CHUNKED_NW(NW, V)                                        \
  if (fp8) {                                                        \
    if (nt) {                                                       \
      if (ws) EP_CHUNKED(NW, V, true, true, true); else EP_CHUNKED(NW, V, true, true, false);   \
    } else {                                                        \
      if (ws) EP_CHUNKED(NW, V, true, false, true); else EP_CHUNKED(NW, V, true, false, false); \
    }                                                               \
  } else {                                                          \
    if (nt) EP_CHUNKED(NW, V, false, true, false); else EP_CHUNKED(NW, V, false, false, false); \
  }
  if (nw >= 16) {
    if (v4) { EP_CHUNKED_NW(16, true) } else { EP_CHUNKED_NW(16, false) }
  } else {
    if (v4) { EP_CHUNKED_NW(8, true) } else { EP_CHUNKED_NW(8, false) }
  }
#undef EP_CHUNKED_NW
#undef EP_CHUNKED
  *err = hipGetLastError();
  return true;
}

template bool launch_layout_dispatch_chunked<int32_t>(const int32_t*, const uint16_t*, const float*, int32_t,
                                                      int32_t, int32_t, int32_t, int32_t, bool, int32_t*, int32_t*,
                                                      int32_t*, int32_t*, void*, float*, float*, hipStream_t,
                                                      hipError_t*);
template bool launch_layout_dispatch_chunked<int64_t>(const int64_t*, const uint16_t*, const float*, int32_t,
                                                      int32_t, int32_t, int32_t, int32_t, bool, int32_t*, int32_t*,
                                                      int32_t*, int32_t*, void*, float*, float*, hipStream_t,
                                                      hipError_t*);

}  // namespace ep
