// Dispatch layout: per-expert counts, exclusive-scan offsets, and the stable
// (ascending token, then k) receive row of every (token, k) entry.
//
// Definition (the handle of the pages' dispatch call, [P4 "使用示例 › MoE
// 训练中的应用"], with the in-expert order fixed to ascending (t, k)):
//   slot[t,k] = offset[e] + #{(t',k') before (t,k) with the same expert e}.
//
// gfx950 design.  Entries are taken in (t, k) order, 64 per wavefront step.
// CDNA has no match instruction, so equal keys inside a step are found
// through LDS: each lane ORs its lane bit into a per-wave lane-mask slot for
// its key and reads the slot back.  A lane's rank among equal keys is the
// popcount of the matching lanes below it (mbcnt) plus a per-wave running
// count, which the lowest matching lane advances.  Masked entries (expert
// outside [0, E)) use the extra key E, so they sort behind every real row
// and slot/src stay a bijection over all T*K entries.  Per-wave counts are
// scanned across waves per key, and the per-key totals across keys for the
// offsets.  Only order-free operations (OR, integer add) meet at one
// address, so every output is a pure function of topk_idx.
//
// The same kernels build the low-latency padded layout when given a
// capacity: expert e then owns rows e*capacity.., an entry's row is
// e*capacity + its rank, and entries ranked past the capacity are dropped
// ([P4 "使用示例 › 推理解码阶段的应用"]: a buffer of num_max_tokens rows per
// expert and a per-expert received count).
//
// Three launch shapes, chosen by T*K:
//  * up to 1024 entries: `layout_single`, one workgroup does everything;
//  * up to 65536: `layout_fused`, one launch of 1024-entry chunks (512
//    with 1024 experts) in which every workgroup also histograms all
//    entries, so no cross-workgroup exchange (and no workspace) is needed;
//  * beyond: `layout_count` ranks 4096-entry chunks and writes per-chunk
//    histograms to the workspace, then `layout_finalize` sums the
//    histograms of earlier chunks per key (16 loads in flight per thread),
//    scans the totals over keys and writes the rows.

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kSingleMaxWaves = 8;  // the single-workgroup path launches at most 8 waves
constexpr int kSingleMaxThreads = kSingleMaxWaves * 64;
constexpr int kSingleMaxEntries = 1024;  // one workgroup, no workspace
constexpr int kOneLaunchMaxEntries = 65536;  // one launch, no workspace
constexpr int kMultiThreads = 256;
constexpr int kMultiWaves = kMultiThreads / kWave;
constexpr int kHistCopies = 4;  // one-launch layout: private histograms per lane & 3

// The keys of this wavefront's entries p_begin + 64*i + lane (E past
// p_end), loaded apart from the ranking so that a caller can issue the
// loads early.
template <int ITERS, typename Idx>
__device__ __forceinline__ void load_wave_keys(const Idx* __restrict__ idx, int p_begin, int p_end, int E,
                                               int (&e)[ITERS]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const int p = p_begin + i * kWave + lane;
    e[i] = p < p_end ? expert_key(idx[p], E) : E;
  }
}

// Rank ITERS consecutive 64-entry steps of this wavefront: entries
// [p_begin, p_end) with keys e (from load_wave_keys).  lmask (E+1 lane
// masks, all zero on entry and on exit) and cnt (E+1 running counts) are
// this wave's LDS rows.  On return key[i] is the entry's key (E for masked,
// -1 past p_end) and rank[i] its position among the wave's entries with
// that key.
//
// Per step every in-range lane ORs its lane bit into lmask[key]; reading
// lmask[key] back gives the set of lanes holding the same key (OR is
// order-free, so the result is deterministic).  The rank is the number of
// those lanes below this one plus the running count; the lowest such lane
// advances the count and clears the mask.  LDS operations of one wavefront
// execute in program order, which is all the step relies on.
template <int ITERS>
__device__ __forceinline__ void rank_wave_keys(const int (&e)[ITERS], int p_begin, int p_end, uint64_t* lmask,
                                               int* cnt, int (&key)[ITERS], int (&rank)[ITERS]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    if (p_begin + i * kWave >= p_end) {  // wave-uniform: nothing left
      key[i] = -1;
      rank[i] = 0;
      continue;
    }
    const int p = p_begin + i * kWave + lane;
    const bool inr = p < p_end;
    const int k = e[i];
    if (inr) __hip_atomic_fetch_or(&lmask[k], 1ull << lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
    __builtin_amdgcn_wave_barrier();
    const uint64_t same = inr ? __hip_atomic_load(&lmask[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT) : 0ull;
    const int below = static_cast<int>(lanes_below(same));
    const int pre = inr ? cnt[k] : 0;
    __builtin_amdgcn_wave_barrier();
    if (inr && below == 0) {
      cnt[k] = pre + static_cast<int>(__popcll(same));
      __hip_atomic_store(&lmask[k], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
    }
    __builtin_amdgcn_wave_barrier();
    key[i] = inr ? k : -1;
    rank[i] = pre + below;
  }
}

// load_wave_keys then rank_wave_keys
template <int ITERS, typename Idx>
__device__ __forceinline__ void rank_wave_range(const Idx* __restrict__ idx, int p_begin, int p_end,
                                                int E, uint64_t* lmask, int* cnt, int (&key)[ITERS],
                                                int (&rank)[ITERS]) {
  int e[ITERS];
  load_wave_keys<ITERS>(idx, p_begin, p_end, E, e);
  rank_wave_keys<ITERS>(e, p_begin, p_end, lmask, cnt, key, rank);
}

// Row of one entry whose rank among the entries of its key is `within`.
// Packed layout (cap == 0): row off[k] + within; masked entries (k == E)
// take the rows after the valid ones with src = -1.  Padded layout
// (cap > 0): expert e owns rows e*cap .. e*cap+cap-1; entries ranked past
// the capacity and masked entries get slot -1 and no row, and the unused
// rows of an expert's block are not written.
__device__ __forceinline__ void write_entry(int p, int k, int within, const int* off, int E, int K, int cap,
                                            int32_t* __restrict__ slot, int32_t* __restrict__ src) {
  const bool valid = k < E;
  const int t = valid ? static_cast<int>(static_cast<uint32_t>(p) / static_cast<uint32_t>(K)) : -1;
  if (cap == 0) {
    const int pos = off[k] + within;
    slot[p] = valid ? pos : -1;
    src[pos] = t;
  } else {
    const bool keep = valid && within < cap;
    slot[p] = keep ? k * cap + within : -1;
    if (keep) src[k * cap + within] = t;
  }
}

// Counts and offsets from the exclusive scan `off` of the per-key totals
// (written by one workgroup); in the padded layout the count is clamped to
// the capacity and there are no offsets.
__device__ __forceinline__ void write_counts(const int* off, int E, int cap, int part, int32_t* __restrict__ counts,
                                             int32_t* __restrict__ offsets) {
  if (part != 0) return;
  const int tid = threadIdx.x, bs = blockDim.x;
  for (int j = tid; j < E; j += bs) {
    const int total = off[j + 1] - off[j];
    counts[j] = cap == 0 ? total : min(total, cap);
  }
  if (cap == 0)
    for (int j = tid; j <= E; j += bs) offsets[j] = off[j];
}

template <int ITERS, typename Idx>
__global__ __launch_bounds__(kSingleMaxThreads) void layout_single(
    const Idx* __restrict__ idx, int32_t R, int32_t K, int32_t E, int32_t cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot, int32_t* __restrict__ src) {
  extern __shared__ uint64_t lds64[];
  const int tid = threadIdx.x, bs = blockDim.x, nw = bs / kWave, w = tid / kWave;
  const int nk = E + 1;
  uint64_t* lmask = lds64;                                // [nw][nk]
  int* cnt = reinterpret_cast<int*>(lmask + nw * nk);     // [nw][nk]
  int* off = cnt + nw * nk;                               // [nk]
  for (int i = tid; i < nw * nk; i += bs) {
    lmask[i] = 0;
    cnt[i] = 0;
  }
  __syncthreads();

  const int per = ((R + nw - 1) / nw + kWave - 1) / kWave * kWave;
  const int p_begin = w * per;
  const int p_end = min(R, p_begin + per);
  int key[ITERS], rank[ITERS];
  rank_wave_range<ITERS>(idx, p_begin, p_end, E, lmask + w * nk, cnt + w * nk, key, rank);
  __syncthreads();

  for (int j = tid; j < nk; j += bs) {
    int run = 0;
    for (int ww = 0; ww < nw; ++ww) {
      const int c = cnt[ww * nk + j];
      cnt[ww * nk + j] = run;
      run += c;
    }
    off[j] = run;
  }
  __syncthreads();
  block_exclusive_scan(off, nk);
  write_counts(off, E, cap, 0, counts, offsets);

  const int lane = tid & (kWave - 1);
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const int k = key[i];
    if (k >= 0) write_entry(p_begin + i * kWave + lane, k, cnt[w * nk + k] + rank[i], off, E, K, cap, slot, src);
  }
}

template <int ITERS, typename Idx>
__global__ __launch_bounds__(kMultiThreads) void layout_count(const Idx* __restrict__ idx, int32_t R,
                                                              int32_t E, int32_t* __restrict__ slot_tmp,
                                                              int32_t* __restrict__ hist) {
  extern __shared__ uint64_t lds64[];
  const int tid = threadIdx.x, w = tid / kWave, lane = tid & (kWave - 1);
  const int nk = E + 1;
  uint64_t* lmask = lds64;                                   // [kMultiWaves][nk]
  int* cnt = reinterpret_cast<int*>(lmask + kMultiWaves * nk);  // [kMultiWaves][nk]
  for (int i = tid; i < kMultiWaves * nk; i += kMultiThreads) {
    lmask[i] = 0;
    cnt[i] = 0;
  }
  __syncthreads();

  constexpr int kChunk = kMultiThreads * ITERS;
  const int p_begin = blockIdx.x * kChunk + w * (kWave * ITERS);
  const int p_end = min(R, p_begin + kWave * ITERS);
  int key[ITERS], rank[ITERS];
  rank_wave_range<ITERS>(idx, p_begin, p_end, E, lmask + w * nk, cnt + w * nk, key, rank);
  __syncthreads();

  for (int j = tid; j < nk; j += kMultiThreads) {
    int run = 0;
#pragma unroll
    for (int ww = 0; ww < kMultiWaves; ++ww) {
      const int c = cnt[ww * nk + j];
      cnt[ww * nk + j] = run;
      run += c;
    }
    hist[static_cast<size_t>(blockIdx.x) * nk + j] = run;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const int p = p_begin + i * kWave + lane;
    if (key[i] >= 0) slot_tmp[p] = cnt[w * nk + key[i]] + rank[i];
  }
}

template <int ITERS, typename Idx>
__global__ __launch_bounds__(kMultiThreads) void layout_finalize(
    const Idx* __restrict__ idx, int32_t R, int32_t K, int32_t E, int32_t cap, int32_t nblocks,
    const int32_t* __restrict__ hist, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot, int32_t* __restrict__ src) {
  extern __shared__ int lds[];
  const int tid = threadIdx.x;
  const int nk = E + 1;
  int* base = lds;            // [nk] rows of this key in earlier chunks
  int* off = lds + nk;        // [nk] totals, then offsets
  const int b = blockIdx.x;
  constexpr int kChunk = kMultiThreads * ITERS;

  // this chunk's entries and their in-chunk ranks, loaded up front so the
  // latency overlaps the histogram loads below
  int e[ITERS], loc[ITERS];  // keys, in-chunk ranks
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const int p = b * kChunk + i * kMultiThreads + tid;
    e[i] = p < R ? expert_key(idx[p], E) : E;
    loc[i] = p < R ? slot[p] : 0;
  }

  constexpr int kBatch = 16;  // independent histogram loads in flight per thread
  for (int j = tid; j < nk; j += kMultiThreads) {
    int before = 0, total = 0;
    for (int bb = 0; bb < nblocks; bb += kBatch) {
      int h[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        h[u] = bb + u < nblocks ? hist[static_cast<size_t>(bb + u) * nk + j] : 0;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        total += h[u];
        before += bb + u < b ? h[u] : 0;
      }
    }
    base[j] = before;
    off[j] = total;
  }
  __syncthreads();
  block_exclusive_scan(off, nk);
  write_counts(off, E, cap, b, counts, offsets);

#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const int p = b * kChunk + i * kMultiThreads + tid;
    if (p < R) write_entry(p, e[i], base[e[i]] + loc[i], off, E, K, cap, slot, src);
  }
}

// One launch for the whole layout.  Block b owns the chunk of NW*64
// consecutive entries starting at b*NW*64 (one 64-entry step per wave) and
// ranks it as above; it also histograms all T*K entries with LDS atomic
// adds (integer addition is order-free, so the counts are exact and
// deterministic): entries before its chunk into `before`, the rest, its
// chunk included, into `after`.  Then for every key: total = before +
// after, offsets are the exclusive scan of the totals, and an entry's row
// is offset + before + (own-chunk rank).  Every block reads all T*K ids
// (from L2 after the first), which trades redundant on-chip work for the
// second launch and the workspace.  Everything in the histogram step is
// paid once per entry (32 per lane at 32768 entries), so it spends one LDS
// atomic and its address per entry: which histogram takes a load's ids is
// one block-uniform comparison per 16-byte load, and lanes spread over
// kHistCopies private copies so that a hot expert's entries in one wave
// collide on fewer addresses.  All blocks walk the ids in the same
// order: one L2 miss per XCD then serves every block on it (a per-block
// rotated start measured 1.7x slower with int64 ids).
// V4: 16-byte id loads (ids aligned to 16 bytes): 4 int32 or 2 int64 ids each.
template <int NW, bool V4, typename Idx>
__global__ __launch_bounds__(NW * kWave) void layout_fused(
    const Idx* __restrict__ idx, int32_t R, int32_t K, int32_t E, int32_t cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot, int32_t* __restrict__ src) {
  extern __shared__ uint64_t lds64[];
  constexpr int kThreads = NW * kWave;
  const int tid = threadIdx.x, w = tid / kWave, lane = tid & (kWave - 1);
  const int nk = E + 1;
  uint64_t* lmask = lds64;                             // [NW][nk]
  int* cnt = reinterpret_cast<int*>(lmask + NW * nk);  // [NW][nk]
  int* before = cnt + NW * nk;                         // [kHistCopies][nk], merged into copy 0
  int* after = before + kHistCopies * nk;              // [kHistCopies][nk], copy 0 later totals and offsets
  // clear the lane masks, running counts and histograms (callers sync)
  auto clear_lds = [&]() {
    for (int i = tid; i < NW * nk; i += kThreads) {
      lmask[i] = 0;
      cnt[i] = 0;
    }
    for (int i = tid; i < kHistCopies * nk; i += kThreads) {
      before[i] = 0;
      after[i] = 0;
    }
  };

  const int c0 = blockIdx.x * kThreads;
  const int c1 = min(R, c0 + kThreads);
  // Histogram every entry: those before this block's chunk into `before`,
  // the rest (the chunk itself included) into `after`, so the per-key total
  // is before + after.  Lanes spread over kHistCopies private copies, so
  // entries of one hot expert in one wave collide on fewer LDS addresses.
  // this wave's 64 entries of the chunk, ranked after the histogram; their
  // keys are loaded with the first batch of ids
  const int p_begin = c0 + w * kWave, p_stop = min(c1, p_begin + kWave);
  int own[1];
  const int copy = (lane & (kHistCopies - 1)) * nk;
  int* const hb = before + copy;
  int* const ha = after + copy;
  if constexpr (V4) {
    // 16-byte loads of kPer ids each, 32 ids in flight per thread.  c0 is
    // a multiple of the chunk size and so of kPer: each load lies wholly
    // before or wholly at/after c0 (one block-uniform comparison per load),
    // and the last R % kPer ids all lie at or after c0
    constexpr int kPer = 16 / static_cast<int>(sizeof(Idx));
    constexpr int kUnroll = 32 / kPer;
    const int4* idx4 = reinterpret_cast<const int4*>(idx);
    const int n4 = R / kPer, qb = c0 / kPer;
    int4 e[kUnroll];
    auto load_batch = [&](int q0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int q = q0 + u * kThreads + tid;
        e[u] = q < n4 ? idx4[q] : make_int4(0, 0, 0, 0);
      }
    };
    // the first batch is loaded before the LDS is cleared, so the loads'
    // latency overlaps the clearing and the waves' start (at 32768 int32 or
    // int64 ids one batch is all of them); the empty asm keeps the compiler
    // from sinking the loads below the clearing
    load_batch(0);
    load_wave_keys<1>(idx, p_begin, p_stop, E, own);
    asm volatile("" ::: "memory");
    clear_lds();
    __syncthreads();
    for (int q0 = 0;;) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int q = q0 + u * kThreads + tid;
        if (q >= n4) continue;
        int* const h = q < qb ? hb : ha;
        int k4[kPer];
        expert_keys16<Idx>(e[u], E, k4);
#pragma unroll
        for (int j = 0; j < kPer; ++j) atomicAdd(&h[k4[j]], 1);
      }
      q0 += kThreads * kUnroll;
      if (q0 >= n4) break;
      load_batch(q0);
    }
    const int p = kPer * n4 + tid;  // the last R % kPer ids
    if (p < R) atomicAdd(&ha[expert_key(idx[p], E)], 1);
  } else {
    load_wave_keys<1>(idx, p_begin, p_stop, E, own);
    clear_lds();
    __syncthreads();
    constexpr int kUnroll = 16;
    for (int q0 = 0; q0 < R; q0 += kThreads * kUnroll) {
      int e[kUnroll];  // keys
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int p = q0 + u * kThreads + tid;
        e[u] = p < R ? expert_key(idx[p], E) : E;
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int p = q0 + u * kThreads + tid;
        if (p < R) atomicAdd(&(p < c0 ? hb : ha)[e[u]], 1);
      }
    }
  }

  int key[1], rank[1];
  rank_wave_keys<1>(own, p_begin, p_stop, lmask + w * nk, cnt + w * nk, key, rank);
  __syncthreads();

  for (int j = tid; j < nk; j += kThreads) {
    int run = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const int c = cnt[ww * nk + j];
      cnt[ww * nk + j] = run;
      run += c;
    }
    int b = 0, a = 0;
#pragma unroll
    for (int cp = 0; cp < kHistCopies; ++cp) {
      b += before[cp * nk + j];
      a += after[cp * nk + j];
    }
    before[j] = b;
    after[j] = b + a;  // total: `after` counted this block's chunk too
  }
  __syncthreads();
  block_exclusive_scan(after, nk);
  write_counts(after, E, cap, blockIdx.x, counts, offsets);

  const int k = key[0];
  if (k >= 0) write_entry(p_begin + lane, k, before[k] + cnt[w * nk + k] + rank[0], after, E, K, cap, slot, src);
}

size_t fused_lds_bytes(int nw, int E) {
  const size_t nk = static_cast<size_t>(E) + 1;
  return nw * nk * 12 + 2 * kHistCopies * nk * 4;
}

// LDS one workgroup may allocate on gfx950: the CU's whole 160 KB.  Up to
// 512 experts the one-launch layout keeps 16 waves; at 1024, 8.
constexpr size_t kLdsLimit = 160 * 1024;

size_t single_lds_bytes(int nw, int E) {
  const size_t nk = static_cast<size_t>(E) + 1;
  return nw * nk * 8 + nw * nk * 4 + nk * 4;
}

int single_waves(int E) {
  // 8 waves: measured a little faster than 16 at 1024 entries (fewer waves
  // to scan per key, two 64-entry steps each)
  int nw = kSingleMaxWaves;
  while (nw > 1 && single_lds_bytes(nw, E) > kLdsLimit) nw >>= 1;
  return nw;
}

int fused_waves(int E) {
  int nw = 16;
  while (nw > 1 && fused_lds_bytes(nw, E) > kLdsLimit) nw >>= 1;
  return nw;
}

enum class LayoutPath { kSingle, kFused, kMulti };

LayoutPath choose_path(int64_t rows) {
  if (rows <= kSingleMaxEntries) return LayoutPath::kSingle;
  if (rows <= kOneLaunchMaxEntries) return LayoutPath::kFused;
  return LayoutPath::kMulti;
}

// two-launch path: chunks of 256*16 = 4096 entries
constexpr int kMultiIters = 16;

}  // namespace

size_t layout_workspace_bytes(int64_t rows, int32_t num_experts) {
  if (choose_path(rows) != LayoutPath::kMulti) return 0;
  const int64_t chunk = static_cast<int64_t>(kMultiThreads) * kMultiIters;
  const int64_t nblocks = (rows + chunk - 1) / chunk;
  return static_cast<size_t>(nblocks) * (num_experts + 1) * sizeof(int32_t);
}

template <typename Idx>
hipError_t launch_layout(const Idx* topk_idx, int32_t rows, int32_t top_k, int32_t num_experts, int32_t capacity,
                         int32_t* counts, int32_t* offsets, int32_t* slot, int32_t* src, void* workspace,
                         hipStream_t stream) {
  const int E = num_experts, nk = E + 1;
  const LayoutPath path = choose_path(rows);
  if (path == LayoutPath::kSingle) {
    const int nw = single_waves(E);
    const int steps = ((rows + nw - 1) / nw + kWave - 1) / kWave;  // 64-entry steps per wave
    const size_t lds = single_lds_bytes(nw, E);
    const dim3 grid(1), block(nw * kWave);
#define EP_LAYOUT_SINGLE(IT)                                                                                  \
  hipLaunchKernelGGL((layout_single<IT, Idx>), grid, block, lds, stream, topk_idx, rows, top_k, E, capacity, \
                     counts, offsets, slot, src)
    if (steps <= 1) EP_LAYOUT_SINGLE(1);
    else if (steps <= 4) EP_LAYOUT_SINGLE(4);
    else EP_LAYOUT_SINGLE(16);
#undef EP_LAYOUT_SINGLE
    return hipGetLastError();
  }
  if (path == LayoutPath::kFused) {
    const int nw = fused_waves(E);
    const int chunk = nw * kWave;
    const dim3 grid((rows + chunk - 1) / chunk), block(chunk);
    const size_t lds = fused_lds_bytes(nw, E);
    // 16-byte id loads: ids aligned to 16 bytes
    const bool v4 = (reinterpret_cast<uintptr_t>(topk_idx) & 15) == 0;
#define EP_LAYOUT_FUSED_V(NW, V)                                                                                  \
  hipLaunchKernelGGL((layout_fused<NW, V, Idx>), grid, block, lds, stream, topk_idx, rows, top_k, E, capacity, \
                     counts, offsets, slot, src)
#define EP_LAYOUT_FUSED(NW) \
  if (v4) EP_LAYOUT_FUSED_V(NW, true); else EP_LAYOUT_FUSED_V(NW, false)
    if (nw >= 16) { EP_LAYOUT_FUSED(16); }
    else if (nw >= 8) { EP_LAYOUT_FUSED(8); }
    else if (nw >= 4) { EP_LAYOUT_FUSED(4); }
    else { EP_LAYOUT_FUSED(1); }
#undef EP_LAYOUT_FUSED
#undef EP_LAYOUT_FUSED_V
    return hipGetLastError();
  }
  const int chunk = kMultiThreads * kMultiIters;
  const int nblocks = (rows + chunk - 1) / chunk;
  int32_t* hist = static_cast<int32_t*>(workspace);
  const size_t lds_count = static_cast<size_t>(kMultiWaves * nk) * (sizeof(uint64_t) + sizeof(int));
  const size_t lds_final = static_cast<size_t>(2 * nk) * sizeof(int);
  const dim3 grid(nblocks), block(kMultiThreads);
  hipLaunchKernelGGL((layout_count<kMultiIters, Idx>), grid, block, lds_count, stream, topk_idx, rows, E, slot,
                     hist);
  hipLaunchKernelGGL((layout_finalize<kMultiIters, Idx>), grid, block, lds_final, stream, topk_idx, rows, top_k, E,
                     capacity, nblocks, hist, counts, offsets, slot, src);
  return hipGetLastError();
}

template hipError_t launch_layout<int32_t>(const int32_t*, int32_t, int32_t, int32_t, int32_t, int32_t*, int32_t*,
                                           int32_t*, int32_t*, void*, hipStream_t);
template hipError_t launch_layout<int64_t>(const int64_t*, int32_t, int32_t, int32_t, int32_t, int32_t*, int32_t*,
                                           int32_t*, int32_t*, void*, hipStream_t);

}  // namespace ep
