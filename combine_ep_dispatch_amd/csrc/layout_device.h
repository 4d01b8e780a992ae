// Device helpers of the layout kernels (internal header): wavefront ranking
// of equal expert keys, the row of an entry, and the one-launch layout of
// one chunk of entries, shared by the layout kernels and the chunked
// layout + dispatch kernel.
#pragma once

#include "ep_device.h"

namespace ep {

constexpr int kHistCopies = 4;  // one-launch layout: private histograms per lane & 3
constexpr int kChunkSteps = 8;  // layout_chunk: calls of the caller's step hook

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

// The key of this lane's entry p_begin + lane (E at or past p_stop), by an
// unconditional load clamped to the last entry (R >= 1).
template <typename Idx>
__device__ __forceinline__ void load_own_key(const Idx* __restrict__ idx, int R, int p_begin, int p_stop, int E,
                                             int& key) {
  const int p = p_begin + static_cast<int>(threadIdx.x & (kWave - 1));
  const int k = expert_key(idx[min(p, R - 1)], E);
  key = p < p_stop ? k : E;
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

// Row of one entry whose rank among the entries of its key is `within`,
// written to slot[p] and returned.
// Packed layout (cap == 0): row off[k] + within; masked entries (k == E)
// take the rows after the valid ones with src = -1.  Padded layout
// (cap > 0): expert e owns rows e*cap .. e*cap+cap-1; entries ranked past
// the capacity and masked entries get slot -1 and no row, and the unused
// rows of an expert's block are not written.
__device__ __forceinline__ int write_entry(int p, int k, int within, const int* off, int E, int K, int cap,
                                           int32_t* __restrict__ slot, int32_t* __restrict__ src) {
  const bool valid = k < E;
  const int t = valid ? static_cast<int>(static_cast<uint32_t>(p) / static_cast<uint32_t>(K)) : -1;
  int row;
  if (cap == 0) {
    const int pos = off[k] + within;
    row = valid ? pos : -1;
    src[pos] = t;
  } else {
    const bool keep = valid && within < cap;
    row = keep ? k * cap + within : -1;
    if (keep) src[k * cap + within] = t;
  }
  slot[p] = row;
  return row;
}

// Counts and offsets from the exclusive scan `off` of the per-key totals
// (written by one workgroup of bs lanes); in the padded layout the count is
// clamped to the capacity and there are no offsets.  The callers pass bs
// rather than read blockDim, which would make every launch carry the
// runtime's 256 bytes of implicit arguments.
__device__ __forceinline__ void write_counts(const int* off, int E, int cap, int part, int bs,
                                             int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  if (part != 0) return;
  const int tid = threadIdx.x;
  for (int j = tid; j < E; j += bs) {
    const int total = off[j + 1] - off[j];
    counts[j] = cap == 0 ? total : min(total, cap);
  }
  if (cap == 0)
    for (int j = tid; j <= E; j += bs) offsets[j] = off[j];
}

// The one-launch layout of the chunk [c0, c1) of entries (c1 - c0 <= NW*64,
// one entry per thread, c0 a multiple of 4), by one workgroup of NW
// wavefronts.  The workgroup ranks its chunk as above (one 64-entry step
// per wave) and also histograms all T*K entries with LDS atomic adds
// (integer addition is order-free, so the counts are exact and
// deterministic): entries before its chunk into `before`, the rest, its
// chunk included, into `after`.  Then for every key: total = before +
// after, offsets are the exclusive scan of the totals, and an entry's row
// is offset + before + (own-chunk rank).  Every workgroup reads all T*K ids
// (from L2 after the first), which trades redundant on-chip work for a
// second launch and a workspace.  Everything in the histogram step is paid
// once per entry (32 per lane at 32768 entries and 16 waves), so it spends
// one LDS atomic and its address per entry: which histogram takes a
// load's ids is one workgroup-uniform comparison per 16-byte load, and
// lanes spread over kHistCopies private copies so that a hot expert's
// entries in one wave collide on fewer addresses.  All workgroups walk the
// ids in the same order: one L2 miss per XCD then serves every workgroup
// on it (a per-workgroup rotated start measured 1.7x slower with int64
// ids).
// V4: 16-byte id loads (ids aligned to 16 bytes): 4 int32 or 2 int64 ids
// each, BATCH ids per thread at a time (fewer for a caller that holds
// registers of its own).
// A caller's own loads go in two hooks.  `early()` runs once the first id
// loads are issued (IDS_FIRST: once they have arrived) and before the LDS
// is cleared; `step(u)`, u = 0 .. kChunkSteps-1, runs before the u-th step
// of the histogram's first batch of ids (with 4- or 8-byte id loads: all
// right after early()).  Loads that the memory system cannot take at once
// stall the wave that issues them, so loads spread over the histogram
// steps keep HBM busy while the other waves count.  Workgroup 0 writes counts and offsets; every
// thread with an entry writes its slot and src and gets its row back (-1
// for a masked or dropped entry, and for threads without an entry).
// Uses chunk_lds_bytes(NW, E) of dynamic LDS at lds64.
template <int NW, bool V4, typename Idx, bool IDS_FIRST, int BATCH = 32, typename Early, typename Step>
__device__ __forceinline__ int layout_chunk(const Idx* __restrict__ idx, int32_t R, int32_t K, int32_t E,
                                            int32_t cap, int c0, int c1, uint64_t* lds64,
                                            int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                            int32_t* __restrict__ slot, int32_t* __restrict__ src, Early&& early, Step&& step) {
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
    // 16-byte loads of kPer ids each, BATCH ids in flight per thread.  c0 is
    // a multiple of kPer: each load lies wholly before or wholly at/after
    // c0 (one workgroup-uniform comparison per load), and the last R % kPer
    // ids all lie at or after c0.  Every load is unconditional, its index
    // clamped to the last full load (R >= kPer): a load under a per-lane
    // branch, or a first batch counted inside the loop, makes the compiler
    // wait for every load issued so far, the caller's early ones included.
    constexpr int kPer = 16 / static_cast<int>(sizeof(Idx));
    constexpr int kUnroll = BATCH / kPer;
    const int4* idx4 = reinterpret_cast<const int4*>(idx);
    const int n4 = R / kPer, qb = c0 / kPer;
    int4 e[kUnroll];
    auto load_batch = [&](int q0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) e[u] = idx4[min(q0 + u * kThreads + tid, n4 - 1)];
    };
    static_assert(kUnroll >= kChunkSteps, "one caller step per histogram step of the first batch");
    auto count_batch = [&](int q0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (q0 == 0 && u < kChunkSteps) step(u);
        const int q = q0 + u * kThreads + tid;
        if (q >= n4) continue;
        int* const h = q < qb ? hb : ha;
        int k4[kPer];
        expert_keys16<Idx>(e[u], E, k4);
#pragma unroll
        for (int j = 0; j < kPer; ++j) atomicAdd(&h[k4[j]], 1);
      }
    };
    // the first batch is loaded before the LDS is cleared, so the loads'
    // latency overlaps the clearing and the waves' start (at 32768 int32 or
    // int64 ids one batch is all of them); the empty asm keeps the compiler
    // from sinking the loads below the clearing
    load_batch(0);
    load_own_key(idx, R, p_begin, p_stop, E, own[0]);
    // IDS_FIRST: the caller's early loads (long HBM reads) wait until the
    // ids are in, so that the ids do not queue behind them in the CU's load
    // path (empty asm statements that read every id load force the wait)
    if constexpr (IDS_FIRST) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) asm volatile("" ::"v"(e[u].x));
      asm volatile("" ::"v"(own[0]));
    }
    early();
    asm volatile("" ::: "memory");
    clear_lds();
    __syncthreads();
    count_batch(0);
    for (int q0 = kThreads * kUnroll; q0 < n4; q0 += kThreads * kUnroll) {
      load_batch(q0);
      count_batch(q0);
    }
    const int p = kPer * n4 + tid;  // the last R % kPer ids
    if (p < R) atomicAdd(&ha[expert_key(idx[p], E)], 1);
  } else {
    load_wave_keys<1>(idx, p_begin, p_stop, E, own);
    early();
#pragma unroll
    for (int u = 0; u < kChunkSteps; ++u) step(u);
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
  write_counts(after, E, cap, blockIdx.x, NW * kWave, counts, offsets);

  const int k = key[0];
  return k >= 0 ? write_entry(p_begin + lane, k, before[k] + cnt[w * nk + k] + rank[0], after, E, K, cap, slot, src)
                : -1;
}

// Dynamic LDS of layout_chunk: per-wave lane masks and running counts, and
// the kHistCopies copies of the two histograms.
__host__ __device__ inline size_t chunk_lds_bytes(int nw, int E) {
  const size_t nk = static_cast<size_t>(E) + 1;
  return nw * nk * 12 + 2 * kHistCopies * nk * 4;
}

// Waves of a layout_chunk workgroup: 16 up to 512 experts, 8 at 1024.
inline int chunk_waves(int E) {
  int nw = 16;
  while (nw > 1 && chunk_lds_bytes(nw, E) > kLdsLimit) nw >>= 1;
  return nw;
}

}  // namespace ep
