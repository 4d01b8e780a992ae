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

#include "ep_internal.h"
#include "layout_device.h"

namespace ep {
namespace {

constexpr int kSingleMaxWaves = 8;  // the single-workgroup path launches at most 8 waves
constexpr int kSingleMaxThreads = kSingleMaxWaves * 64;
constexpr int kSingleMaxEntries = 1024;  // one workgroup, no workspace
constexpr int kMultiThreads = 256;
constexpr int kMultiWaves = kMultiThreads / kWave;

template <int ITERS, typename Idx>
__global__ __launch_bounds__(kSingleMaxThreads) void layout_single(
    const Idx* __restrict__ idx, int32_t R, int32_t K, int32_t E, int32_t cap, int32_t bs, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot, int32_t* __restrict__ src) {
  extern __shared__ uint64_t lds64[];
  const int tid = threadIdx.x, nw = bs / kWave, w = tid / kWave;  // bs: the workgroup's lanes
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
  write_counts(off, E, cap, 0, bs, counts, offsets);

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
  write_counts(off, E, cap, b, kMultiThreads, counts, offsets);

#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const int p = b * kChunk + i * kMultiThreads + tid;
    if (p < R) write_entry(p, e[i], base[e[i]] + loc[i], off, E, K, cap, slot, src);
  }
}

// One launch for the whole layout: workgroup b owns the chunk of NW*64
// consecutive entries from b*NW*64 (layout_chunk).
template <int NW, bool V4, typename Idx>
__global__ __launch_bounds__(NW * kWave) void layout_fused(
    const Idx* __restrict__ idx, int32_t R, int32_t K, int32_t E, int32_t cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot, int32_t* __restrict__ src) {
  extern __shared__ uint64_t lds64[];
  const int c0 = blockIdx.x * NW * kWave;
  layout_chunk<NW, V4, Idx, false>(idx, R, K, E, cap, c0, min(R, c0 + NW * kWave), lds64, counts, offsets, slot,
                                   src, [] {}, [](int) {});
}

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
                     nw * kWave, counts, offsets, slot, src)
    if (steps <= 1) EP_LAYOUT_SINGLE(1);
    else if (steps <= 4) EP_LAYOUT_SINGLE(4);
    else EP_LAYOUT_SINGLE(16);
#undef EP_LAYOUT_SINGLE
    return hipGetLastError();
  }
  if (path == LayoutPath::kFused) {
    const int nw = chunk_waves(E);
    const int chunk = nw * kWave;
    const dim3 grid((rows + chunk - 1) / chunk), block(chunk);
    const size_t lds = chunk_lds_bytes(nw, E);
    // 16-byte id loads: ids aligned to 16 bytes
    const bool v4 = (reinterpret_cast<uintptr_t>(topk_idx) & 15) == 0;
#define EP_LAYOUT_FUSED_V(NW, V)                                                                                  \
  hipLaunchKernelGGL((layout_fused<NW, V, Idx>), grid, block, lds, stream, topk_idx, rows, top_k, E, capacity, \
                     counts, offsets, slot, src)
#define EP_LAYOUT_FUSED(NW) \
  if (v4) EP_LAYOUT_FUSED_V(NW, true); else EP_LAYOUT_FUSED_V(NW, false)
    // the kernel's NW must equal the launched waves; up to EP_MAX_EXPERTS
    // (1024) experts chunk_waves gives 16 or 8
    if (nw == 16) { EP_LAYOUT_FUSED(16); }
    else if (nw == 8) { EP_LAYOUT_FUSED(8); }
    else { return hipErrorInvalidValue; }
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
