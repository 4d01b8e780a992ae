// Dispatch layout: per-expert counts, exclusive-scan offsets, and the stable
// (ascending token, then k) receive row of every (token, k) entry.
//
// Definition (the handle of the pages' dispatch call, [P4 "使用示例 › MoE
// 训练中的应用"], with the in-expert order fixed to ascending (t, k)):
//   slot[t,k] = offset[e] + #{(t',k') before (t,k) with the same expert e}.
//
// gfx950 design.  Entries are taken in (t, k) order, 64 per wavefront step.
// Equal keys inside a step are found with one ballot per key bit (there is
// no match instruction on CDNA); a lane's rank among equal keys is the
// popcount of the matching lanes below it (mbcnt), and the lowest matching
// lane adds the group size to a per-wave LDS counter for that key.  Masked
// entries (expert outside [0, E)) use the extra key E so that they sort
// behind every real row, which keeps slot and src a bijection over all T*K
// entries.  Per-wave counters are scanned across waves, per key, in LDS;
// the per-key totals are scanned across keys for the offsets.  No atomics:
// every output is a pure function of topk_idx.
//
// Small inputs (<= 4096 entries) run in one workgroup.  Larger ones use two
// launches: `layout_count` ranks entries inside fixed 1024..4096-entry
// chunks and writes each chunk's per-key histogram to the workspace;
// `layout_finalize` sums the histograms of earlier chunks (a per-key scan
// over chunks), scans the totals over keys and writes the final rows.

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kSingleMaxThreads = 1024;
constexpr int kSingleMaxIters = 4;
constexpr int kMultiThreads = 256;
constexpr int kMultiWaves = kMultiThreads / kWave;

__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  return x;
}

// Exclusive prefix sum of data[0..n) in LDS, in place.  Every thread of the
// block must call it.  wave_tot needs blockDim.x / 64 ints of LDS.
__device__ void block_exclusive_scan(int* data, int n, int* wave_tot) {
  const int tid = threadIdx.x, bs = blockDim.x;
  const int lane = tid & (kWave - 1), w = tid / kWave, nw = bs / kWave;
  const int per = (n + bs - 1) / bs;
  const int beg = min(n, tid * per), end = min(n, beg + per);
  int local = 0;
  for (int i = beg; i < end; ++i) local += data[i];
  const int incl = wave_inclusive_scan(local);
  if (lane == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int v = lane < nw ? wave_tot[lane] : 0;
    const int s = wave_inclusive_scan(v);
    if (lane < nw) wave_tot[lane] = s - v;
  }
  __syncthreads();
  int run = wave_tot[w] + incl - local;
  for (int i = beg; i < end; ++i) {
    const int c = data[i];
    data[i] = run;
    run += c;
  }
  __syncthreads();
}

// Rank ITERS consecutive 64-entry steps of this wavefront: entries
// [p_begin, p_end).  cnt is this wave's LDS counter row (E+1 keys).  On
// return key[i] is the entry's key (E for masked) and rank[i] its position
// among the wave's entries with that key.  Lanes past p_end get key -1.
template <int ITERS>
__device__ __forceinline__ void rank_wave_range(const int32_t* __restrict__ idx, int p_begin, int p_end,
                                                int E, int nbits, int* cnt, int (&key)[ITERS],
                                                int (&rank)[ITERS]) {
  const int lane = threadIdx.x & (kWave - 1);
  int e[ITERS];
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const int p = p_begin + i * kWave + lane;
    e[i] = p < p_end ? idx[p] : -1;
  }
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const int p = p_begin + i * kWave + lane;
    const bool inr = p < p_end;
    const int k = (e[i] >= 0 && e[i] < E) ? e[i] : E;
    uint64_t mask = wave_ballot(inr);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (k >> b) & 1;
      const uint64_t bal = wave_ballot(bit);
      mask &= bit ? bal : ~bal;
    }
    const int below = static_cast<int>(lanes_below(mask));
    const int group = static_cast<int>(__popcll(mask));
    const int pre = inr ? cnt[k] : 0;
    if (inr && below == 0) cnt[k] = pre + group;
    key[i] = inr ? k : -1;
    rank[i] = pre + below;
  }
}

__device__ __forceinline__ int key_bits(int E) { return 32 - __clz(E); }  // covers keys 0..E

template <int ITERS>
__global__ __launch_bounds__(kSingleMaxThreads) void layout_single(
    const int32_t* __restrict__ idx, int32_t R, int32_t K, int32_t E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot, int32_t* __restrict__ src) {
  extern __shared__ int lds[];
  const int tid = threadIdx.x, bs = blockDim.x, nw = bs / kWave, w = tid / kWave;
  const int nk = E + 1;
  int* cnt = lds;              // [nw][nk]
  int* off = lds + nw * nk;    // [nk]
  int* wave_tot = off + nk;    // [nw]
  for (int i = tid; i < nw * nk; i += bs) cnt[i] = 0;
  __syncthreads();

  const int per = ((R + nw - 1) / nw + kWave - 1) / kWave * kWave;
  const int p_begin = w * per;
  const int p_end = min(R, p_begin + per);
  int key[ITERS], rank[ITERS];
  rank_wave_range<ITERS>(idx, p_begin, p_end, E, key_bits(E), cnt + w * nk, key, rank);
  __syncthreads();

  for (int j = tid; j < nk; j += bs) {
    int run = 0;
    for (int ww = 0; ww < nw; ++ww) {
      const int c = cnt[ww * nk + j];
      cnt[ww * nk + j] = run;
      run += c;
    }
    off[j] = run;
    if (j < E) counts[j] = run;
  }
  __syncthreads();
  block_exclusive_scan(off, nk, wave_tot);
  for (int j = tid; j < nk; j += bs) offsets[j] = off[j];

  const int lane = tid & (kWave - 1);
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const int p = p_begin + i * kWave + lane;
    const int k = key[i];
    if (k >= 0) {
      const int pos = off[k] + cnt[w * nk + k] + rank[i];
      const bool valid = k < E;
      slot[p] = valid ? pos : -1;
      src[pos] = valid ? static_cast<int>(static_cast<uint32_t>(p) / static_cast<uint32_t>(K)) : -1;
    }
  }
}

template <int ITERS>
__global__ __launch_bounds__(kMultiThreads) void layout_count(const int32_t* __restrict__ idx, int32_t R,
                                                              int32_t E, int32_t* __restrict__ slot_tmp,
                                                              int32_t* __restrict__ hist) {
  extern __shared__ int lds[];
  const int tid = threadIdx.x, w = tid / kWave, lane = tid & (kWave - 1);
  const int nk = E + 1;
  int* cnt = lds;  // [kMultiWaves][nk]
  for (int i = tid; i < kMultiWaves * nk; i += kMultiThreads) cnt[i] = 0;
  __syncthreads();

  constexpr int kChunk = kMultiThreads * ITERS;
  const int p_begin = blockIdx.x * kChunk + w * (kWave * ITERS);
  const int p_end = min(R, p_begin + kWave * ITERS);
  int key[ITERS], rank[ITERS];
  rank_wave_range<ITERS>(idx, p_begin, p_end, E, key_bits(E), cnt + w * nk, key, rank);
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

template <int ITERS>
__global__ __launch_bounds__(kMultiThreads) void layout_finalize(
    const int32_t* __restrict__ idx, int32_t R, int32_t K, int32_t E, int32_t nblocks,
    const int32_t* __restrict__ hist, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot, int32_t* __restrict__ src) {
  extern __shared__ int lds[];
  const int tid = threadIdx.x;
  const int nk = E + 1;
  int* base = lds;            // [nk] rows of this key in earlier chunks
  int* off = lds + nk;        // [nk] totals, then offsets
  int* wave_tot = off + nk;   // [kMultiWaves]
  const int b = blockIdx.x;
  for (int j = tid; j < nk; j += kMultiThreads) {
    int before = 0, total = 0;
    for (int bb = 0; bb < nblocks; ++bb) {
      const int h = hist[static_cast<size_t>(bb) * nk + j];
      total += h;
      before += bb < b ? h : 0;
    }
    base[j] = before;
    off[j] = total;
    if (b == 0 && j < E) counts[j] = total;
  }
  __syncthreads();
  block_exclusive_scan(off, nk, wave_tot);
  if (b == 0)
    for (int j = tid; j < nk; j += kMultiThreads) offsets[j] = off[j];

  constexpr int kChunk = kMultiThreads * ITERS;
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const int p = b * kChunk + i * kMultiThreads + tid;
    if (p < R) {
      const int e = idx[p];
      const bool valid = e >= 0 && e < E;
      const int k = valid ? e : E;
      const int pos = off[k] + base[k] + slot[p];
      slot[p] = valid ? pos : -1;
      src[pos] = valid ? static_cast<int>(static_cast<uint32_t>(p) / static_cast<uint32_t>(K)) : -1;
    }
  }
}

int single_waves(int E) {
  // LDS: nw*(E+1) counters + (E+1) offsets + nw wave totals, within 64 KiB
  int nw = kSingleMaxThreads / kWave;
  while (nw > 1 && static_cast<size_t>(nw * (E + 1) + (E + 1) + nw) * 4 > 65536) nw >>= 1;
  return nw;
}

int multi_iters(int64_t rows) {
  // chunk of 256*ITERS entries; grow the chunk so that at most 64 chunks
  // exist, which bounds the per-key scan over chunks in layout_finalize
  if (rows <= 64LL * kMultiThreads * 4) return 4;
  if (rows <= 64LL * kMultiThreads * 8) return 8;
  return 16;
}

}  // namespace

size_t layout_workspace_bytes(int64_t rows, int32_t num_experts) {
  const int nw = single_waves(num_experts);
  if (rows <= static_cast<int64_t>(nw) * kWave * kSingleMaxIters) return 0;
  const int64_t chunk = static_cast<int64_t>(kMultiThreads) * multi_iters(rows);
  const int64_t nblocks = (rows + chunk - 1) / chunk;
  return static_cast<size_t>(nblocks) * (num_experts + 1) * sizeof(int32_t);
}

hipError_t launch_layout(const int32_t* topk_idx, int32_t rows, int32_t top_k, int32_t num_experts,
                         int32_t* counts, int32_t* offsets, int32_t* slot, int32_t* src,
                         void* workspace, hipStream_t stream) {
  const int E = num_experts, nk = E + 1;
  const int nw = single_waves(E);
  if (rows <= nw * kWave * kSingleMaxIters) {
    const int per_wave = ((rows + nw - 1) / nw + kWave - 1) / kWave;  // 64-entry steps per wave
    const size_t lds = static_cast<size_t>(nw * nk + nk + nw) * sizeof(int);
    const dim3 grid(1), block(nw * kWave);
    if (per_wave <= 1)
      hipLaunchKernelGGL(layout_single<1>, grid, block, lds, stream, topk_idx, rows, top_k, E, counts,
                         offsets, slot, src);
    else if (per_wave <= 2)
      hipLaunchKernelGGL(layout_single<2>, grid, block, lds, stream, topk_idx, rows, top_k, E, counts,
                         offsets, slot, src);
    else
      hipLaunchKernelGGL(layout_single<4>, grid, block, lds, stream, topk_idx, rows, top_k, E, counts,
                         offsets, slot, src);
    return hipGetLastError();
  }
  const int iters = multi_iters(rows);
  const int chunk = kMultiThreads * iters;
  const int nblocks = (rows + chunk - 1) / chunk;
  int32_t* hist = static_cast<int32_t*>(workspace);
  const size_t lds_count = static_cast<size_t>(kMultiWaves * nk) * sizeof(int);
  const size_t lds_final = static_cast<size_t>(2 * nk + kMultiWaves) * sizeof(int);
  const dim3 grid(nblocks), block(kMultiThreads);
  switch (iters) {
    case 4:
      hipLaunchKernelGGL(layout_count<4>, grid, block, lds_count, stream, topk_idx, rows, E, slot, hist);
      hipLaunchKernelGGL(layout_finalize<4>, grid, block, lds_final, stream, topk_idx, rows, top_k, E,
                         nblocks, hist, counts, offsets, slot, src);
      break;
    case 8:
      hipLaunchKernelGGL(layout_count<8>, grid, block, lds_count, stream, topk_idx, rows, E, slot, hist);
      hipLaunchKernelGGL(layout_finalize<8>, grid, block, lds_final, stream, topk_idx, rows, top_k, E,
                         nblocks, hist, counts, offsets, slot, src);
      break;
    default:
      hipLaunchKernelGGL(layout_count<16>, grid, block, lds_count, stream, topk_idx, rows, E, slot, hist);
      hipLaunchKernelGGL(layout_finalize<16>, grid, block, lds_final, stream, topk_idx, rows, top_k, E,
                         nblocks, hist, counts, offsets, slot, src);
      break;
  }
  return hipGetLastError();
}

}  // namespace ep
