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

}  // namespace

template <typename Idx>
bool launch_layout_dispatch_chunked(const Idx* topk_idx, const uint16_t* x, const float* topk_weights,
                                    int32_t T, int32_t H, int32_t K, int32_t E, int32_t capacity, bool fp8,
                                    int32_t* counts, int32_t* offsets, int32_t* slot, int32_t* src, void* recv,
                                    float* recv_scale, float* recv_weight, hipStream_t stream, hipError_t* err) {
  const int64_t n = static_cast<int64_t>(T) * K;
  if (n <= kFusedMaxEntries || n > kOneLaunchMaxEntries || K > kChunkMaxK) return false;
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
