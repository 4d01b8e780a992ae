/*
 * ep_step - one MoE step through the C ABI of libep.so, from plain C and the
 * HIP runtime, with no Python (test driver).
 *
 *   ep_step DIR T H K E CAPACITY MODE [IDS64]
 *
 * Reads DIR/topk_idx.bin (int32 [T,K]), DIR/x.bin (bf16 bits [T,H]),
 * DIR/w.bin (float32 [T,K]) and DIR/y.bin (bf16 bits [rows,H]; rows = T*K,
 * or E*CAPACITY when CAPACITY > 0).  MODE 0 runs the layout call then
 * ep_dispatch; MODE 1 runs ep_layout_dispatch; both then run ep_combine.
 * MODE 2 records the step in an ep_step_plan and runs the plan's two
 * launches twice, as a serving loop would.
 * With IDS64 = 1, topk_idx.bin holds int64 ids and the *_i64 layout calls
 * are used.  The FP8 receive format is used.  Writes counts.bin, offsets.bin
 * (packed only), slot.bin, src.bin, recv.bin, scale.bin, rweight.bin and
 * out.bin to DIR.  Exits non-zero, with a message, on any error.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ep.h"

#define HIP_CHECK(call)                                                              \
  do {                                                                               \
    hipError_t e_ = (call);                                                          \
    if (e_ != hipSuccess) {                                                          \
      fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #call, hipGetErrorString(e_)); \
      exit(2);                                                                       \
    }                                                                                \
  } while (0)

#define EP_CHECK(call)                                                                 \
  do {                                                                                 \
    ep_status s_ = (call);                                                             \
    if (s_ != EP_OK) {                                                                 \
      fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #call, ep_status_string(s_)); \
      exit(3);                                                                         \
    }                                                                                  \
  } while (0)

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    exit(4);
  }
  void* buf = malloc(bytes ? bytes : 1);
  if (!buf || fread(buf, 1, bytes, f) != bytes) {
    fprintf(stderr, "short read of %s (%zu bytes expected)\n", path, bytes);
    exit(4);
  }
  fclose(f);
  return buf;
}

static void write_file(const char* dir, const char* name, const void* dev, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  void* host = malloc(bytes ? bytes : 1);
  if (!host) exit(5);
  if (bytes) HIP_CHECK(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost));
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(host, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", path);
    exit(5);
  }
  fclose(f);
  free(host);
}

static void* upload(const void* host, size_t bytes) {
  void* dev = NULL;
  HIP_CHECK(hipMalloc(&dev, bytes ? bytes : 16));
  if (bytes) HIP_CHECK(hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice));
  return dev;
}

static void* device_buffer(size_t bytes, int fill) {
  void* dev = NULL;
  HIP_CHECK(hipMalloc(&dev, bytes ? bytes : 16));
  HIP_CHECK(hipMemset(dev, fill, bytes ? bytes : 16));
  return dev;
}

int main(int argc, char** argv) {
  if (argc != 8 && argc != 9) {
    fprintf(stderr, "usage: %s DIR T H K E CAPACITY MODE [IDS64]\n", argv[0]);
    return 1;
  }
  const int ids64 = argc == 9 && atoi(argv[8]) == 1;
  const size_t id_bytes = ids64 ? 8 : 4;
  const char* dir = argv[1];
  const int64_t T = atoll(argv[2]);
  const int32_t H = atoi(argv[3]), K = atoi(argv[4]), E = atoi(argv[5]), cap = atoi(argv[6]);
  const int mode = atoi(argv[7]);
  const size_t rows = cap > 0 ? (size_t)E * (size_t)cap : (size_t)T * (size_t)K;
  const size_t n = (size_t)T * (size_t)K;

  void* h_idx = read_file(dir, "topk_idx.bin", n * id_bytes);
  void* h_x = read_file(dir, "x.bin", (size_t)T * H * 2);
  void* h_w = read_file(dir, "w.bin", n * 4);
  void* h_y = read_file(dir, "y.bin", rows * H * 2);

  void* idx = upload(h_idx, n * id_bytes);
  void* x = upload(h_x, (size_t)T * H * 2);
  float* w = (float*)upload(h_w, n * 4);
  void* y = upload(h_y, rows * H * 2);
  int32_t* counts = (int32_t*)device_buffer((size_t)E * 4, 0xFF);
  int32_t* offsets = cap > 0 ? NULL : (int32_t*)device_buffer(((size_t)E + 1) * 4, 0xFF);
  int32_t* slot = (int32_t*)device_buffer(n * 4, 0xFF);
  int32_t* src = (int32_t*)device_buffer(rows * 4, 0xFF);
  uint8_t* recv = (uint8_t*)device_buffer(rows * H, 0xA5);
  float* scale = (float*)device_buffer(rows * (H / 128) * 4, 0xFF);
  float* rweight = (float*)device_buffer(rows * 4, 0xFF);
  void* out = device_buffer((size_t)T * H * 2, 0xFF);
  const size_t ws_bytes = ep_layout_workspace_bytes(T, K, E);
  void* ws = ws_bytes ? device_buffer(ws_bytes, 0) : NULL;

  hipStream_t stream;
  HIP_CHECK(hipStreamCreate(&stream));
  if (mode == 2) {
    ep_step_plan plan;
    EP_CHECK(ep_step_plan_init(&plan, idx, ids64 ? 8 : 4, x, w, T, H, K, E, cap, EP_RECV_FP8_E4M3_G128, counts,
                               offsets, slot, src, recv, scale, rweight, ws, ws_bytes, y, out, stream));
    for (int rep = 0; rep < 2; ++rep) {
      EP_CHECK(ep_step_plan_layout_dispatch(&plan));
      EP_CHECK(ep_step_plan_combine(&plan));
    }
  } else if (mode == 1 && ids64) {
    EP_CHECK(ep_layout_dispatch_i64((const int64_t*)idx, x, w, T, H, K, E, cap, EP_RECV_FP8_E4M3_G128, counts,
                                    offsets, slot, src, recv, scale, rweight, ws, ws_bytes, stream));
  } else if (mode == 1) {
    EP_CHECK(ep_layout_dispatch((const int32_t*)idx, x, w, T, H, K, E, cap, EP_RECV_FP8_E4M3_G128, counts, offsets,
                                slot, src, recv, scale, rweight, ws, ws_bytes, stream));
  } else {
    if (cap > 0 && ids64)
      EP_CHECK(ep_dispatch_layout_padded_i64((const int64_t*)idx, T, K, E, cap, counts, slot, src, ws, ws_bytes,
                                             stream));
    else if (cap > 0)
      EP_CHECK(ep_dispatch_layout_padded((const int32_t*)idx, T, K, E, cap, counts, slot, src, ws, ws_bytes, stream));
    else if (ids64)
      EP_CHECK(ep_dispatch_layout_i64((const int64_t*)idx, T, K, E, counts, offsets, slot, src, ws, ws_bytes, stream));
    else
      EP_CHECK(ep_dispatch_layout((const int32_t*)idx, T, K, E, counts, offsets, slot, src, ws, ws_bytes, stream));
    EP_CHECK(ep_dispatch(x, T, H, K, slot, w, EP_RECV_FP8_E4M3_G128, recv, scale, rweight, stream));
  }
  if (mode != 2) EP_CHECK(ep_combine(y, slot, w, T, H, K, out, stream));
  HIP_CHECK(hipStreamSynchronize(stream));

  write_file(dir, "counts.bin", counts, (size_t)E * 4);
  if (offsets) write_file(dir, "offsets.bin", offsets, ((size_t)E + 1) * 4);
  write_file(dir, "slot.bin", slot, n * 4);
  write_file(dir, "src.bin", src, rows * 4);
  write_file(dir, "recv.bin", recv, rows * H);
  write_file(dir, "scale.bin", scale, rows * (H / 128) * 4);
  write_file(dir, "rweight.bin", rweight, rows * 4);
  write_file(dir, "out.bin", out, (size_t)T * H * 2);

  HIP_CHECK(hipStreamDestroy(stream));
  void* bufs[] = {idx, x, w, y, counts, offsets, slot, src, recv, scale, rweight, out, ws};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
    if (bufs[i]) HIP_CHECK(hipFree(bufs[i]));
  free(h_idx);
  free(h_x);
  free(h_w);
  free(h_y);
  printf("ep_step ok: T=%lld H=%d K=%d E=%d capacity=%d mode=%d ids64=%d\n", (long long)T, H, K, E, cap, mode,
         ids64);
  return 0;
}
