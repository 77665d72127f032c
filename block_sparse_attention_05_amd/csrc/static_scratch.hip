// sparse_attn_route_noalloc: sparse_attn_route with its workspace (the
// pooled Q and K means) in a library-held device array instead of a caller
// buffer, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on
// holds its own copy of SA_STATIC_SCRATCH_BYTES until the process ends.  In
// host code the array's name is only a host-side stand-in, so its device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept; kernels get that address, never the name.
//
// Nothing here allocates: the lookup loads no memory of its own and the
// entry point itself calls no hipMalloc / hipFree.  Every call on a GPU uses
// that GPU's one array: calls that overlap on one GPU (two streams, or two
// host threads) race on it, so callers serialise them.  The pooling kernel
// writes every mean the route kernel reads as a result; padding entries
// between tiles are read but reach only unused score rows and columns, so
// the array needs no clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "sparse_attn.h"

static __device__ __align__(256) unsigned char scratch[SA_STATIC_SCRATCH_BYTES];

namespace sa {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on `device`, looked up on first use with that
// device current (the caller's current device is restored).
hipError_t scratch_on(int device, void **ptr) {
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[device] != nullptr) {
    *ptr = g_scratch_ptr[device];
    return hipSuccess;
  }
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
  void *p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (cur != device) {
    const hipError_t e2 = hipSetDevice(cur);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) return e;
  if (p == nullptr) return hipErrorInvalidSymbol;
  g_scratch_ptr[device] = p;
  *ptr = p;
  return hipSuccess;
}

}  // namespace
}  // namespace sa

extern "C" sa_status sparse_attn_route_noalloc(const void *q, const void *k, int32_t B, int32_t T,
                                               int32_t H, int32_t D, int32_t sink_start,
                                               int32_t sink_tokens, int32_t video_tail_mode,
                                               float topk_ratio, int32_t local_radius,
                                               int32_t *block_idx, int32_t max_sel,
                                               int32_t *block_cnt, float *route_scores,
                                               void *stream) {
  // Arguments and size are checked before anything touches a device.
  const sa_status st = sa::check_route_args(q, k, B, T, H, D, sink_start, sink_tokens,
                                            video_tail_mode, topk_ratio, local_radius, block_idx,
                                            max_sel, block_cnt, route_scores);
  if (st != SA_OK) return st;
  if (sa_num_query_blocks(T, sink_start, video_tail_mode) == 0)
    return sparse_attn_route(q, k, B, T, H, D, sink_start, sink_tokens, video_tail_mode,
                             topk_ratio, local_radius, block_idx, max_sel, block_cnt, route_scores,
                             nullptr, 0, stream);
  const size_t need = sa_route_workspace_bytes(B, T, H, sink_start, video_tail_mode);
  if (need > (size_t)SA_STATIC_SCRATCH_BYTES)
    return sa::set_error(SA_ERR_WORKSPACE,
                         "sparse_attn_route_noalloc: the pooled means need %zu bytes, more than "
                         "the library's static scratch of %zu bytes (use sparse_attn_route with "
                         "a caller workspace)",
                         need, (size_t)SA_STATIC_SCRATCH_BYTES);
  int device = 0;
  hipError_t e = stream != nullptr ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &device)
                                   : hipGetDevice(&device);
  if (e != hipSuccess)
    return sa::set_error(SA_ERR_HIP, "sparse_attn_route_noalloc: device of the stream: %s",
                         hipGetErrorString(e));
  if (device < 0 || device >= sa::kMaxDevices)
    return sa::set_error(SA_ERR_UNSUPPORTED, "sparse_attn_route_noalloc: device %d beyond %d",
                         device, sa::kMaxDevices);
  void *ws = nullptr;
  if ((e = sa::scratch_on(device, &ws)) != hipSuccess)
    return sa::set_error(SA_ERR_HIP, "sparse_attn_route_noalloc: static scratch address: %s",
                         hipGetErrorString(e));
  return sparse_attn_route(q, k, B, T, H, D, sink_start, sink_tokens, video_tail_mode, topk_ratio,
                           local_radius, block_idx, max_sel, block_cnt, route_scores, ws,
                           (size_t)SA_STATIC_SCRATCH_BYTES, stream);
}
