// rkl_noalloc.hip -- rkl_forward_hidden_noalloc: the hidden-state forward
// with its split partials in a file-scope device array instead of a caller
// workspace, for callers that cannot allocate device memory.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "rkl.h"
#include "rkl_internal.h"
#include "rkl_noalloc.h"

namespace {

// The forward's only scratch: [nsplit][5][N] fp32 split partials.  Every
// GPU the library runs on holds its own copy until the process ends.
constexpr size_t kScratchBytes = RKL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

// Device address of `scratch` per device, looked up once per device with
// that device current (the array's name is a host-side stand-in).
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  return rkl::set_last_error(code, buf);
}

int scratch_of(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RKL_DEVICE_ERROR, "device of the stream: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(RKL_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return fail(RKL_DEVICE_ERROR, "hipGetDevice: %s", hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(RKL_DEVICE_ERROR, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess) return fail(RKL_DEVICE_ERROR, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return RKL_OK;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

int rkl_forward_hidden_noalloc(int64_t N, int64_t V, int64_t Hs, int64_t Ht, const rkl_bf16* h_s,
                               const rkl_bf16* W_s, const rkl_bf16* h_t, const rkl_bf16* W_t, const uint8_t* row_mask,
                               float* loss, float* stats, rkl_stream_t stream) {
  void* ws = nullptr;
  if (N > 0) {
    if (int rc = scratch_of(static_cast<hipStream_t>(stream), &ws)) return rc;
  }
  const int rc = rkl_forward_hidden(N, V, Hs, Ht, h_s, W_s, h_t, W_t, row_mask, loss, stats, ws, kScratchBytes,
                                    stream);
  if (rc == RKL_WORKSPACE_TOO_SMALL)
    return fail(RKL_UNSUPPORTED,
                "N=%lld rows at V=%lld need more than the %zu bytes of device scratch this entry point holds "
                "(20 bytes per row per vocabulary split); split the rows or use rkl_forward_hidden",
                (long long)N, (long long)V, kScratchBytes);
  return rc;
}

}  // extern "C"
#pragma GCC visibility pop
