// Allocation-free decode scoring: tq_score_ip with its workspace taken from a fixed
// file-scope device array instead of a caller buffer, for callers that cannot allocate
// (code under HIP graph capture, tight serving loops).
//
// Each GPU the library runs on holds one copy of `scratch` (kScratchBytes) until the process
// ends.  Host code never passes the array's name to a kernel: the name is a host-side
// stand-in, so its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and cached.  Every call on one GPU shares that GPU's array; the
// scoring kernels overwrite what they read (the query operands are written by the query
// prep of the same call before the scan reads them), so nothing needs clearing between
// calls, but calls that overlap on one GPU race.
#include "tq.h"
#include "tq_internal.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;   // 8 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the device that owns `stream` (the current device for
// the null stream), looked up on the first call per device.
int scratch_for(void* stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return tq::report_error(TQ_EHIP, "tq_score_ip_noalloc: hipGetDevice failed");
  int dev = cur;
  if (stream) {
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev);
    if (e != hipSuccess) return tq::report_error(TQ_EHIP, "tq_score_ip_noalloc: hipStreamGetDevice failed");
  }
  if (dev < 0 || dev >= kMaxDevices) return tq::report_error(TQ_EUNSUPPORTED, "tq_score_ip_noalloc: device id");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess)
      return tq::report_error(TQ_EHIP, "tq_score_ip_noalloc: hipSetDevice failed");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p)
      return tq::report_error(TQ_EHIP, "tq_score_ip_noalloc: hipGetSymbolAddress(scratch) failed");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return TQ_OK;
}

}  // namespace

extern "C" {

size_t tq_score_noalloc_max_ws_bytes(void) { return kScratchBytes; }

int tq_score_ip_noalloc(const void* params, int d, int b, const void* q, int q_dtype,
                        const uint32_t* codes, const float* nu, const float* gamma, int64_t groups,
                        int64_t G, int64_t T, int mode, float* logits, void* stream) {
  // Empty or invalid sizes: tq_score_ip's own result (a no-op or its validation error),
  // before any device call.  A request beyond the fixed scratch fails the same way.
  const size_t need = (groups > 0 && G > 0 && T > 0) ? tq_score_ws_bytes(d, b, groups, G, T) : 0;
  if (need == 0)
    return tq_score_ip(params, d, b, q, q_dtype, codes, nu, gamma, groups, G, T, mode, logits, nullptr, 0,
                       stream);
  if (need > kScratchBytes) {
    char msg[200];
    std::snprintf(msg, sizeof(msg),
                  "tq_score_ip_noalloc: needs %zu bytes of scratch, the fixed scratch holds %zu "
                  "(use tq_score_ip with a workspace)", need, kScratchBytes);
    return tq::report_error(TQ_EUNSUPPORTED, msg);
  }
  void* ws = nullptr;
  const int rc = scratch_for(stream, &ws);
  if (rc != TQ_OK) return rc;
  // same validation, kernels and results as tq_score_ip; nothing on this path allocates
  return tq_score_ip(params, d, b, q, q_dtype, codes, nu, gamma, groups, G, T, mode, logits, ws,
                     kScratchBytes, stream);
}

}  // extern "C"
