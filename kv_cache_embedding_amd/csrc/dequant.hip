// Reconstruction of TurboQuant codes ([review, QJL paragraph]: dequantization is the
// inverse rotation followed by renormalisation):
//   prod: xhat = nu (Pi^T chat + alpha gamma S^T (2z - 1)),   mse: xhat = nu Pi^T chat.
// One workgroup per vector; off the timed path, written for clarity (float32 FMA).
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kMaxD = 4096;

__global__ __launch_bounds__(256) void dequant_kernel(const unsigned char* __restrict__ params,
                                                      size_t off_pi, size_t off_s, int d, int b,
                                                      const uint32_t* __restrict__ codes,
                                                      const float* __restrict__ nu,
                                                      const float* __restrict__ gamma, int mode,
                                                      float* __restrict__ xhat) {
  const Header* hdr = reinterpret_cast<const Header*>(params);
  __shared__ float chat[kMaxD];
  __shared__ float sgn[kMaxD];
  const long v = blockIdx.x;
  const int groups = d / 32;
  const uint32_t* cv = codes + size_t(v) * groups * b;
  for (int t = threadIdx.x; t < d; t += blockDim.x) {
    const int w = t >> 5, bit = t & 31;
    int idx = 0;
    for (int p = 0; p < b - 1; ++p) idx |= int((cv[w * b + p] >> bit) & 1u) << p;
    chat[t] = hdr->cen[idx];
    sgn[t] = ((cv[w * b + b - 1] >> bit) & 1u) ? 1.f : -1.f;
  }
  __syncthreads();
  const float* Pi = reinterpret_cast<const float*>(params + off_pi);
  const float* S = reinterpret_cast<const float*>(params + off_s);
  const float scale = hdr->alpha * gamma[v];
  const float nv = nu[v];
  for (int k = threadIdx.x; k < d; k += blockDim.x) {
    float acc = 0.f;
    for (int t = 0; t < d; ++t) acc = fmaf(Pi[size_t(t) * d + k], chat[t], acc);
    if (mode == 0) {
      float qj = 0.f;
      for (int i = 0; i < d; ++i) qj = fmaf(S[size_t(i) * d + k], sgn[i], qj);
      acc = fmaf(scale, qj, acc);
    }
    xhat[size_t(v) * d + k] = nv * acc;
  }
}

}  // namespace

hipError_t launch_dequantize(const void* params, int d, int b, const uint32_t* codes,
                             const float* nu, const float* gamma, int64_t n, int mode,
                             float* xhat, hipStream_t s) {
  const Layout lay(d, b);
  const int block = d < 256 ? d : 256;
  for (int64_t v0 = 0; v0 < n; v0 += (int64_t(1) << 30)) {
    const int64_t cnt = (n - v0) < (int64_t(1) << 30) ? (n - v0) : (int64_t(1) << 30);
    hipLaunchKernelGGL(dequant_kernel, dim3(unsigned(cnt)), dim3(block), 0, s,
                       static_cast<const unsigned char*>(params), lay.off_pi, lay.off_s, d, b,
                       codes + size_t(v0) * (d / 32) * b, nu + v0, gamma + v0, mode,
                       xhat + size_t(v0) * d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tq
