// Quantize-on-write of one token per group into an existing cache ([explainer, step 1]: the
// quantizer is data-oblivious, so a new token is encoded on arrival with no calibration and
// no other token involved): the groups' vectors are encoded into the workspace by the bulk
// encoders, then this kernel writes vector g's code words, nu and gamma into cache slot
// (g, pos) of caches laid out [groups][cap].
#include "tq_internal.h"

namespace tq {
namespace {

// One workgroup per group; words = d / 32 * planes code words per vector.
__global__ __launch_bounds__(64) void scatter_slot_kernel(const uint32_t* __restrict__ src_codes,
                                                          const float* __restrict__ src_nu,
                                                          const float* __restrict__ src_gamma,
                                                          int words, long cap, long pos,
                                                          uint32_t* __restrict__ codes,
                                                          float* __restrict__ nu,
                                                          float* __restrict__ gamma) {
  const long g = blockIdx.x;
  const long slot = g * cap + pos;
  for (int i = threadIdx.x; i < words; i += 64) codes[slot * words + i] = src_codes[g * words + i];
  if (threadIdx.x == 0) {
    nu[slot] = src_nu[g];
    if (gamma) gamma[slot] = src_gamma[g];
  }
}

}  // namespace

hipError_t launch_scatter_slot(const uint32_t* src_codes, const float* src_nu,
                               const float* src_gamma, int words, int64_t groups, int64_t cap,
                               int64_t pos, uint32_t* codes, float* nu, float* gamma,
                               hipStream_t s) {
  hipLaunchKernelGGL(scatter_slot_kernel, dim3(unsigned(groups)), dim3(64), 0, s, src_codes, src_nu,
                     src_gamma, words, long(cap), long(pos), codes, nu, gamma);
  return hipGetLastError();
}

}  // namespace tq
