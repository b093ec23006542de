// One decode step of attention over a TurboQuant KV cache: keys carry the inner-product
// quantizer, values the MSE quantizer alone ([review, problem statement]: the two
// quantizers; [news, KV-cache paragraph]: KV caches compressed to about 3 bits):
//   o[g][h] = sum_t softmax_t(scale * l[g][h][t]) * nu_t Pi_v^T chat_t,
// with l the unbiased logit estimate of the keys (the scoring kernels write it).  Pi_v^T is
// linear, so the weighted sum runs in the values' rotated coordinates and one inverse
// rotation per head finishes it:  o = Pi_v^T a,  a = sum_t p_t nu_t chat_t / sum_t p_t.
//
// attn_block_kernel: one workgroup per (group, pass of AH heads, block of KB keys).  Lanes
//   first hold one key each: scaled logits, the block maximum per head, the weights
//   p = exp(l - max) and p nu.  Then each wave walks its 64 keys with the lanes over the
//   coordinates (64 per step): the value's plane words are the same for every lane (scalar
//   loads), a lane picks its word and bit, looks the centroid up in LDS and accumulates it
//   times the key's weight for every head.  Out: per block and head the maximum, the sum of
//   p and the weighted sum of centroids.
// attn_combine_kernel: one workgroup per (group, head): merges the blocks (log-sum-exp) and
//   applies Pi_v^T (a row of Pi_v is contiguous, so thread j reads column j coalesced).
#include "tq_internal.h"

#include <cmath>

namespace tq {
namespace {

constexpr int AH = 4;      // query heads per pass
constexpr int KB = 256;    // keys per workgroup (64 per wave)
constexpr int CPL = 4;     // coordinates per lane per chunk (a chunk is 256 coordinates)

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <int BV>   // index planes of a value
__global__ __launch_bounds__(256) void attn_block_kernel(
    const unsigned char* __restrict__ params_v, const float* __restrict__ logits,
    const uint32_t* __restrict__ vcodes, const float* __restrict__ vnu, int d, long G, long T,
    long nkb, long passes, float scale, float* __restrict__ part_m, float* __restrict__ part_s,
    float* __restrict__ part_acc) {
  constexpr int L = 1 << BV;
  const Header* hdr = reinterpret_cast<const Header*>(params_v);
  __shared__ float cen[L];
  __shared__ float red[4][AH];
  __shared__ float accs[4][AH][64 * CPL];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar code loads
  if (tid < L) cen[tid] = hdr->cen[tid];

  const long kb = blockIdx.x % nkb;
  const long gp = blockIdx.x / nkb;
  const long g = gp / passes;
  const long h0 = (gp % passes) * AH;
  const long nh = G - h0 < AH ? G - h0 : AH;   // heads of this pass
  const long tw0 = kb * KB + wave * 64;        // first key of this wave
  const long t = tw0 + lane;                   // the lane's key in the prologue
  const bool valid = t < T;

  // prologue: scaled logits of the lane's key, block maximum per head
  float l[AH];
#pragma unroll
  for (int hh = 0; hh < AH; ++hh) {
    const long h = h0 + (hh < nh ? hh : nh - 1);
    l[hh] = valid ? scale * logits[size_t(g * G + h) * T + t] : -INFINITY;
    const float m = wave_max(l[hh]);
    if (lane == 0) red[wave][hh] = m;
  }
  __syncthreads();   // also publishes cen
  float M[AH];
#pragma unroll
  for (int hh = 0; hh < AH; ++hh)
    M[hh] = fmaxf(fmaxf(red[0][hh], red[1][hh]), fmaxf(red[2][hh], red[3][hh]));
  __syncthreads();
  const float nu_t = valid ? vnu[g * T + t] : 0.f;
  float w[AH];
#pragma unroll
  for (int hh = 0; hh < AH; ++hh) {
    const float p = valid ? __expf(l[hh] - M[hh]) : 0.f;
    w[hh] = p * nu_t;
    const float sp = wave_sum(p);
    if (lane == 0) red[wave][hh] = sp;
  }
  __syncthreads();
  const long prow = g * G + h0;                 // partial rows of this pass: prow + hh
#pragma unroll
  for (int hh = 0; hh < AH; ++hh) {
    if (tid == hh && hh < nh) {
      part_m[(prow + hh) * nkb + kb] = M[hh];
      part_s[(prow + hh) * nkb + kb] = (red[0][hh] + red[1][hh]) + (red[2][hh] + red[3][hh]);
    }
  }

  // weighted sum of the centroids of the wave's keys, 256 coordinates per chunk
  const int W = d / 32;
  const long nk = T - tw0 < 64 ? (T - tw0 > 0 ? T - tw0 : 0) : 64;
  for (int c0 = 0; c0 < d; c0 += 64 * CPL) {
    float acc[AH][CPL];
#pragma unroll
    for (int hh = 0; hh < AH; ++hh)
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[hh][i] = 0.f;
    for (int j = 0; j < nk; ++j) {
      float wj[AH];
#pragma unroll
      for (int hh = 0; hh < AH; ++hh)
        wj[hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w[hh]), j));
      const uint32_t* kc = vcodes + (size_t(g * T + tw0 + j) * W + c0 / 32) * BV;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        if (c0 + 64 * i >= d) break;            // uniform
        uint32_t idx = 0;
#pragma unroll
        for (int p = 0; p < BV; ++p) {
          const uint32_t wlo = kc[(2 * i) * BV + p], whi = kc[(2 * i + 1) * BV + p];
          const uint32_t word = lane < 32 ? wlo : whi;
          idx |= ((word >> (lane & 31)) & 1u) << p;
        }
        const float c = cen[idx];
#pragma unroll
        for (int hh = 0; hh < AH; ++hh) acc[hh][i] = fmaf(wj[hh], c, acc[hh][i]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < AH; ++hh)
#pragma unroll
      for (int i = 0; i < CPL; ++i) accs[wave][hh][64 * i + lane] = acc[hh][i];
    __syncthreads();
    for (int e = tid; e < AH * 64 * CPL; e += 256) {
      const int hh = e / (64 * CPL), c = e % (64 * CPL);
      if (hh < nh && c0 + c < d)
        part_acc[((prow + hh) * nkb + kb) * d + c0 + c] =
            (accs[0][hh][c] + accs[1][hh][c]) + (accs[2][hh][c] + accs[3][hh][c]);
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void attn_combine_kernel(
    const unsigned char* __restrict__ params_v, size_t off_pi, int d, long nkb,
    const float* __restrict__ part_m, const float* __restrict__ part_s,
    const float* __restrict__ part_acc, float* __restrict__ out) {
  extern __shared__ float a[];   // the head's combined rotated-space sum, d floats
  __shared__ float red[4];
  const long row = blockIdx.x;   // group * G + head
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* pm = part_m + row * nkb;
  const float* ps = part_s + row * nkb;
  float mx = -INFINITY;
  for (long k = tid; k < nkb; k += 256) mx = fmaxf(mx, pm[k]);
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.f;
  for (long k = tid; k < nkb; k += 256) sum += __expf(pm[k] - M) * ps[k];
  sum = wave_sum(sum);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  const float inv = 1.f / ((red[0] + red[1]) + (red[2] + red[3]));
  for (int c = tid; c < d; c += 256) {
    float v = 0.f;
    for (long k = 0; k < nkb; ++k) v = fmaf(__expf(pm[k] - M), part_acc[(row * nkb + k) * d + c], v);
    a[c] = v * inv;
  }
  __syncthreads();
  const float* Pi = reinterpret_cast<const float*>(params_v + off_pi);
  for (int j = tid; j < d; j += 256) {
    float v = 0.f;
    for (int i = 0; i < d; ++i) v = fmaf(Pi[size_t(i) * d + j], a[i], v);
    out[row * d + j] = v;
  }
}

}  // namespace

size_t attention_part_bytes(int d, int64_t groups, int64_t G, int64_t T) {
  const size_t nkb = size_t((T + KB - 1) / KB);
  return size_t(groups) * G * nkb * (2 + size_t(d)) * 4;
}

hipError_t launch_attention_values(const void* params_v, int d, int b_v, const float* logits,
                                   const uint32_t* vcodes, const float* vnu, int64_t groups,
                                   int64_t G, int64_t T, float scale, float* out, void* part,
                                   hipStream_t s) {
  const unsigned char* pv = static_cast<const unsigned char*>(params_v);
  const long nkb = (T + KB - 1) / KB;
  const long passes = (G + AH - 1) / AH;
  const size_t rows = size_t(groups) * G;
  float* part_m = static_cast<float*>(part);
  float* part_s = part_m + rows * nkb;
  float* part_acc = part_s + rows * nkb;
  const dim3 grid(unsigned(groups * passes * nkb));
  switch (b_v) {
    case 2: hipLaunchKernelGGL(attn_block_kernel<1>, grid, dim3(256), 0, s, pv, logits, vcodes, vnu, d,
                               long(G), long(T), nkb, passes, scale, part_m, part_s, part_acc); break;
    case 3: hipLaunchKernelGGL(attn_block_kernel<2>, grid, dim3(256), 0, s, pv, logits, vcodes, vnu, d,
                               long(G), long(T), nkb, passes, scale, part_m, part_s, part_acc); break;
    case 4: hipLaunchKernelGGL(attn_block_kernel<3>, grid, dim3(256), 0, s, pv, logits, vcodes, vnu, d,
                               long(G), long(T), nkb, passes, scale, part_m, part_s, part_acc); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const Layout lay(d, b_v);
  hipLaunchKernelGGL(attn_combine_kernel, dim3(unsigned(rows)), dim3(256), size_t(d) * 4, s, pv,
                     lay.off_pi, d, nkb, part_m, part_s, part_acc, out);
  return hipGetLastError();
}

bool attention_grid_fits(int64_t groups, int64_t G, int64_t T) {
  const int64_t nkb = (T + KB - 1) / KB;
  return groups * G < (int64_t(1) << 31) && groups * ((G + AH - 1) / AH) * nkb < (int64_t(1) << 31);
}

}  // namespace tq
