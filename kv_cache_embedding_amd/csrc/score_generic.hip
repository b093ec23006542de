// Attention logits over a TurboQuant key cache for the shapes the d = 128 kernel does not
// take: any d that is a multiple of 64, any number G of query heads per group.
//
// Estimate ([review, problem statement]: the query is exact, the key quantized, unbiased;
// [tldr, step 2]):
//   l = nu (<Pi q, chat> + alpha gamma <S q, 2z - 1>),  alpha = sqrt(pi/2)/m,
// with <S q, 2z - 1> = 2 sum_{t : z_t = 1} (S q)_t - sum_t (S q)_t, so per coordinate a key
// needs one centroid times (Pi q)_t and one sign-bit-selected (S q)_t for each head.
//
// generic_qprep_kernel: qh = Pi q and sh = S q in float32, one workgroup per (group, head);
//   a wave forms one output as a 64-lane strided dot product over one row of Pi or S (rows
//   are contiguous), and the workgroup sums sh.
// generic_score_kernel: one lane per key and HB heads per pass.  The key's plane words of a
//   32-coordinate group are loaded once; per coordinate the index bits pick the centroid
//   from an LDS table and the sign bit weights sh.  The query values are the same for every
//   lane of a workgroup, so they come in through scalar loads.
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int HB = 4;        // query heads per pass of the scoring kernel
constexpr int KEYS = 256;    // keys per workgroup (one per lane)

__global__ __launch_bounds__(256) void generic_qprep_kernel(
    const unsigned char* __restrict__ params, size_t off_pi, size_t off_s, int d, long qpitch,
    const void* __restrict__ q, int q_f32, float* __restrict__ qs, float* __restrict__ ssum) {
  extern __shared__ float qv[];            // the query row, d floats
  __shared__ float red[4];
  const long row = blockIdx.x;             // (group, head) = group * G + head
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int k = tid; k < d; k += 256) {
    if (q_f32) {
      qv[k] = static_cast<const float*>(q)[row * qpitch + k];
    } else {
      const uint32_t hbits = static_cast<const uint16_t*>(q)[row * qpitch + k];
      qv[k] = __uint_as_float(hbits << 16);
    }
  }
  __syncthreads();
  const float* Pi = reinterpret_cast<const float*>(params + off_pi);
  const float* S = reinterpret_cast<const float*>(params + off_s);
  float sacc = 0.f;
  for (int o = wave; o < 2 * d; o += 4) {  // output o: row o of Pi (o < d), else row o - d of S
    const bool is_s = o >= d;
    const int r = is_s ? o - d : o;
    const float* m = (is_s ? S : Pi) + size_t(r) * d;
    float acc = 0.f;
    for (int k = lane; k < d; k += 64) acc = fmaf(m[k], qv[k], acc);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) qs[(row * 2 + (is_s ? 1 : 0)) * d + r] = acc;
    if (is_s) sacc += acc;
  }
  if (lane == 0) red[wave] = sacc;
  __syncthreads();
  if (tid == 0) ssum[row] = (red[0] + red[1]) + (red[2] + red[3]);
}

// grid: one workgroup per (group, head pass, block of KEYS keys), flattened into x.  ACC adds
// the estimate to the logits already there (the channel groups of a fractional rate).
template <int BITS, bool PROD, bool ACC>
__global__ __launch_bounds__(KEYS) void generic_score_kernel(
    const unsigned char* __restrict__ params, const float* __restrict__ qs,
    const float* __restrict__ ssum, const uint32_t* __restrict__ codes,
    const float* __restrict__ nu, const float* __restrict__ gamma, int d, long G, long T,
    long kblocks, long passes, float* __restrict__ logits) {
  constexpr int L = 1 << (BITS - 1);
  const Header* hdr = reinterpret_cast<const Header*>(params);
  __shared__ float cen[L];
  const int tid = threadIdx.x;
  if (tid < L) cen[tid] = hdr->cen[tid];
  const float alpha = hdr->alpha;
  __syncthreads();

  const long blk = blockIdx.x;
  const long kb = blk % kblocks;
  const long gp = blk / kblocks;           // group * passes + pass
  const long g = gp / passes;
  const long h0 = (gp % passes) * HB;
  const long nh = G - h0 < HB ? G - h0 : HB;   // heads of this pass
  const long t = kb * KEYS + tid;
  const bool valid = t < T;
  const long key = g * T + (valid ? t : T - 1);  // ragged block: read a valid key, store nothing
  const int words = d / 32;
  const uint32_t* kc = codes + size_t(key) * words * BITS;
  // query rows of the pass; heads past G repeat the last one (results not stored)
  const float* qrow[HB];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    const long h = h0 + (hh < nh ? hh : nh - 1);
    qrow[hh] = qs + size_t(g * G + h) * 2 * d;
  }
  float mse[HB], zsum[HB];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) mse[hh] = zsum[hh] = 0.f;
  for (int w = 0; w < words; ++w) {
    uint32_t pl[BITS];
#pragma unroll
    for (int p = 0; p < BITS; ++p) pl[p] = kc[w * BITS + p];
#pragma unroll 4
    for (int e = 0; e < 32; ++e) {
      const int c0 = 32 * w + e;
      uint32_t idx = 0;
#pragma unroll
      for (int p = 0; p < BITS - 1; ++p) idx |= ((pl[p] >> e) & 1u) << p;
      const float c = cen[idx];
      const float zf = float((pl[BITS - 1] >> e) & 1u);
#pragma unroll
      for (int hh = 0; hh < HB; ++hh) {
        mse[hh] = fmaf(qrow[hh][c0], c, mse[hh]);
        if constexpr (PROD) zsum[hh] = fmaf(qrow[hh][d + c0], zf, zsum[hh]);
      }
    }
  }
  if (!valid) return;
  const float n_k = nu[key], g_k = gamma[key];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    if (hh >= nh) break;
    const long h = h0 + hh;
    float l = mse[hh];
    if constexpr (PROD) l = fmaf(alpha * g_k, 2.f * zsum[hh] - ssum[g * G + h], l);
    float* dst = logits + size_t(g * G + h) * T + t;
    *dst = ACC ? *dst + n_k * l : n_k * l;
  }
}

template <int BITS, bool ACC>
hipError_t launch_b(const void* params_v, int d, const void* q, int q_dtype, long qpitch,
                    const uint32_t* codes, const float* nu, const float* gamma, int64_t groups,
                    int64_t G, int64_t T, int mode, float* logits, void* ws, hipStream_t s) {
  const unsigned char* params = static_cast<const unsigned char*>(params_v);
  const Layout lay(d, BITS);
  float* qs = static_cast<float*>(ws);
  float* ssum = qs + size_t(groups) * G * 2 * d;
  const long rows = long(groups) * G;
  hipLaunchKernelGGL(generic_qprep_kernel, dim3(unsigned(rows)), dim3(256), size_t(d) * 4, s, params,
                     lay.off_pi, lay.off_s, d, qpitch, q, q_dtype == 0 ? 1 : 0, qs, ssum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long kblocks = (T + KEYS - 1) / KEYS;
  const long passes = (G + HB - 1) / HB;
  const dim3 grid(unsigned(groups * passes * kblocks));
  if (mode == 0)
    hipLaunchKernelGGL((generic_score_kernel<BITS, true, ACC>), grid, dim3(KEYS), 0, s, params, qs, ssum,
                       codes, nu, gamma, d, long(G), long(T), kblocks, passes, logits);
  else
    hipLaunchKernelGGL((generic_score_kernel<BITS, false, ACC>), grid, dim3(KEYS), 0, s, params, qs, ssum,
                       codes, nu, gamma, d, long(G), long(T), kblocks, passes, logits);
  return hipGetLastError();
}

}  // namespace

size_t score_generic_ws_bytes(int d, int64_t groups, int64_t G) {
  return size_t(groups) * G * (2 * size_t(d) + 1) * 4;
}

bool score_generic_grid_fits(int64_t groups, int64_t G, int64_t T) {
  const int64_t blocks = groups * ((G + HB - 1) / HB) * ((T + KEYS - 1) / KEYS);
  return groups * G < (int64_t(1) << 31) && blocks < (int64_t(1) << 31);
}

hipError_t launch_score_generic(const void* params, int d, int b, const void* q, int q_dtype,
                                const uint32_t* codes, const float* nu, const float* gamma,
                                int64_t groups, int64_t G, int64_t T, int mode, float* logits,
                                void* ws, hipStream_t s, int64_t qpitch, bool accumulate) {
  const long qp = qpitch > 0 ? long(qpitch) : long(d);
#define TQ_GEN_CASE(B)                                                                            \
  case B:                                                                                         \
    return accumulate                                                                             \
               ? launch_b<B, true>(params, d, q, q_dtype, qp, codes, nu, gamma, groups, G, T, mode, \
                                   logits, ws, s)                                                 \
               : launch_b<B, false>(params, d, q, q_dtype, qp, codes, nu, gamma, groups, G, T,      \
                                    mode, logits, ws, s);
  switch (b) {
    TQ_GEN_CASE(2)
    TQ_GEN_CASE(3)
    TQ_GEN_CASE(4)
    default: return hipErrorInvalidValue;
  }
#undef TQ_GEN_CASE
}

}  // namespace tq
