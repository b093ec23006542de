// Top-k search for k beyond the lists the fused scan keeps (32 < k <= 1024): the estimates
// of a batch of queries against every key are written to the workspace by the general
// scoring kernels (one group, the batch's queries as its heads), then one workgroup per
// query selects and sorts its k best ([news, vector-search paragraph]: a flat scan over the
// codes).  Order: decreasing score, equal scores by increasing key index.
//
// Selection of one query's k best among n scores:
//   1. the k-th largest score, as an order-preserving 32-bit key, by four radix passes of
//      8 bits over the scores (LDS histogram per pass);
//   2. every score above it, and the smallest-index scores equal to it until k are taken:
//      each thread owns a contiguous index range, counts both kinds, and two exclusive
//      prefix sums over the threads give every element its output slot in index order;
//   3. a bitonic sort of the k (score, index) pairs in LDS.
#include "tq_internal.h"

#include <climits>
#include <cmath>

namespace tq {
namespace {

constexpr int ST = 1024;           // threads of a selection workgroup
constexpr int KCAP = 1024;         // largest k of this path
constexpr size_t BATCH_SCORE_BYTES = size_t(256) << 20;   // scores of one query batch

// Larger score -> larger key; -0 is folded onto +0 so that the two compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of one value per thread over the workgroup (ST threads); also
// returns the total.  Uses scan[ST] of LDS.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scan, uint32_t& total) {
  const int tid = threadIdx.x;
  scan[tid] = v;
  __syncthreads();
  for (int off = 1; off < ST; off <<= 1) {
    const uint32_t add = tid >= off ? scan[tid - off] : 0u;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  total = scan[ST - 1];
  const uint32_t incl = scan[tid];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(ST) void select_topk_kernel(const float* __restrict__ scores, long n,
                                                         int k, long q0, int32_t* __restrict__ idx_out,
                                                         float* __restrict__ score_out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan[ST];
  __shared__ float sel_s[KCAP];
  __shared__ int32_t sel_i[KCAP];
  __shared__ uint32_t sh_pre, sh_need;
  const int tid = threadIdx.x;
  const float* s = scores + size_t(blockIdx.x) * n;

  // 1. radix select of the k-th largest key
  uint32_t pre = 0, mask = 0, need = uint32_t(k);
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (long i = tid; i < n; i += ST) {
      const uint32_t u = order_key(s[i]);
      if ((u & mask) == pre) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t above = 0;
      int bin = 255;
      for (; bin > 0; --bin) {
        if (above + hist[bin] >= need) break;
        above += hist[bin];
      }
      sh_pre = pre | (uint32_t(bin) << shift);
      sh_need = need - above;
    }
    __syncthreads();
    pre = sh_pre;
    need = sh_need;
    mask |= 255u << shift;
    __syncthreads();
  }
  // pre is the key of the k-th largest score; need of the scores equal to it are taken

  // 2. collect, in index order within each kind
  const long per = (n + ST - 1) / ST;
  const long lo = tid * per, hi = lo + per < n ? lo + per : n;
  uint32_t ngt = 0, neq = 0;
  for (long i = lo; i < hi; ++i) {
    const uint32_t u = order_key(s[i]);
    ngt += u > pre ? 1u : 0u;
    neq += u == pre ? 1u : 0u;
  }
  uint32_t tot_gt = 0, tot_eq = 0;
  uint32_t pos_gt = block_exclusive_scan(ngt, scan, tot_gt);
  uint32_t pos_eq = block_exclusive_scan(neq, scan, tot_eq);
  for (long i = lo; i < hi && (ngt > 0 || (neq > 0 && pos_eq < need)); ++i) {
    const float v = s[i];
    const uint32_t u = order_key(v);
    if (u > pre) {
      sel_s[pos_gt] = v;
      sel_i[pos_gt] = int32_t(i);
      ++pos_gt;
      --ngt;
    } else if (u == pre) {
      if (pos_eq < need) {
        sel_s[tot_gt + pos_eq] = v;
        sel_i[tot_gt + pos_eq] = int32_t(i);
      }
      ++pos_eq;
      --neq;
    }
  }
  // tot_gt + need == k
  __syncthreads();

  // 3. bitonic sort of the k pairs (padded to a power of two): decreasing score, then
  // increasing index
  int P = 1;
  while (P < k) P <<= 1;
  for (int i = k + tid; i < P; i += ST) {
    sel_s[i] = -INFINITY;
    sel_i[i] = INT_MAX;
  }
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P; i += ST) {
        const int j = i ^ stride;
        if (j > i) {
          const bool desc = (i & size) == 0;     // this pair's run sorts best-first
          const float si = sel_s[i], sj = sel_s[j];
          const int32_t ii = sel_i[i], ij = sel_i[j];
          const bool j_first = sj > si || (sj == si && ij < ii);   // j ranks before i
          if (j_first == desc) {
            sel_s[i] = sj;
            sel_s[j] = si;
            sel_i[i] = ij;
            sel_i[j] = ii;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < k; i += ST) {
    idx_out[size_t(q0 + blockIdx.x) * k + i] = sel_i[i];
    score_out[size_t(q0 + blockIdx.x) * k + i] = sel_s[i];
  }
}

long batch_queries(int64_t nq, int64_t n) {
  long qb = long(BATCH_SCORE_BYTES / (size_t(n) * 4));
  if (qb < 1) qb = 1;
  return qb < nq ? qb : long(nq);
}

}  // namespace

size_t topk_large_ws_bytes(int d, int64_t nq, int64_t n) {
  const long qb = batch_queries(nq, n);
  return align256(size_t(qb) * n * 4) + align256(score_generic_ws_bytes(d, 1, qb));
}

hipError_t launch_topk_large(const void* params, int d, int b, const void* q, int q_dtype,
                             int64_t nq, const uint32_t* codes, const float* nu, const float* gamma,
                             int64_t n, int k, int mode, int32_t* idx, float* score, void* ws,
                             hipStream_t s) {
  if (k > KCAP) return hipErrorNotSupported;
  const long qb = batch_queries(nq, n);
  if (!score_generic_grid_fits(1, qb, n)) return hipErrorNotSupported;
  unsigned char* w = static_cast<unsigned char*>(ws);
  float* scores = reinterpret_cast<float*>(w);
  void* sws = w + align256(size_t(qb) * n * 4);
  const size_t qrow = size_t(d) * (q_dtype == 0 ? 4 : 2);
  for (long q0 = 0; q0 < nq; q0 += qb) {
    const long nb = nq - q0 < qb ? nq - q0 : qb;
    const void* qb_ptr = static_cast<const unsigned char*>(q) + size_t(q0) * qrow;
    hipError_t e = launch_score_generic(params, d, b, qb_ptr, q_dtype, codes, nu, gamma, 1, nb, n,
                                        mode, scores, sws, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(select_topk_kernel, dim3(unsigned(nb)), dim3(ST), 0, s, scores, long(n), k, q0,
                       idx, score);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tq
