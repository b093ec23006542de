// Attention logits over a TurboQuant key cache, d = 128, GQA groups of G query heads
// (G a multiple of 4: each quad of heads is scored as one "virtual group" over the keys).
//
// Estimate ([review, problem statement]: the query is exact, the key quantized, unbiased;
// [explainer, step 2]; [tldr, step 2]):
//   l = nu (<Pi q, chat> + alpha gamma <S q, 2z - 1>),  alpha = sqrt(pi/2)/m.
// With the index bits b_p and sigma_p = 2 b_p - 1, an odd-symmetric codebook is an exact
// Walsh sum over odd subsets P of the bits: chat = sum_P e_P prod_{p in P} sigma_p
// (b = 2: {b0}; b = 3: {b0}, {b1}; b = 4: {b0}, {b1}, {b2}, {b0 b1 b2}, the last plane being
// b0 ^ b1 ^ b2).  Hence
//   <Pi q, chat> = 2 sum_P e_P <Pi q, bits_P> - (sum_P e_P) sum_t (Pi q)_t
//   <S q, 2z-1>  = 2 <S q, z> - sum_t (S q)_t,
// and every term is a sum of query values selected by one bit plane of the key.  These
// masked sums run on v_mfma_i32_16x16x64_i8 with
//   A (16 rows x K) = query values as exact int8 digits (value = 128 hi + lo), rows
//                     4 h + {MSE hi, MSE lo, QJL hi, QJL lo} for query head h,
//   B (K x 16 keys) = key bits, bytes holding 0/1 (or 0/2 for the odd bit positions,
//                     whose query values are stored halved so the product is exact).
// In the 16x16 accumulator layout lane l holds key l % 16 and rows 4 (l/16) .. +3, i.e.
// the four partial sums of one logit, so the epilogue is lane-local.
// The key planes stream from HBM once (coalesced 16 B per lane per 16-key tile); the
// query operand stays in registers for the wave's whole key range.
#include "tq_internal.h"

namespace tq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr int G = 4;
constexpr int UNR = 4;        // tiles loaded ahead per wave iteration
constexpr float kDigitRange = 16000.f;

int cu_count_s() {
  static int cached = 0;
  if (!cached) {
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      c = 256;
    cached = c;
  }
  return cached;
}

// ------------------------------------------------------------------------ query prep
// One workgroup per (virtual group, query head h): qh = Pi q, sh = S q (float32, one row
// per thread), the head's scales, then its rows 4h .. 4h+3 of the MFMA A operands in
// register order ws[g][m][lane][16 bytes] (m = 2 word + j; lane l holds row l % 16), and
// its four epilogue constants.
template <int BITS>
__global__ __launch_bounds__(256) void score_qprep_kernel(const unsigned char* __restrict__ params,
                                                           size_t off_pi, size_t off_s,
                                                           const void* __restrict__ q, int q_f32,
                                                           unsigned char* __restrict__ ws) {
  constexpr int NW = score_words(BITS);
  const Header* hdr = reinterpret_cast<const Header*>(params);
  const long g = blockIdx.x / G;
  const int h = blockIdx.x % G;
  __shared__ float qv[D];
  __shared__ float qh[D];
  __shared__ float sh[D];
  __shared__ float stats[4];   // max|qh|, sum qh, max|sh|, sum sh

  if (threadIdx.x < D) {
    const long off = (g * G + h) * D + threadIdx.x;
    qv[threadIdx.x] = q_f32 ? static_cast<const float*>(q)[off]
                            : __uint_as_float(uint32_t(static_cast<const uint16_t*>(q)[off]) << 16);
  }
  __syncthreads();
  {
    // thread i: row i % D of Pi (i < D) or of S (i >= D)
    const int row = threadIdx.x % D, type = threadIdx.x / D;
    const float4* src = reinterpret_cast<const float4*>(params + (type ? off_s : off_pi)) +
                        size_t(row) * (D / 4);
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j4 = 0; j4 < D / 4; j4 += 2) {
      const float4 m0 = src[j4], m1 = src[j4 + 1];
      a0 = fmaf(m0.x, qv[4 * j4 + 0], a0);
      a1 = fmaf(m0.y, qv[4 * j4 + 1], a1);
      a0 = fmaf(m0.z, qv[4 * j4 + 2], a0);
      a1 = fmaf(m0.w, qv[4 * j4 + 3], a1);
      a0 = fmaf(m1.x, qv[4 * j4 + 4], a0);
      a1 = fmaf(m1.y, qv[4 * j4 + 5], a1);
      a0 = fmaf(m1.z, qv[4 * j4 + 6], a0);
      a1 = fmaf(m1.w, qv[4 * j4 + 7], a1);
    }
    (type ? sh : qh)[row] = a0 + a1;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    // 4 statistics, 16 threads each
    const int stat = threadIdx.x / 16, sub = threadIdx.x % 16;
    const float* v = (stat < 2) ? qh : sh;
    float r = 0.f;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) {
      const float x = v[sub + 16 * k];
      r = (stat % 2 == 0) ? fmaxf(r, fabsf(x)) : r + x;
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
      const float o = __shfl_xor(r, off, 16);
      r = (stat % 2 == 0) ? fmaxf(r, o) : r + o;
    }
    if (sub == 0) stats[stat] = r;
  }
  __syncthreads();

  const int ne = hdr->ne;
  const float ma = hdr->emax * stats[0];
  const float sa = ma > 0.f ? kDigitRange / ma : 1.f;
  const float sb = stats[2] > 0.f ? kDigitRange / stats[2] : 1.f;
  unsigned char* base = ws + size_t(g) * score_ws_per_group(BITS);
  // this head's A operand chunks: 2 NW MFMAs x 4 K groups x 4 rows
  for (int item = threadIdx.x; item < 2 * NW * 16; item += 256) {
    const int m = item / 16, part = (item / 4) % 4, grp = item % 4;
    const int lane = 16 * grp + 4 * h + part;
    const int word = m / 2, j = m % 2;
    const bool mse_word = word < ne;
    uint32_t packed[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t dw = 0;
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        const int coord = 32 * grp + 8 * bi + 2 * k + j;
        float xval = 0.f;
        if (mse_word && part < 2) xval = hdr->e[word] * qh[coord] * sa;
        if (!mse_word && part >= 2) xval = sh[coord] * sb;
        // value as an integer; odd bit positions carry weight 2, so keep them even
        const int v = (j == 0) ? int(rintf(xval)) : 2 * int(rintf(0.5f * xval));
        const int vj = v >> j;
        const int hi = (vj + 64) >> 7;
        const int lo = vj - 128 * hi;
        const int digit = (part % 2 == 0) ? hi : lo;
        dw |= uint32_t(uint8_t(int8_t(digit))) << (8 * bi);
      }
      packed[k] = dw;
    }
    reinterpret_cast<uint4*>(base)[m * 64 + lane] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  }
  // epilogue constants: l = nu (A wA - cA + gamma (B wB - cB))
  if (threadIdx.x == 0) {
    float4 c;
    c.x = 2.f / sa;
    c.y = hdr->esum * stats[1];
    c.z = 2.f * hdr->alpha / sb;
    c.w = hdr->alpha * stats[3];
    reinterpret_cast<float4*>(base + size_t(2 * NW) * 64 * 16)[h] = c;
  }
}

// --------------------------------------------------------------------------- scoring
template <int BITS, bool PROD>
__global__ __launch_bounds__(256) void score_kernel(const uint32_t* __restrict__ codes,
                                                     const float* __restrict__ nu,
                                                     const float* __restrict__ gamma,
                                                     const unsigned char* __restrict__ ws,
                                                     float* __restrict__ logits, long T, long qpg,
                                                     long tiles_per_group, long ranges_per_group,
                                                     long tiles_per_range, long total_ranges) {
  constexpr int NW = score_words(BITS);
  constexpr int NWU = PROD ? NW : NW - 1;     // MSE-only skips the sign plane
  const int lane = threadIdx.x & 63;
  const long range = long(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (range >= total_ranges) return;
  const long g = range / ranges_per_group;    // virtual group: key group g / qpg, quad g % qpg
  const long kg = g / qpg;
  const long t0 = (range % ranges_per_group) * tiles_per_range;
  long t1 = t0 + tiles_per_range;
  if (t1 > tiles_per_group) t1 = tiles_per_group;

  const unsigned char* base = ws + size_t(g) * score_ws_per_group(BITS);
  v4i A[2 * NW];
#pragma unroll
  for (int m = 0; m < 2 * NWU; ++m) A[m] = reinterpret_cast<const v4i*>(base)[m * 64 + lane];
  const int h = lane >> 4;
  const float4 cst = reinterpret_cast<const float4*>(base + size_t(2 * NW) * 64 * 16)[h];

  const int grp = lane >> 4;
  const uint32_t* gcodes = codes + size_t(kg) * T * (D / 32) * BITS;
  const float* gnu = nu + size_t(kg) * T;
  const float* ggm = gamma + size_t(kg) * T;
  float* out = logits + (size_t(g) * G + h) * T;

  for (long tb = t0; tb < t1; tb += UNR) {
    uint32_t w[UNR][BITS];
    float nk[UNR], gk[UNR];
    long key[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      key[u] = (tb + u) * 16 + (lane & 15);
      const bool ok = (tb + u < t1) && key[u] < T;
      if (ok) {
        const uint32_t* src = gcodes + (key[u] * (D / 32) + grp) * BITS;
        if constexpr (BITS == 4) {
          const uint4 v = *reinterpret_cast<const uint4*>(src);
          w[u][0] = v.x; w[u][1] = v.y; w[u][2] = v.z; w[u][3] = v.w;
        } else if constexpr (BITS == 2) {
          const uint2 v = *reinterpret_cast<const uint2*>(src);
          w[u][0] = v.x; w[u][1] = v.y;
        } else {
#pragma unroll
          for (int p = 0; p < BITS; ++p) w[u][p] = src[p];
        }
        nk[u] = gnu[key[u]];
        gk[u] = ggm[key[u]];
      } else {
#pragma unroll
        for (int p = 0; p < BITS; ++p) w[u][p] = 0u;
        nk[u] = 0.f;
        gk[u] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      uint32_t word[NW];
      if constexpr (BITS == 4) {
        word[0] = w[u][0]; word[1] = w[u][1]; word[2] = w[u][2];
        word[3] = w[u][0] ^ w[u][1] ^ w[u][2];
        word[4] = w[u][3];
      } else {
#pragma unroll
        for (int p = 0; p < BITS; ++p) word[p] = w[u][p];
      }
      v4i acc = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < NWU; ++i) {
        const uint32_t W = word[i];
        const uint32_t s2 = W >> 2, s4 = W >> 4, s6 = W >> 6;
        const v4i b0 = {int(W & 0x01010101u), int(s2 & 0x01010101u), int(s4 & 0x01010101u),
                        int(s6 & 0x01010101u)};
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[2 * i], b0, acc, 0, 0, 0);
        const v4i b1 = {int(W & 0x02020202u), int(s2 & 0x02020202u), int(s4 & 0x02020202u),
                        int(s6 & 0x02020202u)};
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[2 * i + 1], b1, acc, 0, 0, 0);
      }
      const int ai = acc[0] * 128 + acc[1];
      float l = fmaf(float(ai), cst.x, -cst.y);
      if constexpr (PROD) {
        const int bi = acc[2] * 128 + acc[3];
        l = fmaf(gk[u], fmaf(float(bi), cst.z, -cst.w), l);
      }
      l *= nk[u];
      if ((tb + u < t1) && key[u] < T) out[key[u]] = l;
    }
  }
}

template <int BITS>
hipError_t launch_b(const void* params, const void* q, int q_dtype, const uint32_t* codes,
                    const float* nu, const float* gamma, int64_t kv_groups, int64_t Gq, int64_t T,
                    int mode, float* logits, void* ws, hipStream_t s) {
  const Layout lay(D, BITS);
  const long qpg = long(Gq / G);
  const int64_t groups = kv_groups * qpg;       // virtual groups of 4 query heads
  hipLaunchKernelGGL((score_qprep_kernel<BITS>), dim3(unsigned(groups * G)), dim3(256), 0, s,
                     static_cast<const unsigned char*>(params), lay.off_pi, lay.off_s, q,
                     q_dtype == 0 ? 1 : 0, static_cast<unsigned char*>(ws));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long tiles_per_group = (T + 15) / 16;
  const long total_tiles = long(groups) * tiles_per_group;
  long tpr = (total_tiles + long(cu_count_s()) * 16 - 1) / (long(cu_count_s()) * 16);
  if (tpr < 8) tpr = 8;
  tpr = (tpr + UNR - 1) / UNR * UNR;
  const long rpg = (tiles_per_group + tpr - 1) / tpr;
  const long total_ranges = long(groups) * rpg;
  const unsigned blocks = unsigned((total_ranges + 3) / 4);
  if (mode == 0)
    hipLaunchKernelGGL((score_kernel<BITS, true>), dim3(blocks), dim3(256), 0, s, codes, nu, gamma,
                       static_cast<const unsigned char*>(ws), logits, long(T), qpg, tiles_per_group,
                       rpg, tpr, total_ranges);
  else
    hipLaunchKernelGGL((score_kernel<BITS, false>), dim3(blocks), dim3(256), 0, s, codes, nu, gamma,
                       static_cast<const unsigned char*>(ws), logits, long(T), qpg, tiles_per_group,
                       rpg, tpr, total_ranges);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_d128(const void* params, int b, const void* q, int q_dtype,
                             const uint32_t* codes, const float* nu, const float* gamma,
                             int64_t groups, int64_t Gq, int64_t T, int mode, float* logits,
                             void* ws, hipStream_t s) {
  switch (b) {
    case 2: return launch_b<2>(params, q, q_dtype, codes, nu, gamma, groups, Gq, T, mode, logits, ws, s);
    case 3: return launch_b<3>(params, q, q_dtype, codes, nu, gamma, groups, Gq, T, mode, logits, ws, s);
    case 4: return launch_b<4>(params, q, q_dtype, codes, nu, gamma, groups, Gq, T, mode, logits, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
