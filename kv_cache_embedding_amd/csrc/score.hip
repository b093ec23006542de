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
#include "score_tile.h"

namespace tq {
namespace {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr int G = 4;
constexpr int RSRC_WORD3 = 0x00020000;   // raw (untyped) buffer resource, gfx9 family
// Bytes in flight: each wave keeps UNR key tiles of loads outstanding, and the key ranges
// are sized for WAVES_PER_CU waves per compute unit (both chosen by measurement on the
// long-context workload: 4 / 16 -> 8 / 32 took the scan from 280 to 258 us).
constexpr int UNR = 8;               // tiles loaded ahead per wave iteration
constexpr int WAVES_PER_CU = 32;     // key ranges (waves) per compute unit
constexpr float kDigitRange = 16000.f;


// ------------------------------------------------------------------------ query prep
// Two workgroups per virtual group (G query heads): type 0 forms qh = Pi q and the MSE rows
// of the MFMA A operands, type 1 forms sh = S q and the QJL rows; the two halves share
// nothing.  Thread i accumulates row i % D over a quarter of the columns (i / D), reading
// column k of the transposed matrix with one contiguous load per wave; its matrix loads are
// issued before the query loads and all of them before the first product, so the kernel
// waits on one round trip to memory.  Outputs: rows 4 h + part of the A operands in register
// order ws[g][m][lane][16 bytes] (m = 2 word + j; lane l holds row l % 16) and the
// epilogue constants per head.
constexpr int QP_THREADS = 512;
constexpr int QP_SLICES = QP_THREADS / D;     // column slices per row
template <int BITS>
__global__ __launch_bounds__(QP_THREADS) void score_qprep_kernel(const unsigned char* __restrict__ params,
                                                                 size_t off_tr,
                                                                 const void* __restrict__ q, int q_f32,
                                                                 unsigned char* __restrict__ ws) {
  constexpr int NW = score_words(BITS);
  constexpr int KS = D / QP_SLICES;        // columns per slice
  const Header* hdr = reinterpret_cast<const Header*>(params);
  const long g = blockIdx.x >> 1;
  const int type = blockIdx.x & 1;         // 0: Pi (MSE rows), 1: S (QJL rows)
  const int tid = threadIdx.x;
  // header fields, read once (a per-lane index into the header would be a memory load in
  // the packing loop)
  const float e0 = hdr->e[0], e1 = hdr->e[1], e2 = hdr->e[2], e3 = hdr->e[3];
  const float emax = hdr->emax, esum = hdr->esum, alpha = hdr->alpha;
  const int ne = hdr->ne;
  __shared__ float4 qv[D];                 // q of the G heads, column-major: qv[k] = heads 0..3
  __shared__ float part_sum[QP_SLICES][G][D];
  __shared__ float stats[G][2];            // per head: max |v|, sum v

  {
    const int row = tid % D, slice = tid / D;
    const float* col = reinterpret_cast<const float*>(params + off_tr) + size_t(type) * D * D +
                       size_t(slice) * KS * D + row;
    float m[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) m[k] = col[size_t(k) * D];
    for (int i = tid; i < G * D; i += QP_THREADS) {
      const long off = g * G * D + i;
      reinterpret_cast<float*>(qv)[(i % D) * G + i / D] =
          q_f32 ? static_cast<const float*>(q)[off]
                : __uint_as_float(uint32_t(static_cast<const uint16_t*>(q)[off]) << 16);
    }
    __syncthreads();                       // q is in LDS
    float acc[G] = {};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const float4 qk = qv[slice * KS + k];
      acc[0] = fmaf(m[k], qk.x, acc[0]);
      acc[1] = fmaf(m[k], qk.y, acc[1]);
      acc[2] = fmaf(m[k], qk.z, acc[2]);
      acc[3] = fmaf(m[k], qk.w, acc[3]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) part_sum[slice][h][row] = acc[h];
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += QP_THREADS) {
    float t = part_sum[0][i / D][i % D];
#pragma unroll
    for (int sl = 1; sl < QP_SLICES; ++sl) t += part_sum[sl][i / D][i % D];
    part_sum[0][i / D][i % D] = t;
  }
  __syncthreads();
  float (*v)[D] = part_sum[0];             // v[h][row]: qh (type 0) or sh (type 1)
  if (tid < G * 2 * 16) {
    // G heads x 2 statistics, 16 threads each
    const int h = tid / 32, stat = (tid / 16) % 2, sub = tid % 16;
    float r = 0.f;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) {
      const float x = v[h][sub + 16 * k];
      r = (stat == 0) ? fmaxf(r, fabsf(x)) : r + x;
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
      const float o = __shfl_xor(r, off, 16);
      r = (stat == 0) ? fmaxf(r, o) : r + o;
    }
    if (sub == 0) stats[h][stat] = r;
  }
  __syncthreads();

  unsigned char* base = ws + size_t(g) * score_ws_per_group(BITS);
  // A operand chunks of this half: per head 2 NW MFMAs x 4 K groups x 2 rows
  for (int item = tid; item < G * 2 * NW * 8; item += QP_THREADS) {
    const int h = item / (2 * NW * 8), r = item % (2 * NW * 8);
    const int m = r / 8, part = 2 * type + (r / 4) % 2, grp = r % 4;
    const int lane = 16 * grp + 4 * h + part;
    const int word = m / 2, j = m % 2;
    const bool mse_word = word < ne;
    const float ew = word == 0 ? e0 : word == 1 ? e1 : word == 2 ? e2 : e3;
    const float mx = type == 0 ? emax * stats[h][0] : stats[h][0];
    const float scale = mx > 0.f ? kDigitRange / mx : 1.f;
    // MSE rows carry e_word Pi q on the codebook words, QJL rows S q on the sign word; the
    // odd bit positions (j = 1) have weight 2, so their value is halved
    const float coef = (type == 0) ? (mse_word ? ew : 0.f) : (mse_word ? 0.f : 1.f);
    const float f = coef * scale * (j ? 0.5f : 1.f);
    const bool hi_part = (part % 2) == 0;
    uint32_t packed[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t dw = 0;
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        const int coord = 32 * grp + 8 * bi + 2 * k + j;
        const int vj = int(rintf(f * v[h][coord]));   // value as an integer: 128 hi + lo
        const int hi = (vj + 64) >> 7;
        const int lo = vj - 128 * hi;
        dw |= uint32_t(uint8_t(int8_t(hi_part ? hi : lo))) << (8 * bi);
      }
      packed[k] = dw;
    }
    reinterpret_cast<uint4*>(base)[m * 64 + lane] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  }
  // epilogue constants: l = nu (A wA - cA + gamma (B wB - cB)); type 0 writes (x, y),
  // type 1 writes (z, w)
  if (tid < G) {
    const int h = tid;
    float* c = reinterpret_cast<float*>(base + size_t(2 * NW) * 64 * 16) + 4 * h;
    if (type == 0) {
      const float ma = emax * stats[h][0];
      const float sa = ma > 0.f ? kDigitRange / ma : 1.f;
      c[0] = 2.f / sa;
      c[1] = esum * stats[h][1];
    } else {
      const float sb = stats[h][0] > 0.f ? kDigitRange / stats[h][0] : 1.f;
      c[2] = 2.f * alpha / sb;
      c[3] = alpha * stats[h][1];
    }
  }
}

// --------------------------------------------------------------------------- scoring
// BUF: the group's codes, nu, gamma and its quad's logits are addressed through buffer
// resources bounded by their arrays (byte offsets within 2^31, checked by the host): loads
// past the last key read zeros and stores past it are dropped, so no access sits under a
// branch (a branch around the store makes the compiler wait for every load in flight before
// it: 8.0 against 9.1 us per decode-layer scan).  Without BUF, 64-bit addresses and guards.
// Waves per SIMD that the scan keeps resident (the register budget): without branches
// between the tiles of an iteration the scheduler would hold all their MFMA accumulators at
// once and halve the occupancy of the narrower codes.
constexpr int scan_waves_per_simd(int bits) { return bits == 2 ? 6 : bits == 3 ? 5 : 4; }

template <int BITS, bool PROD, bool BUF>
__global__ __launch_bounds__(256, scan_waves_per_simd(BITS)) void score_kernel(const uint32_t* __restrict__ codes,
                                                     const float* __restrict__ nu,
                                                     const float* __restrict__ gamma,
                                                     const unsigned char* __restrict__ ws,
                                                     float* __restrict__ logits, long T, long qpg,
                                                     long tiles_per_group, long ranges_per_group,
                                                     long tiles_per_range, long total_ranges) {
  constexpr int NW = score_words(BITS);
  constexpr int NWU = PROD ? NW : NW - 1;     // MSE-only skips the sign plane
  const int lane = threadIdx.x & 63;
  const long range = long(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
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
  if constexpr (BUF) {
    // (ranges hold a multiple of UNR tiles, so a tile past t1 is past the group's last key)
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(gcodes), 0, int(T * (D / 32) * BITS * 4), RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t nrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(gnu), 0, int(T * 4),
                                                                        RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(ggm), 0, int(T * 4),
                                                                        RSRC_WORD3);
    // the quad's G rows of logits, [head][key]; a key past the end stores past the resource
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(logits + size_t(g) * G * T, 0,
                                                                        int(G * T * 4), RSRC_WORD3);
    for (long tb = t0; tb < t1; tb += UNR) {
      uint32_t w[UNR][BITS];
      float nk[UNR], gk[UNR];
      int key[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        key[u] = int((tb + u) * 16) + (lane & 15);
        const int off = (key[u] * (D / 32) + grp) * BITS * 4;
        if constexpr (BITS == 4) {
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(crs, off, 0, 0);
          w[u][0] = v[0]; w[u][1] = v[1]; w[u][2] = v[2]; w[u][3] = v[3];
        } else if constexpr (BITS == 3) {
          const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(crs, off, 0, 0);
          w[u][0] = v[0]; w[u][1] = v[1]; w[u][2] = v[2];
        } else {
          const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(crs, off, 0, 0);
          w[u][0] = v[0]; w[u][1] = v[1];
        }
        nk[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(nrs, key[u] * 4, 0, 0));
        gk[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(grs, key[u] * 4, 0, 0));
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const float l = score_tile_logit<BITS, PROD>(A, cst, w[u], nk[u], gk[u]);
        const int oo = key[u] < T ? (h * int(T) + key[u]) * 4 : int(G * T * 4);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l), ors, oo, 0, 0);
      }
    }
    return;
  }
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
      const float l = score_tile_logit<BITS, PROD>(A, cst, w[u], nk[u], gk[u]);
      if ((tb + u < t1) && key[u] < T) out[key[u]] = l;
    }
  }
}

template <int BITS>
hipError_t launch_b(const void* params, const void* q, int q_dtype, const uint32_t* codes,
                    const float* nu, const float* gamma, int64_t kv_groups, int64_t Gq, int64_t T,
                    int mode, float* logits, void* ws, hipStream_t s, int phases) {
  const Layout lay(D, BITS);
  const long qpg = long(Gq / G);
  const int64_t groups = kv_groups * qpg;       // virtual groups of 4 query heads
  if (phases & kScorePrep) {
    hipLaunchKernelGGL((score_qprep_kernel<BITS>), dim3(unsigned(2 * groups)), dim3(QP_THREADS), 0, s,
                       static_cast<const unsigned char*>(params), lay.off_tr, q,
                       q_dtype == 0 ? 1 : 0, static_cast<unsigned char*>(ws));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(phases & kScoreScan)) return hipSuccess;
  const long tiles_per_group = (T + 15) / 16;
  const long total_tiles = long(groups) * tiles_per_group;
  long tpr = (total_tiles + long(device_cu_count()) * WAVES_PER_CU - 1) / (long(device_cu_count()) * WAVES_PER_CU);
  if (tpr < 8) tpr = 8;
  tpr = (tpr + UNR - 1) / UNR * UNR;
  const long rpg = (tiles_per_group + tpr - 1) / tpr;
  const long total_ranges = long(groups) * rpg;
  const unsigned blocks = unsigned((total_ranges + 3) / 4);
  // buffer addressing needs every byte offset of a group's codes and of a quad's logits (keys
  // padded to whole tiles) within 2^31
  const int64_t Tp = tiles_per_group * 16;
  const bool buf = Tp * (D / 32) * BITS * 4 < (int64_t(1) << 31) && Tp * G * 4 < (int64_t(1) << 31);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, s, codes, nu, gamma,
                       static_cast<const unsigned char*>(ws), logits, long(T), qpg, tiles_per_group, rpg,
                       tpr, total_ranges);
  };
  if (mode == 0) {
    if (buf) go(score_kernel<BITS, true, true>); else go(score_kernel<BITS, true, false>);
  } else {
    if (buf) go(score_kernel<BITS, false, true>); else go(score_kernel<BITS, false, false>);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_d128(const void* params, int b, const void* q, int q_dtype,
                             const uint32_t* codes, const float* nu, const float* gamma,
                             int64_t groups, int64_t Gq, int64_t T, int mode, float* logits,
                             void* ws, hipStream_t s, int phases) {
  switch (b) {
    case 2: return launch_b<2>(params, q, q_dtype, codes, nu, gamma, groups, Gq, T, mode, logits, ws, s, phases);
    case 3: return launch_b<3>(params, q, q_dtype, codes, nu, gamma, groups, Gq, T, mode, logits, ws, s, phases);
    case 4: return launch_b<4>(params, q, q_dtype, codes, nu, gamma, groups, Gq, T, mode, logits, ws, s, phases);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
