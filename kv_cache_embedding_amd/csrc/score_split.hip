// Attention logits over a fractional-rate key cache split 64 + 64: channels 0..63 and 64..127
// of d = 128 are two TurboQuant instances of d = 64 (each with its own rotation, QJL matrix and
// codebook, at b0 and b1 bits), and a logit is the sum of the two groups' estimates
// ([review, experiments paragraph]: 2.5 and 3.5 bits per channel from two channel groups).
//
// Scan layout.  In the d = 128 scorer the four 16-lane chunks of an MFMA's K = 64 are the four
// 32-coordinate groups and a plane word takes two MFMAs (even bits, odd bits).  Here one MFMA
// covers a whole 64-channel group: chunk c of K holds coordinate group c / 2 of that channel
// group and bit parity c % 2, so a word of one channel group takes one MFMA whose A operand
// has no zero half, and each channel group's sums land in an accumulator of their own (its
// estimate takes its own nu, gamma, digit scale and constants).  A lane loads both channel
// groups' words of its key and coordinate group; lanes 16 apart load the same words and keep
// the other bit parity.  The query is rounded to digits per (head, channel group) row exactly
// as in the d = 128 scorer.
#include "score_tile.h"

namespace tq {
namespace {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int DG = 64;                 // channels per group (two groups: d = 128)
constexpr int G = 4;                   // query heads per operand block (a quad)
constexpr int WAVES_PER_CU = 32;       // key ranges (waves) per compute unit
constexpr float kDigitRange = 16000.f;
constexpr int RSRC_WORD3 = 0x00020000;   // raw (untyped) buffer resource, gfx9 family
constexpr int QP_THREADS = 512;
constexpr int QP_SLICES = QP_THREADS / (2 * DG);

// -------------------------------------------------------------------------- query prep
// Two workgroups per quad (type 0: Pi q and the MSE rows; type 1: S q and the QJL rows).
// Thread i forms row i % 128 (row r of group r / 64) over a quarter of that group's 64
// columns, reading the group's row-major matrix (four 16-byte loads, issued with the query
// loads before any product).  Then per (group, head) the largest |value| (the digit scale)
// and the sum (the constants), and the operand chunks in MFMA register order.
template <int B0, int B1>
__global__ __launch_bounds__(QP_THREADS) void split_qprep_kernel(const unsigned char* __restrict__ params0,
                                                                 const unsigned char* __restrict__ params1,
                                                                 size_t off_pi, size_t off_s,
                                                                 const void* __restrict__ q, int q_f32,
                                                                 unsigned char* __restrict__ ws) {
  constexpr int D = 2 * DG;
  constexpr int NW0 = score_words(B0), NW1 = score_words(B1);
  constexpr int KS = DG / QP_SLICES;       // columns per slice (16)
  const long g = blockIdx.x >> 1;
  const int type = blockIdx.x & 1;         // 0: Pi (MSE rows), 1: S (QJL rows)
  const int tid = threadIdx.x;
  const Header* h0 = reinterpret_cast<const Header*>(params0);
  const Header* h1 = reinterpret_cast<const Header*>(params1);
  __shared__ float4 qv[D];                 // q of the G heads, column-major: qv[k] = heads 0..3
  __shared__ float part_sum[QP_SLICES][G][D];
  __shared__ float stats[2][G][2];         // [group][head]: max |v|, sum v

  {
    const int row = tid % D, slice = tid / D;
    const int gr = row / DG, rl = row % DG;
    const float4* src = reinterpret_cast<const float4*>((gr ? params1 : params0) + (type ? off_s : off_pi)) +
                        (size_t(rl) * DG + size_t(slice) * KS) / 4;
    float4 m4[KS / 4];
#pragma unroll
    for (int j = 0; j < KS / 4; ++j) m4[j] = src[j];
    for (int i = tid; i < G * D; i += QP_THREADS) {
      const long off = g * G * D + i;
      reinterpret_cast<float*>(qv)[(i % D) * G + i / D] =
          q_f32 ? static_cast<const float*>(q)[off]
                : __uint_as_float(uint32_t(static_cast<const uint16_t*>(q)[off]) << 16);
    }
    __syncthreads();                       // q is in LDS
    float acc[G] = {};
#pragma unroll
    for (int j = 0; j < KS / 4; ++j) {
      const float mv[4] = {m4[j].x, m4[j].y, m4[j].z, m4[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float4 qk = qv[gr * DG + slice * KS + 4 * j + e];
        acc[0] = fmaf(mv[e], qk.x, acc[0]);
        acc[1] = fmaf(mv[e], qk.y, acc[1]);
        acc[2] = fmaf(mv[e], qk.z, acc[2]);
        acc[3] = fmaf(mv[e], qk.w, acc[3]);
      }
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
  float (*v)[D] = part_sum[0];             // v[h][row]: Pi_g q_g (type 0) or S_g q_g (type 1)
  if (tid < 2 * G * 2 * 16) {
    // 2 groups x G heads x 2 statistics, 16 threads each
    const int gg = tid >> 7, h = (tid >> 5) & 3, stat = (tid >> 4) & 1, sub = tid & 15;
    float r = 0.f;
#pragma unroll
    for (int k = 0; k < DG / 16; ++k) {
      const float x = v[h][gg * DG + sub + 16 * k];
      r = (stat == 0) ? fmaxf(r, fabsf(x)) : r + x;
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
      const float o = __shfl_xor(r, off, 16);
      r = (stat == 0) ? fmaxf(r, o) : r + o;
    }
    if (sub == 0) stats[gg][h][stat] = r;
  }
  __syncthreads();

  unsigned char* base = ws + size_t(g) * score_split_ws_per_group(B0, B1);
  // A operand chunks of this half: group 0's items, then group 1's; per head NW MFMAs x 4
  // K chunks x 2 rows (digit hi, lo)
  constexpr int ITEMS0 = G * NW0 * 4 * 2, ITEMS = ITEMS0 + G * NW1 * 4 * 2;
  for (int item = tid; item < ITEMS; item += QP_THREADS) {
    const int gg = item < ITEMS0 ? 0 : 1;
    const int it = gg ? item - ITEMS0 : item;
    const int nwg = gg ? NW1 : NW0;
    const int h = it / (nwg * 8), r = it % (nwg * 8);
    const int m = r / 8, part = 2 * type + (r / 4) % 2, c = r % 4;
    const int lane = 16 * c + 4 * h + part;
    const int cg = c >> 1, j = c & 1;      // K chunk: coordinate group of the channel group, bit parity
    // header fields by a uniform select of the block (an indexed header would be a memory
    // load per item)
    const Header* hd = gg ? h1 : h0;
    const bool mse_word = m < hd->ne;
    const float ew = m == 0 ? hd->e[0] : m == 1 ? hd->e[1] : m == 2 ? hd->e[2] : hd->e[3];
    const float mx = type == 0 ? hd->emax * stats[gg][h][0] : stats[gg][h][0];
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
        const int coord = gg * DG + 32 * cg + 8 * bi + 2 * k + j;
        const int vj = int(rintf(f * v[h][coord]));   // value as an integer: 128 hi + lo
        const int hi = (vj + 64) >> 7;
        const int lo = vj - 128 * hi;
        dw |= uint32_t(uint8_t(int8_t(hi_part ? hi : lo))) << (8 * bi);
      }
      packed[k] = dw;
    }
    reinterpret_cast<uint4*>(base + (gg ? size_t(NW0) * 64 * 16 : 0))[m * 64 + lane] =
        make_uint4(packed[0], packed[1], packed[2], packed[3]);
  }
  // epilogue constants per (group, head): l_g = nu_g (A_g wA - cA + gamma_g (B_g wB - cB));
  // type 0 writes (x, y), type 1 writes (z, w)
  if (tid < 2 * G) {
    const int gg = tid / G, h = tid % G;
    const Header* hd = gg ? h1 : h0;
    float* cs = reinterpret_cast<float*>(base + size_t(NW0 + NW1) * 64 * 16) + 4 * (gg * G + h);
    if (type == 0) {
      const float ma = hd->emax * stats[gg][h][0];
      const float sa = ma > 0.f ? kDigitRange / ma : 1.f;
      cs[0] = 2.f / sa;
      cs[1] = hd->esum * stats[gg][h][1];
    } else {
      const float sb = stats[gg][h][0] > 0.f ? kDigitRange / stats[gg][h][0] : 1.f;
      cs[2] = 2.f * hd->alpha / sb;
      cs[3] = hd->alpha * stats[gg][h][1];
    }
  }
}

// ---------------------------------------------------------------------------- scoring
template <int B> __device__ __forceinline__ void load_words(__amdgpu_buffer_rsrc_t rs, int off, uint32_t* w) {
  if constexpr (B == 4) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else if constexpr (B == 3) {
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rs, off, 0, 0);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2];
  } else {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
    w[0] = v[0]; w[1] = v[1];
  }
}

// Tiles loaded ahead per wave iteration, and the waves per SIMD the scan keeps resident (the
// register budget: both groups' operands and the tiles' words, nu and gamma in flight; the
// tiles' MFMA chains are kept apart so that their accumulators are not live at once).
constexpr int split_unroll(int b0, int b1) { return b0 + b1 >= 8 ? 4 : 8; }
constexpr int split_waves_per_simd(int b0, int b1) { return b0 + b1 <= 4 ? 4 : 3; }

// One wave per key range, as the d = 128 scan.  Every access goes through a buffer resource
// bounded by its array: keys past the end read zeros and their logit stores fall past the
// logits resource, so no access sits under a branch.
template <int B0, int B1, bool PROD>
__global__ __launch_bounds__(256, split_waves_per_simd(B0, B1)) void split_score_kernel(
    const uint32_t* __restrict__ codes0, const float* __restrict__ nu0, const float* __restrict__ gamma0,
    const uint32_t* __restrict__ codes1, const float* __restrict__ nu1, const float* __restrict__ gamma1,
    const unsigned char* __restrict__ ws, float* __restrict__ logits, long T, long qpg,
    long tiles_per_group, long ranges_per_group, long tiles_per_range, long total_ranges) {
  constexpr int NW0 = score_words(B0), NW1 = score_words(B1);
  constexpr int NWU0 = PROD ? NW0 : NW0 - 1, NWU1 = PROD ? NW1 : NW1 - 1;
  constexpr int UNR = split_unroll(B0, B1);
  const int lane = threadIdx.x & 63;
  const long range = long(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  if (range >= total_ranges) return;
  const long g = range / ranges_per_group;    // quad of heads: key group g / qpg, quad g % qpg
  const long kg = g / qpg;
  const long t0 = (range % ranges_per_group) * tiles_per_range;
  long t1 = t0 + tiles_per_range;
  if (t1 > tiles_per_group) t1 = tiles_per_group;

  const unsigned char* base = ws + size_t(g) * score_split_ws_per_group(B0, B1);
  v4i A0[NW0], A1[NW1];
#pragma unroll
  for (int m = 0; m < NWU0; ++m) A0[m] = reinterpret_cast<const v4i*>(base)[m * 64 + lane];
#pragma unroll
  for (int m = 0; m < NWU1; ++m) A1[m] = reinterpret_cast<const v4i*>(base + size_t(NW0) * 64 * 16)[m * 64 + lane];
  const int hq = lane >> 4;                   // output rows 4 (lane / 16) .. +3: one head's sums
  const float4* cst = reinterpret_cast<const float4*>(base + size_t(NW0 + NW1) * 64 * 16);
  const float4 c0 = cst[hq], c1 = cst[G + hq];
  const int cg = lane >> 5;                   // coordinate group within each channel group
  const uint32_t mj = 0x01010101u << ((lane >> 4) & 1);   // bit parity of this K chunk

  const __amdgpu_buffer_rsrc_t crs0 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(codes0) + size_t(kg) * T * 2 * B0, 0, int(T * 2 * B0 * 4), RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t crs1 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(codes1) + size_t(kg) * T * 2 * B1, 0, int(T * 2 * B1 * 4), RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t nrs0 =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(nu0) + size_t(kg) * T, 0, int(T * 4), RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t nrs1 =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(nu1) + size_t(kg) * T, 0, int(T * 4), RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t grs0 =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(gamma0) + size_t(kg) * T, 0, int(T * 4), RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t grs1 =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(gamma1) + size_t(kg) * T, 0, int(T * 4), RSRC_WORD3);
  // the quad's G rows of logits, [head][key]; a key past the end stores past the resource
  const __amdgpu_buffer_rsrc_t ors =
      __builtin_amdgcn_make_buffer_rsrc(logits + size_t(g) * G * T, 0, int(G * T * 4), RSRC_WORD3);
  // (ranges hold a multiple of UNR tiles, so a tile past t1 is past the group's last key)
  for (long tb = t0; tb < t1; tb += UNR) {
    uint32_t w0[UNR][4], w1[UNR][4];
    float nk0[UNR], gk0[UNR], nk1[UNR], gk1[UNR];
    int key[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      key[u] = int((tb + u) * 16) + (lane & 15);
      load_words<B0>(crs0, (key[u] * 2 + cg) * B0 * 4, w0[u]);
      load_words<B1>(crs1, (key[u] * 2 + cg) * B1 * 4, w1[u]);
      nk0[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(nrs0, key[u] * 4, 0, 0));
      nk1[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(nrs1, key[u] * 4, 0, 0));
      gk0[u] = PROD ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(grs0, key[u] * 4, 0, 0)) : 0.f;
      gk1[u] = PROD ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(grs1, key[u] * 4, 0, 0)) : 0.f;
      // loads return in issue order: a tile's loads stay together, ahead of the next tile's
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      __builtin_amdgcn_sched_barrier(0);
      const v4i s0 = score_split_tile_sums<B0, PROD>(A0, w0[u], mj);
      const v4i s1 = score_split_tile_sums<B1, PROD>(A1, w1[u], mj);
      const float l = score_tile_estimate<PROD>(s0, c0, nk0[u], gk0[u]) +
                      score_tile_estimate<PROD>(s1, c1, nk1[u], gk1[u]);
      const int oo = key[u] < T ? (hq * int(T) + key[u]) * 4 : int(G * T * 4);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l), ors, oo, 0, 0);
    }
  }
}

template <int B0, int B1>
hipError_t launch_bs(const void* params0, const void* params1, const void* q, int q_dtype,
                     const uint32_t* codes0, const float* nu0, const float* gamma0, const uint32_t* codes1,
                     const float* nu1, const float* gamma1, int64_t kv_groups, int64_t Gq, int64_t T, int mode,
                     float* logits, void* ws, hipStream_t s, int phases) {
  const Layout lay(DG, B0);   // the matrices' offsets do not depend on b
  const long qpg = long(Gq / G);
  const int64_t groups = kv_groups * qpg;
  if (phases & kScorePrep) {
    hipLaunchKernelGGL((split_qprep_kernel<B0, B1>), dim3(unsigned(2 * groups)), dim3(QP_THREADS), 0, s,
                       static_cast<const unsigned char*>(params0), static_cast<const unsigned char*>(params1),
                       lay.off_pi, lay.off_s, q, q_dtype == 0 ? 1 : 0, static_cast<unsigned char*>(ws));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(phases & kScoreScan)) return hipSuccess;
  const long tiles_per_group = (T + 15) / 16;
  const long total_tiles = long(groups) * tiles_per_group;
  long tpr = (total_tiles + long(device_cu_count()) * WAVES_PER_CU - 1) / (long(device_cu_count()) * WAVES_PER_CU);
  if (tpr < 8) tpr = 8;
  constexpr int UNR = split_unroll(B0, B1);
  tpr = (tpr + UNR - 1) / UNR * UNR;
  const long rpg = (tiles_per_group + tpr - 1) / tpr;
  const long total_ranges = long(groups) * rpg;
  const unsigned blocks = unsigned((total_ranges + 3) / 4);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, s, codes0, nu0, gamma0, codes1, nu1, gamma1,
                       static_cast<const unsigned char*>(ws), logits, long(T), qpg, tiles_per_group, rpg, tpr,
                       total_ranges);
  };
  if (mode == 0) go(split_score_kernel<B0, B1, true>); else go(split_score_kernel<B0, B1, false>);
  return hipGetLastError();
}

template <int B0>
hipError_t launch_b0(int b1, const void* params0, const void* params1, const void* q, int q_dtype,
                     const uint32_t* codes0, const float* nu0, const float* gamma0, const uint32_t* codes1,
                     const float* nu1, const float* gamma1, int64_t kv_groups, int64_t Gq, int64_t T, int mode,
                     float* logits, void* ws, hipStream_t s, int phases) {
  switch (b1) {
    case 2: return launch_bs<B0, 2>(params0, params1, q, q_dtype, codes0, nu0, gamma0, codes1, nu1, gamma1,
                                     kv_groups, Gq, T, mode, logits, ws, s, phases);
    case 3: return launch_bs<B0, 3>(params0, params1, q, q_dtype, codes0, nu0, gamma0, codes1, nu1, gamma1,
                                     kv_groups, Gq, T, mode, logits, ws, s, phases);
    case 4: return launch_bs<B0, 4>(params0, params1, q, q_dtype, codes0, nu0, gamma0, codes1, nu1, gamma1,
                                     kv_groups, Gq, T, mode, logits, ws, s, phases);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool score_split_d128_shape(int d, int d0, int b0, int b1, int64_t G) {
  return d == 2 * DG && d0 == DG && G % 4 == 0 && b0 >= 2 && b0 <= 4 && b1 >= 2 && b1 <= 4;
}

bool score_split_d128_applies(int d, int d0, int b0, int b1, int64_t G, int64_t T) {
  if (!score_split_d128_shape(d, d0, b0, b1, G)) return false;
  // buffer byte offsets (keys padded to whole tiles) within 2^31: a key group's codes of up to
  // 4 words per coordinate group, a quad's 4 rows of logits
  const int64_t tp = (T + 15) / 16 * 16;
  return tp * 2 * 4 * 4 < (int64_t(1) << 31) && tp * 4 * 4 < (int64_t(1) << 31);
}

size_t score_split_d128_ws_bytes(int b0, int b1, int64_t groups, int64_t G) {
  return align256(size_t(groups) * size_t(G / 4) * score_split_ws_per_group(b0, b1));
}

hipError_t launch_score_split_d128(const void* params0, const void* params1, int b0, int b1, const void* q,
                                   int q_dtype, const uint32_t* codes0, const float* nu0, const float* gamma0,
                                   const uint32_t* codes1, const float* nu1, const float* gamma1,
                                   int64_t kv_groups, int64_t Gq, int64_t T, int mode, float* logits, void* ws,
                                   hipStream_t s, int phases) {
  switch (b0) {
    case 2: return launch_b0<2>(b1, params0, params1, q, q_dtype, codes0, nu0, gamma0, codes1, nu1, gamma1,
                                kv_groups, Gq, T, mode, logits, ws, s, phases);
    case 3: return launch_b0<3>(b1, params0, params1, q, q_dtype, codes0, nu0, gamma0, codes1, nu1, gamma1,
                                kv_groups, Gq, T, mode, logits, ws, s, phases);
    case 4: return launch_b0<4>(b1, params0, params1, q, q_dtype, codes0, nu0, gamma0, codes1, nu1, gamma1,
                                kv_groups, Gq, T, mode, logits, ws, s, phases);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
