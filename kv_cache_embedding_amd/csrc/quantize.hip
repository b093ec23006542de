// Fused TurboQuant encoder for d = 128 on gfx950.
//
// Per vector x ([review, inner-product paragraph]; [tldr, steps 1-2]):
//   nu = |x|;  u = Pi x / nu                       rotation   (MFMA, bf16 hi/lo split)
//   idx_t = #{i : u_t >= tau_i};  chat = c[idx]     Lloyd-Max  (VALU, per coordinate)
//   r' = u - chat;  gamma = |r'|                   residual in the rotated space
//   z_i = [ (S' r')_i >= 0 ],  S' = S Pi^T          QJL signs  (MFMA, bf16 hi/lo split)
// S' r' equals S (x/nu - Pi^T chat), the sketch of the original-space residual, because
// Pi is orthogonal; this saves the Pi^T chat product.
//
// Data flow of one wave (32 vectors, one 32-column MFMA tile):
//   GEMM1  U^T[128 x 32] = Pi~ X^T with v_mfma_f32_32x32x16_bf16; Pi~ is Pi with its rows
//          permuted so that lane half h, accumulator register r of row tile mt holds
//          canonical coordinate 32 mt + 16 h + r of the lane's vector (lane % 32).
//          Passes: Pi_hi x + Pi_lo x (bf16 input is exact in bf16), plus Pi_hi x_lo for
//          float32 input (x = x_hi + x_lo).  Fragments of Pi~ are read from LDS.
//   bucketize in registers against thresholds scaled by nu (no division by nu); the
//          index bits are shifted into 16-bit half words, the residual is split into
//          bf16 hi/lo pairs that are directly the B operand of GEMM2.
//   GEMM2  Y^T = S'~ R'^T, passes S'_hi r_hi + S'_lo r_hi + S'_hi r_lo; the sign of each
//          output is shifted into half words the same way.
//   Lanes h = 0 / 1 of a vector swap half words and store whole words (canonical layout).
//
// Split mode (fractional bit rates: channels 0..63 and 64..127 as two TurboQuant instances
// of d = 64 at B0 and B1 bits): the two rotations and QJL matrices act on the 128-vector as
// block-diagonal matrices, so the same two GEMMs run on fragments assembled in LDS from the
// two 64-d parameter blocks (zeros off the diagonal blocks).  Lane half h already holds the
// channels of group h, so its half of the squared norm is that group's nu^2; row tiles 0, 1
// (coordinates of group 0) are bucketized with group 0's codebook and nu, tiles 2, 3 with
// group 1's; the residual of each group is projected by its own block of S', whose signs
// do not depend on the group's scale.  Lane half h stores group h's words, nu and gamma.
#include "tq_internal.h"

namespace tq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;
constexpr int WAVES = 8;                    // waves per workgroup (2 per SIMD)
constexpr int VPW = 32;                     // vectors per wave tile
constexpr int FRAG_U4 = 64 * 1024 / 16;     // uint4 per fragment set (Pi~ or S'~)

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32-row tile held by MFMA output lane rho % 32 (the fragment row permutation).
__device__ __forceinline__ int row_coord(int rho) { return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3); }

// Lane masks of one comparison, and the two VALU ops that consume one: the comparison's
// 64-bit lane mask stays in an SGPR pair, from which v_addc shifts the bit into a plane word
// (w = 2 w + bit) and v_cndmask selects between two values.  Written as separate asm
// statements so that the compiler schedules the comparisons of several coordinates ahead
// of their uses.  The compiler keeps the wait states between such asm statements, but not
// those between an MFMA and an asm statement that reads its result: code that compares
// MFMA results reads them first with ordinary instructions behind a scheduling barrier.
typedef unsigned long long lanemask;

__device__ __forceinline__ lanemask ge_abs(float u, float t) {   // |u| >= t
  lanemask m;
  asm("v_cmp_ge_f32_e64 %0, |%1|, %2" : "=s"(m) : "v"(u), "v"(t));
  return m;
}
__device__ __forceinline__ uint32_t shift_in(uint32_t w, lanemask m) {   // 2 w + bit
  uint32_t r;
  lanemask carry;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry) : "v"(w), "s"(m));
  return r;
}
__device__ __forceinline__ float select(float if0, float if1, lanemask m) {
  float r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(if0), "v"(if1), "s"(m));
  return r;
}

// Bucketize one 32-row tile of u (this lane's 16 coordinates of it) against nu-scaled
// positive thresholds T and centroids M: the index planes' half words into hb[0 .. BITS-2]
// (the top index bit is the sign of u; hb[BITS-1] is left for the QJL signs), the residual as
// bf16 hi/lo B operands of GEMM2 (K steps 2 mt, 2 mt + 1) and its squared norm into g2.
template <int BITS>
__device__ __forceinline__ void bucketize_tile(const f32x16& Um, const float* T, const float* M,
                                               uint32_t* hb, bf16x8* rh, bf16x8* rl, float& g2) {
  // Index bits from |u| against the positive thresholds (a binary search over the
  // magnitude index k of the level; a tie goes to the outer cell), the level's side from
  // the sign of u: for u >= 0 the index is L/2 + k, for u < 0 it is L/2 - 1 - k, i.e. the
  // bits of k complemented.  So the index planes are the k planes xor the sign plane,
  // applied once per 16-coordinate word.
  uint32_t w0 = 0, w1 = 0, ws = 0;
  float rr[16];
#pragma unroll
  for (int r = 15; r >= 0; --r) ws = __builtin_amdgcn_alignbit(ws, __float_as_uint(Um[r]), 31);   // 1 = u < 0
  // Um holds MFMA results: the reads above carry the compiler's wait states after the MFMA,
  // and the barrier keeps the asm comparisons below after them
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 15; r >= 0; --r) {
    const float u = Um[r];
    float cm;
    if constexpr (BITS == 2) {
      cm = M[0];
    } else if constexpr (BITS == 3) {
      const lanemask k0 = ge_abs(u, T[0]);
      w0 = shift_in(w0, k0);
      cm = select(M[0], M[1], k0);
    } else {
      // k = c0 + c1 + c2 with c_i = [|u| >= T_i] (monotone in i): bit 1 of k is c1, bit 0
      // is c0 ^ c1 ^ c2, formed on the scalar unit from the lane masks
      const lanemask c0 = ge_abs(u, T[0]), c1 = ge_abs(u, T[1]), c2 = ge_abs(u, T[2]);
      w1 = shift_in(w1, c1);
      w0 = shift_in(w0, c0 ^ c1 ^ c2);
      cm = select(select(select(M[0], M[1], c0), M[2], c1), M[3], c2);
    }
    const float c = __uint_as_float((__float_as_uint(cm) & 0x7fffffffu) | (__float_as_uint(u) & 0x80000000u));
    const float rv = u - c;
    rr[r] = rv;
    g2 = fmaf(rv, rv, g2);
  }
  const uint32_t sgn = ws & 0xffffu;          // 1 = u < 0
  const uint32_t wsign = ~ws & 0xffffu;       // sign plane: 1 = u >= 0
  if constexpr (BITS == 2) {
    hb[0] = wsign;
  } else if constexpr (BITS == 3) {
    hb[0] = w0 ^ sgn;
    hb[1] = wsign;
  } else {
    hb[0] = w0 ^ sgn;
    hb[1] = w1 ^ sgn;
    hb[2] = wsign;
  }
  // hi = RNE(v); lo = RNE(v - hi), two coordinates at a time.  v - hi is exact in float32
  // and comes from one dot2 each: hi pair . (-1, 0) + v.  The two selector pairs are held in
  // SGPRs (opaque to the compiler), so that no inline constant stands for a bf16 pair.
  uint32_t sel_lo = 0x0000bf80u, sel_hi = 0xbf800000u;   // bf16 pairs (-1, 0) and (0, -1)
  asm("" : "+s"(sel_lo), "+s"(sel_hi));
  const bf16x2 neg_lo = __builtin_bit_cast(bf16x2, sel_lo);
  const bf16x2 neg_hi = __builtin_bit_cast(bf16x2, sel_hi);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float v0 = rr[8 * hf + e], v1 = rr[8 * hf + e + 1];
      const f32x2 v2 = {v0, v1};
      const bf16x2 h2 = __builtin_convertvector(v2, bf16x2);
      const f32x2 l2f = {__builtin_amdgcn_fdot2_f32_bf16(h2, neg_lo, v0, false),
                         __builtin_amdgcn_fdot2_f32_bf16(h2, neg_hi, v1, false)};
      hw[e / 2] = __builtin_bit_cast(uint32_t, h2);
      lw[e / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(l2f, bf16x2));
    }
    rh[hf] = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
    rl[hf] = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
  }
}

// 2 P words of one lane (word k P + p taken from out[k PM + p]) to dst: 16-byte stores when P
// is even (dst is then 16-byte aligned), 8-byte ones otherwise.
template <int P, int PM>
__device__ __forceinline__ void store_words(uint32_t* dst, const uint32_t* out) {
  uint32_t o[2 * P];
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int p = 0; p < P; ++p) o[k * P + p] = out[k * PM + p];
  if constexpr (P % 2 == 0) {
#pragma unroll
    for (int i = 0; i < P / 2; ++i)
      reinterpret_cast<uint4*>(dst)[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  } else {
#pragma unroll
    for (int i = 0; i < P; ++i) reinterpret_cast<uint2*>(dst)[i] = make_uint2(o[2 * i], o[2 * i + 1]);
  }
}

// MSE: the MSE quantizer alone (attention values): GEMM1 and the index planes only, b-1
// planes per coordinate group, nu but no gamma (also in split mode).  Without SPLIT, B0 == B1 is the b of params
// and params1, codes1, nu1_out, gamma1_out are unused; with SPLIT, params / params1 are the
// d = 64 blocks of channel groups 0 / 1 (gmat_off: their bf16 matrices) and group 1's
// results go to codes1, nu1_out, gamma1_out.
// UOUT (diagnostic, no split): u = Pi x / nu of every vector is also written to u_out
// [n][128] float32, from the accumulators that the bucketize reads.
template <int B0, int B1, bool F32IN, bool MSE, bool SPLIT, bool UOUT = false>
__global__ __launch_bounds__(WAVES * 64, 1) void quantize_d128_kernel(
    const unsigned char* __restrict__ params, const unsigned char* __restrict__ params1,
    size_t frag_off, size_t gmat_off, const void* __restrict__ xin, long n,
    uint32_t* __restrict__ codes, float* __restrict__ nu_out, float* __restrict__ gamma_out,
    uint32_t* __restrict__ codes1, float* __restrict__ nu1_out, float* __restrict__ gamma1_out,
    float* __restrict__ u_out) {
  static_assert(SPLIT || B0 == B1, "one bit width without split");
  static_assert(!(UOUT && SPLIT), "rotation output without split only");
  __shared__ uint4 frag[2 * FRAG_U4];  // [0, FRAG_U4): Pi~ fragments; then S'~ fragments
  __shared__ int next_tile;            // work queue of this workgroup's tile range

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kh = lane >> 5;               // lane half: K group of the operands
  const long ntiles = (n + VPW - 1) / VPW;
  // Each workgroup owns a contiguous range of tiles; its waves take tiles from it through
  // an LDS counter.  The two waves that share a SIMD do not progress at the same rate (the
  // older one wins issue arbitration), so a static split would leave the SIMD running one
  // wave for the last part of the kernel.
  const long per_wg = (ntiles + gridDim.x - 1) / gridDim.x;
  const long t_begin = long(blockIdx.x) * per_wg;
  const long t_end = t_begin + per_wg < ntiles ? t_begin + per_wg : ntiles;
  long tile = t_begin + wave;            // the first tile of each wave is fixed
  if (threadIdx.x == 0) next_tile = 0;
  auto grab = [&]() -> long {            // next tile of this wave (t_end when none is left)
    int k = 0;
    if (lane == 0) k = atomicAdd(&next_tile, 1);
    const long t = t_begin + WAVES + __builtin_amdgcn_readfirstlane(k);
    return t < t_end ? t : t_end;
  };

  // Raw input of this lane's half vector (coordinates 64 kh .. 64 kh + 63), loaded one
  // tile ahead of its use.
  constexpr int NRAW = F32IN ? 16 : 8;
  uint4 raw[NRAW];
  auto load_tile = [&](long tl) {
    const long vec = tl * VPW + (lane & 31);
    const long vrow = vec < n ? vec : n - 1;   // ragged tail: read a valid row, store nothing
    const uint4* p = F32IN ? reinterpret_cast<const uint4*>(static_cast<const float*>(xin) + vrow * D + 64 * kh)
                           : reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xin) + vrow * D + 64 * kh);
#pragma unroll
    for (int i = 0; i < NRAW; ++i) raw[i] = p[i];
  };
  if (tile < t_end) load_tile(tile);      // in flight while the fragments fill LDS
  // the fragments: every load first, then the LDS stores, so that the fill costs one round
  // trip to memory rather than one per pass of a load-wait-store loop
  constexpr int FILL = 2 * FRAG_U4 / (WAVES * 64);
  static_assert(FILL * WAVES * 64 == 2 * FRAG_U4, "the threads fill the fragments evenly");
  if constexpr (!SPLIT) {
    const uint4* src = reinterpret_cast<const uint4*>(params + frag_off);
    uint4 fv[FILL];
#pragma unroll
    for (int j = 0; j < FILL; ++j) fv[j] = src[threadIdx.x + j * WAVES * 64];
#pragma unroll
    for (int j = 0; j < FILL; ++j) frag[threadIdx.x + j * WAVES * 64] = fv[j];
  } else {
    // fragment element e of lane ln: Pi~ [s][mt][pass] holds Pi[32 mt + row_coord(ln % 32)]
    // [64 (ln / 32) + 8 s + e]; S'~ [mt][s][pass] holds S'[32 mt + row_coord(ln % 32)]
    // [32 (s / 2) + 16 (ln / 32) + 8 (s % 2) + e]; block g of the block-diagonal matrices is
    // group g's 64 x 64 matrix (row-major bf16 hi and lo: Pi at 0 and 4096 elements, S' at
    // 8192 and 12288), every other block zero
    const uint16_t* gm[2] = {reinterpret_cast<const uint16_t*>(params + gmat_off),
                             reinterpret_cast<const uint16_t*>(params1 + gmat_off)};
    uint4 fv[FILL];
#pragma unroll
    for (int f = 0; f < FILL; ++f) {
      const int i = threadIdx.x + f * WAVES * 64;
      const bool is_s = i >= FRAG_U4;
      const int k = is_s ? i - FRAG_U4 : i;
      const int ln = k & 63, j = k >> 6, pass = j & 1, m = j >> 1;
      const int mt = is_s ? m >> 3 : m & 3;
      const int st = is_s ? m & 7 : m >> 2;
      const int rg = mt >> 1;                               // group of the output row
      const int cg = is_s ? st >> 2 : ln >> 5;              // group of the input column
      const int col = is_s ? 32 * (st >> 1) + 16 * (ln >> 5) + 8 * (st & 1) - 64 * cg : 8 * st;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (rg == cg) {
        const int row = 32 * mt + row_coord(ln & 31) - 64 * rg;
        v = *reinterpret_cast<const uint4*>(gm[rg] + (is_s ? 8192 : 0) + pass * 4096 + row * 64 + col);
      }
      fv[f] = v;
    }
#pragma unroll
    for (int f = 0; f < FILL; ++f) frag[threadIdx.x + f * WAVES * 64] = fv[f];
  }
  __syncthreads();

  const Header* hdr = reinterpret_cast<const Header*>(params);
  const Header* hdr1 = reinterpret_cast<const Header*>(SPLIT ? params1 : params);
  constexpr int L0 = 1 << (B0 - 1), L1 = 1 << (B1 - 1);
  float tp0[L0 / 2 > 1 ? L0 / 2 - 1 : 1], tp1[L1 / 2 > 1 ? L1 / 2 - 1 : 1];   // positive thresholds
  float mp0[L0 / 2], mp1[L1 / 2];                                             // positive centroids
#pragma unroll
  for (int k = 0; k < L0 / 2 - 1; ++k) tp0[k] = hdr->tpos[k];
#pragma unroll
  for (int k = 0; k < L0 / 2; ++k) mp0[k] = hdr->mpos[k];
#pragma unroll
  for (int k = 0; k < L1 / 2 - 1; ++k) tp1[k] = hdr1->tpos[k];
#pragma unroll
  for (int k = 0; k < L1 / 2; ++k) mp1[k] = hdr1->mpos[k];

  while (tile < t_end) {
    const long vec = tile * VPW + (lane & 31);
    const bool valid = vec < n;

    // ---- operands of GEMM1 and the squared norm
    bf16x8 xh[8];
    bf16x8 xl[F32IN ? 8 : 1];
    float ss = 0.f;
    if constexpr (!F32IN) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        xh[s] = as_bf16x8(raw[s]);
        const uint32_t ws4[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const bf16x2 p2 = __builtin_bit_cast(bf16x2, ws4[k]);
          ss = __builtin_amdgcn_fdot2_f32_bf16(p2, p2, ss, false);
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float4 a = __builtin_bit_cast(float4, raw[2 * s]);
        const float4 b = __builtin_bit_cast(float4, raw[2 * s + 1]);
        const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ss = fmaf(f[e], f[e], ss);
          const __bf16 hi = (__bf16)f[e];
          xh[s][e] = hi;
          xl[s][e] = (__bf16)(f[e] - (float)hi);
        }
      }
    }
    // squared norms of group 0 (channels 0..63, lane half 0) and group 1 (half 1); without
    // SPLIT both are the whole vector's
    const float ss_other = __shfl_xor(ss, 32);
    const float ssa = SPLIT ? (kh == 0 ? ss : ss_other) : ss + ss_other;
    const float ssb = SPLIT ? (kh == 0 ? ss_other : ss) : ssa;
    const float nu0 = sqrtf(ssa), nu1 = sqrtf(ssb);
    const float sc0 = nu0 > 0.f ? nu0 : 1.f;   // zero vector: u is taken as 0, grid unscaled
    const float sc1 = nu1 > 0.f ? nu1 : 1.f;

    // ---- GEMM1: U^T = Pi~ X^T, one 32-row tile at a time
    f32x16 U[4];
#pragma unroll
    for (int mp = 0; mp < 4; mp += 2) {
      // two independent accumulation chains (row tiles mp, mp + 1) interleaved
      U[mp] = f32x16{};
      U[mp + 1] = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int mt = mp + t;
          const bf16x8 ahi = as_bf16x8(frag[((s * 4 + mt) * 2 + 0) * 64 + lane]);
          U[mt] = mfma(ahi, xh[s], U[mt]);
          if constexpr (F32IN) U[mt] = mfma(ahi, xl[s], U[mt]);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int mt = mp + t;
          const bf16x8 alo = as_bf16x8(frag[((s * 4 + mt) * 2 + 1) * 64 + lane]);
          U[mt] = mfma(alo, xh[s], U[mt]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // bound the fragment reads in flight
    }
    if constexpr (UOUT) {
      // lane half h, register r of row tile mt holds coordinate 32 mt + 16 h + r
      if (valid) {
        const float inv = nu0 > 0.f ? 1.f / nu0 : 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            *reinterpret_cast<float4*>(u_out + vec * D + 32 * mt + 16 * kh + 4 * r4) =
                make_float4(U[mt][4 * r4] * inv, U[mt][4 * r4 + 1] * inv, U[mt][4 * r4 + 2] * inv,
                            U[mt][4 * r4 + 3] * inv);
      }
    }
    // the input registers are free: fetch the next tile while this one is finished
    const long next = grab();
    if (next < t_end) load_tile(next);

    // ---- bucketize + residual against nu-scaled thresholds (u is never divided by nu).
    // Bits of the sign plane are the float sign bits of u, shifted in with v_alignbit and
    // inverted at the end (u is never -0: the MFMA sum starts from +0).
    float T0[L0 / 2 > 1 ? L0 / 2 - 1 : 1], M0[L0 / 2], T1[L1 / 2 > 1 ? L1 / 2 - 1 : 1], M1[L1 / 2];
#pragma unroll
    for (int k = 0; k < L0 / 2 - 1; ++k) T0[k] = tp0[k] * sc0;
#pragma unroll
    for (int k = 0; k < L0 / 2; ++k) M0[k] = mp0[k] * sc0;
#pragma unroll
    for (int k = 0; k < L1 / 2 - 1; ++k) T1[k] = tp1[k] * sc1;
#pragma unroll
    for (int k = 0; k < L1 / 2; ++k) M1[k] = mp1[k] * sc1;

    uint32_t hb[4][4];        // [row tile][plane]: this lane's 16-bit half words
    bf16x8 rh[8], rl[8];      // GEMM2 B operands, K step 2 mt + half
    float g2a = 0.f, g2b = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      bucketize_tile<B0>(U[mt], T0, M0, hb[mt], rh + 2 * mt, rl + 2 * mt, g2a);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int mt = 2; mt < 4; ++mt) {
      bucketize_tile<B1>(U[mt], T1, M1, hb[mt], rh + 2 * mt, rl + 2 * mt, SPLIT ? g2b : g2a);
      __builtin_amdgcn_sched_barrier(0);
    }
    g2a += __shfl_xor(g2a, 32);
    if constexpr (SPLIT) g2b += __shfl_xor(g2b, 32);
    const float gamma0 = sqrtf(g2a) / sc0;
    const float gamma1 = SPLIT ? sqrtf(g2b) / sc1 : gamma0;

    // ---- GEMM2: Y^T = S'~ R'^T, one 32-row tile of projections at a time; the sign
    //      bits of y are shifted in the same way (y is never -0 either)
#pragma unroll
    for (int mp = 0; mp < (MSE ? 0 : 4); mp += 2) {
      f32x16 Y[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        bf16x8 ahi[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          ahi[t] = as_bf16x8(frag[FRAG_U4 + (((mp + t) * 8 + s) * 2 + 0) * 64 + lane]);
          Y[t] = mfma(ahi[t], rh[s], Y[t]);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 alo = as_bf16x8(frag[FRAG_U4 + (((mp + t) * 8 + s) * 2 + 1) * 64 + lane]);
          Y[t] = mfma(alo, rh[s], Y[t]);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) Y[t] = mfma(ahi[t], rl[s], Y[t]);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint32_t w = 0;
#pragma unroll
        for (int r = 15; r >= 0; --r) w = __builtin_amdgcn_alignbit(w, __float_as_uint(Y[t][r]), 31);
        hb[mp + t][(mp + t < 2 ? B0 : B1) - 1] = ~w & 0xffffu;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- assemble whole words: half h = 0 finishes row tiles 0,1; h = 1 tiles 2,3
    constexpr int P0 = MSE ? B0 - 1 : B0, P1 = MSE ? B1 - 1 : B1;   // planes per coordinate group
    constexpr int PM = P0 > P1 ? P0 : P1;
    uint32_t out[2 * PM];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
#pragma unroll
      for (int p = 0; p < PM; ++p) {
        // planes a group does not have are sent but not stored
        const uint32_t send = kh == 0 ? (p < P1 ? hb[2 + k][p] : 0u) : (p < P0 ? hb[k][p] : 0u);
        const uint32_t recv = __shfl_xor(send, 32);
        out[k * PM + p] = kh == 0 ? ((p < P0 ? hb[k][p] : 0u) | (recv << 16))
                                  : (recv | ((p < P1 ? hb[2 + k][p] : 0u) << 16));
      }
    }
    if (valid) {
      if constexpr (!SPLIT) {
        // 2 P words at a multiple of 8 P words (16-byte aligned when P is even)
        store_words<P0, PM>(codes + (vec * 4 + 2 * kh) * P0, out);
        if (kh == 0) {
          nu_out[vec] = nu0;
          if constexpr (!MSE) gamma_out[vec] = gamma0;
        }
      } else if (kh == 0) {
        store_words<P0, PM>(codes + vec * 2 * P0, out);
        nu_out[vec] = nu0;
        if constexpr (!MSE) gamma_out[vec] = gamma0;
      } else {
        store_words<P1, PM>(codes1 + vec * 2 * P1, out);
        nu1_out[vec] = nu1;
        if constexpr (!MSE) gamma1_out[vec] = gamma1;
      }
    }
    tile = next;
  }
}

int grid_for(int64_t n) {
  const long ntiles = (n + VPW - 1) / VPW;
  const long need = (ntiles + WAVES - 1) / WAVES;
  return int(need < device_cu_count() ? need : device_cu_count());
}

template <int BITS, bool F32IN, bool MSE = false>
hipError_t launch(const void* params, const void* x, int64_t n, uint32_t* codes, float* nu,
                  float* gamma, hipStream_t s) {
  hipLaunchKernelGGL((quantize_d128_kernel<BITS, BITS, F32IN, MSE, false>), dim3(grid_for(n)),
                     dim3(WAVES * 64), 0, s, static_cast<const unsigned char*>(params), nullptr,
                     Layout(D, BITS).off_qfrag, size_t(0), x, long(n), codes, nu, gamma, nullptr,
                     nullptr, nullptr, nullptr);
  return hipGetLastError();
}

template <int BITS, bool F32IN>
hipError_t launch_u(const void* params, const void* x, int64_t n, uint32_t* codes, float* nu,
                    float* gamma, float* u, hipStream_t s) {
  hipLaunchKernelGGL((quantize_d128_kernel<BITS, BITS, F32IN, false, false, true>), dim3(grid_for(n)),
                     dim3(WAVES * 64), 0, s, static_cast<const unsigned char*>(params), nullptr,
                     Layout(D, BITS).off_qfrag, size_t(0), x, long(n), codes, nu, gamma, nullptr,
                     nullptr, nullptr, u);
  return hipGetLastError();
}

template <int B0, int B1, bool F32IN, bool MSE = false>
hipError_t launch_split(const void* params0, const void* params1, const void* x, int64_t n,
                        uint32_t* codes0, float* nu0, float* gamma0, uint32_t* codes1, float* nu1,
                        float* gamma1, hipStream_t s) {
  hipLaunchKernelGGL((quantize_d128_kernel<B0, B1, F32IN, MSE, true>), dim3(grid_for(n)),
                     dim3(WAVES * 64), 0, s, static_cast<const unsigned char*>(params0),
                     static_cast<const unsigned char*>(params1), size_t(0), Layout(64, B0).off_gmat, x,
                     long(n), codes0, nu0, gamma0, codes1, nu1, gamma1, nullptr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_d128(const void* params, int b, const void* x, int x_dtype, int64_t n,
                                uint32_t* codes, float* nu, float* gamma, hipStream_t s) {
  const bool f32 = x_dtype == 0;
  switch (b) {
    case 2: return f32 ? launch<2, true>(params, x, n, codes, nu, gamma, s)
                       : launch<2, false>(params, x, n, codes, nu, gamma, s);
    case 3: return f32 ? launch<3, true>(params, x, n, codes, nu, gamma, s)
                       : launch<3, false>(params, x, n, codes, nu, gamma, s);
    case 4: return f32 ? launch<4, true>(params, x, n, codes, nu, gamma, s)
                       : launch<4, false>(params, x, n, codes, nu, gamma, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quantize_d128_u(const void* params, int b, const void* x, int x_dtype, int64_t n,
                                  uint32_t* codes, float* nu, float* gamma, float* u, hipStream_t s) {
  const bool f32 = x_dtype == 0;
  switch (b) {
    case 2: return f32 ? launch_u<2, true>(params, x, n, codes, nu, gamma, u, s)
                       : launch_u<2, false>(params, x, n, codes, nu, gamma, u, s);
    case 3: return f32 ? launch_u<3, true>(params, x, n, codes, nu, gamma, u, s)
                       : launch_u<3, false>(params, x, n, codes, nu, gamma, u, s);
    case 4: return f32 ? launch_u<4, true>(params, x, n, codes, nu, gamma, u, s)
                       : launch_u<4, false>(params, x, n, codes, nu, gamma, u, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq

namespace tq {

hipError_t launch_quantize_d128_mse(const void* params, int b, const void* x, int x_dtype,
                                    int64_t n, uint32_t* codes, float* nu, hipStream_t s) {
  const bool f32 = x_dtype == 0;
  switch (b) {
    case 2: return f32 ? launch<2, true, true>(params, x, n, codes, nu, nullptr, s)
                       : launch<2, false, true>(params, x, n, codes, nu, nullptr, s);
    case 3: return f32 ? launch<3, true, true>(params, x, n, codes, nu, nullptr, s)
                       : launch<3, false, true>(params, x, n, codes, nu, nullptr, s);
    case 4: return f32 ? launch<4, true, true>(params, x, n, codes, nu, nullptr, s)
                       : launch<4, false, true>(params, x, n, codes, nu, nullptr, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq

namespace tq {

hipError_t launch_quantize_d128_split(const void* params0, const void* params1, int b0, int b1,
                                      const void* x, int x_dtype, int64_t n, uint32_t* codes0,
                                      float* nu0, float* gamma0, uint32_t* codes1, float* nu1,
                                      float* gamma1, hipStream_t s, bool mse) {
  const bool f32 = x_dtype == 0;
#define TQ_SPLIT_CASE(B0, B1)                                                                         \
  if (b0 == B0 && b1 == B1) {                                                                         \
    if (mse)                                                                                          \
      return f32 ? launch_split<B0, B1, true, true>(params0, params1, x, n, codes0, nu0, nullptr, codes1, \
                                                    nu1, nullptr, s)                                  \
                 : launch_split<B0, B1, false, true>(params0, params1, x, n, codes0, nu0, nullptr,      \
                                                     codes1, nu1, nullptr, s);                        \
    return f32 ? launch_split<B0, B1, true>(params0, params1, x, n, codes0, nu0, gamma0, codes1, nu1,   \
                                            gamma1, s)                                                \
               : launch_split<B0, B1, false>(params0, params1, x, n, codes0, nu0, gamma0, codes1,       \
                                             nu1, gamma1, s);                                         \
  }
  TQ_SPLIT_CASE(2, 2) TQ_SPLIT_CASE(2, 3) TQ_SPLIT_CASE(2, 4)
  TQ_SPLIT_CASE(3, 2) TQ_SPLIT_CASE(3, 3) TQ_SPLIT_CASE(3, 4)
  TQ_SPLIT_CASE(4, 2) TQ_SPLIT_CASE(4, 3) TQ_SPLIT_CASE(4, 4)
#undef TQ_SPLIT_CASE
  return hipErrorInvalidValue;
}

}  // namespace tq
