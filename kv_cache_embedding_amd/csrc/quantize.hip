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

// MSE: the MSE quantizer alone (attention values): GEMM1 and the index planes only, b-1
// planes per coordinate group, nu but no gamma.
template <int BITS, bool F32IN, bool MSE>
__global__ __launch_bounds__(WAVES * 64, 1) void quantize_d128_kernel(
    const unsigned char* __restrict__ params, size_t frag_off, const void* __restrict__ xin,
    long n, uint32_t* __restrict__ codes, float* __restrict__ nu_out,
    float* __restrict__ gamma_out) {
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
  {
    const uint4* src = reinterpret_cast<const uint4*>(params + frag_off);
    for (int i = threadIdx.x; i < 2 * FRAG_U4; i += WAVES * 64) frag[i] = src[i];
  }
  __syncthreads();

  const Header* hdr = reinterpret_cast<const Header*>(params);
  constexpr int L = 1 << (BITS - 1);
  float tp[L / 2 > 1 ? L / 2 - 1 : 1];   // positive thresholds
  float mp[L / 2];                        // positive centroids
#pragma unroll
  for (int k = 0; k < L / 2 - 1; ++k) tp[k] = hdr->tpos[k];
#pragma unroll
  for (int k = 0; k < L / 2; ++k) mp[k] = hdr->mpos[k];

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
    ss += __shfl_xor(ss, 32);
    const float nu = sqrtf(ss);
    const float sc = nu > 0.f ? nu : 1.f;   // zero vector: u is taken as 0, grid unscaled

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
    // the input registers are free: fetch the next tile while this one is finished
    const long next = grab();
    if (next < t_end) load_tile(next);

    // ---- bucketize + residual against nu-scaled thresholds (u is never divided by nu).
    // Bits of the sign plane are the float sign bits of u, shifted in with v_alignbit and
    // inverted at the end (u is never -0: the MFMA sum starts from +0).
    float T[L / 2 > 1 ? L / 2 - 1 : 1], M[L / 2];
#pragma unroll
    for (int k = 0; k < L / 2 - 1; ++k) T[k] = tp[k] * sc;
#pragma unroll
    for (int k = 0; k < L / 2; ++k) M[k] = mp[k] * sc;

    uint32_t hb[BITS][4];     // [plane][row tile]: this lane's 16-bit half words
    bf16x8 rh[8], rl[8];      // GEMM2 B operands, K step 2 mt + half
    float g2 = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      // Index bits from |u| against the positive thresholds (a binary search over the
      // magnitude index k of the level), the level's sign from u: for u >= 0 the index is
      // L/2 + k, for u < 0 it is L/2 - 1 - k, i.e. the bits of k complemented.  So the index
      // planes are the k planes xor the sign plane, applied once per 16-coordinate word.
      uint32_t w0 = 0, w1 = 0, ws = 0;
      float rr[16];
#pragma unroll
      for (int r = 15; r >= 0; --r) {
        const float u = U[mt][r];
        const float a = fabsf(u);
        ws = __builtin_amdgcn_alignbit(ws, __float_as_uint(u), 31);   // 1 = u < 0
        float cm;
        if constexpr (BITS == 2) {
          cm = M[0];
        } else if constexpr (BITS == 3) {
          const bool k0 = a >= T[0];
          cm = k0 ? M[1] : M[0];
          w0 = (w0 << 1) | uint32_t(k0);
        } else {
          const bool k1 = a >= T[1];
          const bool k0 = a >= (k1 ? T[2] : T[0]);
          const float mlo = k0 ? M[1] : M[0];
          const float mhi = k0 ? M[3] : M[2];
          cm = k1 ? mhi : mlo;
          w0 = (w0 << 1) | uint32_t(k0);
          w1 = (w1 << 1) | uint32_t(k1);
        }
        const float c = __uint_as_float((__float_as_uint(cm) & 0x7fffffffu) | (__float_as_uint(u) & 0x80000000u));
        const float rv = u - c;
        rr[r] = rv;
        g2 = fmaf(rv, rv, g2);
      }
      const uint32_t sgn = ws & 0xffffu;          // 1 = u < 0
      const uint32_t wsign = ~ws & 0xffffu;       // sign plane: 1 = u >= 0
      if constexpr (BITS == 2) {
        hb[0][mt] = wsign;
      } else if constexpr (BITS == 3) {
        hb[0][mt] = w0 ^ sgn;
        hb[1][mt] = wsign;
      } else {
        hb[0][mt] = w0 ^ sgn;
        hb[1][mt] = w1 ^ sgn;
        hb[2][mt] = wsign;
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          // hi = RNE(v); lo = RNE(v - hi): converted two at a time
          const f32x2 v2 = {rr[8 * hf + e], rr[8 * hf + e + 1]};
          const bf16x2 h2 = __builtin_convertvector(v2, bf16x2);
          const uint32_t hb2 = __builtin_bit_cast(uint32_t, h2);
          const f32x2 hf2 = {__uint_as_float(hb2 << 16), __uint_as_float(hb2 & 0xffff0000u)};
          const bf16x2 l2 = __builtin_convertvector(v2 - hf2, bf16x2);
          rh[2 * mt + hf][e] = h2[0];
          rh[2 * mt + hf][e + 1] = h2[1];
          rl[2 * mt + hf][e] = l2[0];
          rl[2 * mt + hf][e + 1] = l2[1];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    g2 += __shfl_xor(g2, 32);
    const float gamma = sqrtf(g2) / sc;

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
        hb[BITS - 1][mp + t] = ~w & 0xffffu;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- assemble whole words: half h = 0 finishes row tiles 0,1; h = 1 tiles 2,3
    constexpr int P = MSE ? BITS - 1 : BITS;   // planes stored per coordinate group
    uint32_t out[2 * P];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const uint32_t send = kh == 0 ? hb[p][2 + k] : hb[p][k];
        const uint32_t recv = __shfl_xor(send, 32);
        out[k * P + p] = kh == 0 ? (hb[p][k] | (recv << 16)) : (recv | (hb[p][2 + k] << 16));
      }
    }
    if (valid) {
      uint32_t* dst = codes + (vec * 4 + 2 * kh) * P;
      if constexpr (P % 2 == 0) {   // 16-byte aligned: 2 P words at a multiple of 8 P words
#pragma unroll
        for (int i = 0; i < P / 2; ++i)
          reinterpret_cast<uint4*>(dst)[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
      } else {
#pragma unroll
        for (int i = 0; i < P; ++i) reinterpret_cast<uint2*>(dst)[i] = make_uint2(out[2 * i], out[2 * i + 1]);
      }
      if (kh == 0) {
        nu_out[vec] = nu;
        if constexpr (!MSE) gamma_out[vec] = gamma;
      }
    }
    tile = next;
  }
}

int cu_count() {
  static int cached = 0;
  if (!cached) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      c = 256;
    cached = c;
  }
  return cached;
}

template <int BITS, bool F32IN, bool MSE = false>
hipError_t launch(const void* params, const void* x, int64_t n, uint32_t* codes, float* nu,
                  float* gamma, hipStream_t s) {

  const long ntiles = (n + VPW - 1) / VPW;
  const long need = (ntiles + WAVES - 1) / WAVES;
  const int grid = int(need < cu_count() ? need : cu_count());
  hipLaunchKernelGGL((quantize_d128_kernel<BITS, F32IN, MSE>), dim3(grid), dim3(WAVES * 64), 0, s,
                     static_cast<const unsigned char*>(params), Layout(D, BITS).off_qfrag, x,
                     long(n), codes, nu, gamma);
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
