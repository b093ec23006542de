// TurboQuant encoder for any d that is a multiple of 128 (e.g. 1536-dimensional embeddings),
// as two tiled MFMA GEMMs per chunk of vectors ([review, inner-product paragraph];
// [tldr, steps 1-2]):
//   phase 1:  U = X Pi^T (rows = vectors, columns = rotated coordinates); its epilogue
//             divides by nu, bucketizes, packs the index planes and writes the residual
//             r' = u - chat as bf16 hi/lo rows to a scratch buffer;
//   phase 2:  Y = R' S'^T with S' = S Pi^T; its epilogue packs the QJL sign plane.
// Both use v_mfma_f32_32x32x16_bf16 with hi/lo operand splits (Pi_hi x + Pi_lo x, plus
// Pi_hi x_lo for float32 inputs; S'_hi r_hi + S'_lo r_hi + S'_hi r_lo), float32
// accumulation.  In the 32x32 accumulator layout (row = 8(r/4) + 4(lane/32) + r%4,
// column = lane % 32) a wave ballot over one accumulator register is exactly two packed
// words of the canonical layout (32 consecutive coordinates of two vectors).
// nu (phase 1) and gamma (phase 2) are row sums of squares taken while the operand rows
// stream through the workgroup.
#include "tq_internal.h"

namespace tq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int TM = 128;          // vectors per tile
constexpr int TN = 128;          // output coordinates per tile
constexpr int BK = 32;
constexpr int LDK = BK + 8;      // padded LDS row (bf16 elements)
constexpr long CHUNK = 16384;    // vectors per pass (scratch: CHUNK x d x 4 bytes)

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;
  return uint32_t(__builtin_bit_cast(uint16_t, ha)) | (uint32_t(__builtin_bit_cast(uint16_t, hb)) << 16);
}

// PHASE 1: A = x (float32 or bf16), B = Pi (hi/lo). PHASE 2: A = r' (hi/lo), B = S' (hi/lo).
template <int PHASE, int BITS, bool F32IN>
__global__ __launch_bounds__(256) void qgemm_kernel(const unsigned char* __restrict__ params,
                                                     const void* __restrict__ a_src, long rows,
                                                     const uint16_t* __restrict__ bhi,
                                                     const uint16_t* __restrict__ blo, int d,
                                                     long v0, uint32_t* __restrict__ codes,
                                                     float* __restrict__ nu_out,
                                                     float* __restrict__ gamma_out,
                                                     uint16_t* __restrict__ rhi,
                                                     uint16_t* __restrict__ rlo) {
  constexpr bool ALO = (PHASE == 2) || F32IN;   // A has a low part
  __shared__ __bf16 Ah[TM * LDK];
  __shared__ __bf16 Al[ALO ? TM * LDK : 1];
  __shared__ __bf16 Bh[TN * LDK];
  __shared__ __bf16 Bl[TN * LDK];
  __shared__ float rowscale[TM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const long r0 = long(blockIdx.x) * TM;       // first row (vector) of the tile in the chunk
  const int c0 = blockIdx.y * TN;              // first output coordinate of the tile
  const int srow = tid >> 1, scol = (tid & 1) * 16;
  const bool row_ok = r0 + srow < rows;
  float rs = 0.f;                              // sum of squares of this thread's row slice

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  for (int kk = 0; kk < d; kk += BK) {
    uint4 ah[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}}, al[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
    if (row_ok) {
      const size_t off = size_t(r0 + srow) * d + kk + scol;
      if constexpr (PHASE == 1 && F32IN) {
        const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(a_src) + off);
        float f[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = src[q];
          f[4 * q] = v.x; f[4 * q + 1] = v.y; f[4 * q + 2] = v.z; f[4 * q + 3] = v.w;
        }
        uint32_t hw[8], lw[8];
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          rs = fmaf(f[e], f[e], rs);
          rs = fmaf(f[e + 1], f[e + 1], rs);
          hw[e / 2] = pack_bf16x2(f[e], f[e + 1]);
          const float h0 = __uint_as_float(hw[e / 2] << 16), h1 = __uint_as_float(hw[e / 2] & 0xffff0000u);
          lw[e / 2] = pack_bf16x2(f[e] - h0, f[e + 1] - h1);
        }
        ah[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        ah[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
        al[0] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        al[1] = make_uint4(lw[4], lw[5], lw[6], lw[7]);
      } else if constexpr (PHASE == 1) {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a_src) + off);
        ah[0] = src[0];
        ah[1] = src[1];
        const uint32_t w8[8] = {ah[0].x, ah[0].y, ah[0].z, ah[0].w, ah[1].x, ah[1].y, ah[1].z, ah[1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float lo = __uint_as_float(w8[e] << 16), hi = __uint_as_float(w8[e] & 0xffff0000u);
          rs = fmaf(lo, lo, fmaf(hi, hi, rs));
        }
      } else {
        const uint4* sh = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a_src) + off);
        const uint4* sl = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a_src) + size_t(CHUNK) * d + off);
        ah[0] = sh[0]; ah[1] = sh[1]; al[0] = sl[0]; al[1] = sl[1];
        const uint32_t h8[8] = {ah[0].x, ah[0].y, ah[0].z, ah[0].w, ah[1].x, ah[1].y, ah[1].z, ah[1].w};
        const uint32_t l8[8] = {al[0].x, al[0].y, al[0].z, al[0].w, al[1].x, al[1].y, al[1].z, al[1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v0e = __uint_as_float(h8[e] << 16) + __uint_as_float(l8[e] << 16);
          const float v1e = __uint_as_float(h8[e] & 0xffff0000u) + __uint_as_float(l8[e] & 0xffff0000u);
          rs = fmaf(v0e, v0e, fmaf(v1e, v1e, rs));
        }
      }
    }
    const size_t boff = size_t(c0 + srow) * d + kk + scol;
    const uint4* bsh = reinterpret_cast<const uint4*>(bhi + boff);
    const uint4* bsl = reinterpret_cast<const uint4*>(blo + boff);
    const uint4 bh0 = bsh[0], bh1 = bsh[1], bl0 = bsl[0], bl1 = bsl[1];
    __syncthreads();   // previous step's fragments are consumed
    *reinterpret_cast<uint4*>(&Ah[srow * LDK + scol]) = ah[0];
    *reinterpret_cast<uint4*>(&Ah[srow * LDK + scol + 8]) = ah[1];
    if constexpr (ALO) {
      *reinterpret_cast<uint4*>(&Al[srow * LDK + scol]) = al[0];
      *reinterpret_cast<uint4*>(&Al[srow * LDK + scol + 8]) = al[1];
    }
    *reinterpret_cast<uint4*>(&Bh[srow * LDK + scol]) = bh0;
    *reinterpret_cast<uint4*>(&Bh[srow * LDK + scol + 8]) = bh1;
    *reinterpret_cast<uint4*>(&Bl[srow * LDK + scol]) = bl0;
    *reinterpret_cast<uint4*>(&Bl[srow * LDK + scol + 8]) = bl1;
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      bf16x8 a_h[2], a_l[2], b_h[2], b_l[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ra = (wm + 32 * i + (lane & 31)) * LDK + ks + 8 * (lane >> 5);
        const int rb = (wn + 32 * i + (lane & 31)) * LDK + ks + 8 * (lane >> 5);
        a_h[i] = *reinterpret_cast<const bf16x8*>(&Ah[ra]);
        if constexpr (ALO) a_l[i] = *reinterpret_cast<const bf16x8*>(&Al[ra]);
        b_h[i] = *reinterpret_cast<const bf16x8*>(&Bh[rb]);
        b_l[i] = *reinterpret_cast<const bf16x8*>(&Bl[rb]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = mfma(a_h[i], b_h[j], acc[i][j]);
          acc[i][j] = mfma(a_h[i], b_l[j], acc[i][j]);
          if constexpr (ALO) acc[i][j] = mfma(a_l[i], b_h[j], acc[i][j]);
        }
    }
  }

  // per-row norms: the two threads of a row hold halves of its sum
  rs += __shfl_xor(rs, 1);
  if ((tid & 1) == 0) {
    const float nrm = sqrtf(rs);
    if constexpr (PHASE == 1) {
      rowscale[srow] = nrm > 0.f ? 1.f / nrm : 0.f;   // zero vector: u is taken as 0
      if (blockIdx.y == 0 && row_ok) nu_out[v0 + r0 + srow] = nrm;
    } else {
      if (blockIdx.y == 0 && row_ok) gamma_out[v0 + r0 + srow] = nrm;
    }
  }
  __syncthreads();

  const Header* hdr = reinterpret_cast<const Header*>(params);
  constexpr int L = 1 << (BITS - 1);
  float T[L / 2 > 1 ? L / 2 - 1 : 1], M[L / 2];
  if constexpr (PHASE == 1) {
#pragma unroll
    for (int k = 0; k < L / 2 - 1; ++k) T[k] = hdr->tpos[k];
#pragma unroll
    for (int k = 0; k < L / 2; ++k) M[k] = hdr->mpos[k];
  }
  const int groups = d / 32;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = c0 + wn + 32 * j + (lane & 31);
      const int w = (c0 + wn + 32 * j) / 32;     // coordinate group of this 32-column tile
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm + 32 * i + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
        const int rowA = wm + 32 * i + 8 * (r / 4) + (r % 4);     // vector of bits 0..31
        const bool okr = r0 + row < rows;
        if constexpr (PHASE == 1) {
          const float u = acc[i][j][r] * rowscale[row];
          bool bit[3] = {false, false, false};
          float c;
          if constexpr (BITS == 2) {
            bit[0] = u >= 0.f;
            c = bit[0] ? M[0] : -M[0];
          } else if constexpr (BITS == 3) {
            bit[1] = u >= 0.f;
            bit[0] = u >= (bit[1] ? T[0] : -T[0]);
            const float mag = (bit[0] == bit[1]) ? M[1] : M[0];
            c = bit[1] ? mag : -mag;
          } else {
            bit[2] = u >= 0.f;
            bit[1] = u >= (bit[2] ? T[1] : -T[1]);
            const bool e1 = (bit[1] == bit[2]);
            const float t2 = e1 ? T[2] : T[0];
            bit[0] = u >= (bit[2] ? t2 : -t2);
            const bool e0 = (bit[0] == bit[2]);
            const float mag = e1 ? (e0 ? M[3] : M[2]) : (e0 ? M[1] : M[0]);
            c = bit[2] ? mag : -mag;
          }
          const float rv = u - c;
          const __bf16 hi = (__bf16)rv;
          const __bf16 lo = (__bf16)(rv - (float)hi);
          if (okr) {
            const size_t ro = size_t(r0 + row) * d + col;
            rhi[ro] = __builtin_bit_cast(uint16_t, hi);
            rlo[ro] = __builtin_bit_cast(uint16_t, lo);
          }
#pragma unroll
          for (int p = 0; p < BITS - 1; ++p) {
            const uint64_t m = __builtin_amdgcn_ballot_w64(bit[p]);
            if (lane == 0) {
              if (r0 + rowA < rows)
                codes[(size_t(v0 + r0 + rowA) * groups + w) * BITS + p] = uint32_t(m);
              if (r0 + rowA + 4 < rows)
                codes[(size_t(v0 + r0 + rowA + 4) * groups + w) * BITS + p] = uint32_t(m >> 32);
            }
          }
        } else {
          const uint64_t m = __builtin_amdgcn_ballot_w64(acc[i][j][r] >= 0.f);
          if (lane == 0) {
            if (r0 + rowA < rows)
              codes[(size_t(v0 + r0 + rowA) * groups + w) * BITS + BITS - 1] = uint32_t(m);
            if (r0 + rowA + 4 < rows)
              codes[(size_t(v0 + r0 + rowA + 4) * groups + w) * BITS + BITS - 1] = uint32_t(m >> 32);
          }
        }
      }
    }
  }
}

template <int BITS, bool F32IN>
hipError_t run(const unsigned char* params, const Layout& lay, const void* x, int64_t n,
               uint32_t* codes, float* nu, float* gamma, hipStream_t s) {
  const int d = lay.d;
  const uint16_t* pih = reinterpret_cast<const uint16_t*>(params + lay.off_gmat);
  const uint16_t* pil = pih + size_t(d) * d;
  const uint16_t* sph = pil + size_t(d) * d;
  const uint16_t* spl = sph + size_t(d) * d;
  const long ch = n < CHUNK ? long(n) : CHUNK;
  uint16_t* scratch = nullptr;
  hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&scratch), size_t(CHUNK) * d * 4, s);
  if (e != hipSuccess) return e;
  for (long c0 = 0; c0 < n; c0 += ch) {
    const long rows = (n - c0) < ch ? (n - c0) : ch;
    const dim3 grid(unsigned((rows + TM - 1) / TM), unsigned(d / TN));
    const void* xs = F32IN ? static_cast<const void*>(static_cast<const float*>(x) + size_t(c0) * d)
                           : static_cast<const void*>(static_cast<const uint16_t*>(x) + size_t(c0) * d);
    hipLaunchKernelGGL((qgemm_kernel<1, BITS, F32IN>), grid, dim3(256), 0, s, params, xs, rows, pih,
                       pil, d, c0, codes, nu, gamma, scratch, scratch + size_t(CHUNK) * d);
    hipLaunchKernelGGL((qgemm_kernel<2, BITS, F32IN>), grid, dim3(256), 0, s, params,
                       static_cast<const void*>(scratch), rows, sph, spl, d, c0, codes, nu, gamma,
                       nullptr, nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) break;
  }
  const hipError_t f = hipFreeAsync(scratch, s);
  return e != hipSuccess ? e : f;
}

}  // namespace

hipError_t launch_quantize_gemm(const void* params_v, int d, int b, const void* x, int x_dtype,
                                int64_t n, uint32_t* codes, float* nu, float* gamma,
                                hipStream_t s) {
  const unsigned char* params = static_cast<const unsigned char*>(params_v);
  const Layout lay(d, b);
  const bool f32 = x_dtype == 0;
  switch (b) {
    case 2: return f32 ? run<2, true>(params, lay, x, n, codes, nu, gamma, s)
                       : run<2, false>(params, lay, x, n, codes, nu, gamma, s);
    case 3: return f32 ? run<3, true>(params, lay, x, n, codes, nu, gamma, s)
                       : run<3, false>(params, lay, x, n, codes, nu, gamma, s);
    case 4: return f32 ? run<4, true>(params, lay, x, n, codes, nu, gamma, s)
                       : run<4, false>(params, lay, x, n, codes, nu, gamma, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
