// One 16-key tile of the d = 128 scorer (keys' bit planes against the query digits of a quad
// of heads on v_mfma_i32_16x16x64_i8), shared by the scoring scan and the fused attention
// block kernel.  The estimate, the Walsh form of the codebook and the operand layouts are
// described at the scoring kernels ([review, problem statement]; [explainer, step 2];
// [tldr, step 2]).
#pragma once

#include "tq_internal.h"

namespace tq {

typedef int v4i __attribute__((ext_vector_type(4)));

// Masked digit sums of the pair this lane holds in a 16-key tile: query head lane / 16 of the
// quad and key lane % 16.  A: the 2 NW query operand registers of the quad (2 NWU used); w: the
// key's BITS plane words of coordinate group lane / 16.  Registers 0, 1 of the result hold the
// MSE digit sums (hi, lo), 2, 3 the QJL ones; PROD adds the QJL words, without it the MSE
// estimate alone.
template <int BITS, bool PROD>
__device__ __forceinline__ v4i score_tile_sums(const v4i* A, const uint32_t* w) {
  constexpr int NW = score_words(BITS);
  constexpr int NWU = PROD ? NW : NW - 1;     // MSE-only skips the sign plane
  uint32_t word[NW];
  if constexpr (BITS == 4) {
    word[0] = w[0]; word[1] = w[1]; word[2] = w[2];
    word[3] = w[0] ^ w[1] ^ w[2];
    word[4] = w[3];
  } else {
#pragma unroll
    for (int p = 0; p < BITS; ++p) word[p] = w[p];
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
  return acc;
}

// The same sums for one 64-channel group of a key split 64 + 64 (a fractional rate), where one
// MFMA's K = 64 covers the whole channel group: K chunk lane / 16 is coordinate group lane / 32
// of the channel group and bit parity (lane / 16) % 2.  A: the group's NW operand registers
// (one per plane word); w: the key's BITS plane words of coordinate group lane / 32 (the B
// operand's column lane % 16); mj: the lane's parity mask (0x01 or 0x02 in every byte).  The
// result is laid out as score_tile_sums's (head lane / 16, key lane % 16).
template <int BITS, bool PROD>
__device__ __forceinline__ v4i score_split_tile_sums(const v4i* A, const uint32_t* w, uint32_t mj) {
  constexpr int NW = score_words(BITS);
  constexpr int NWU = PROD ? NW : NW - 1;     // MSE-only skips the sign plane
  uint32_t word[NW];
  if constexpr (BITS == 4) {
    word[0] = w[0]; word[1] = w[1]; word[2] = w[2];
    word[3] = w[0] ^ w[1] ^ w[2];
    word[4] = w[3];
  } else {
#pragma unroll
    for (int p = 0; p < BITS; ++p) word[p] = w[p];
  }
  v4i acc = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < NWU; ++i) {
    const uint32_t W = word[i];
    const v4i b = {int(W & mj), int((W >> 2) & mj), int((W >> 4) & mj), int((W >> 6) & mj)};
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[i], b, acc, 0, 0, 0);
  }
  return acc;
}

// The estimate from the digit sums: cst holds the epilogue constants of the lane's head
// (l = nu (s_mse cst.x - cst.y + gamma (s_qjl cst.z - cst.w))); nk, gk: the key's nu and gamma.
template <bool PROD>
__device__ __forceinline__ float score_tile_estimate(const v4i& acc, const float4& cst, float nk, float gk) {
  const int ai = acc[0] * 128 + acc[1];
  float l = fmaf(float(ai), cst.x, -cst.y);
  if constexpr (PROD) {
    const int bi = acc[2] * 128 + acc[3];
    l = fmaf(gk, fmaf(float(bi), cst.z, -cst.w), l);
  }
  return l * nk;
}

// Logit of the pair this lane holds in a 16-key tile (see score_tile_sums); keys past the end
// pass zero words and nu = 0 and get 0.
template <int BITS, bool PROD>
__device__ __forceinline__ float score_tile_logit(const v4i* A, const float4& cst, const uint32_t* w,
                                                  float nk, float gk) {
  return score_tile_estimate<PROD>(score_tile_sums<BITS, PROD>(A, w), cst, nk, gk);
}

}  // namespace tq
