// One decode step of attention over a TurboQuant KV cache: keys carry the inner-product
// quantizer, values the MSE quantizer alone ([review, problem statement]: the two
// quantizers; [news, KV-cache paragraph]: KV caches compressed to about 3 bits):
//   o[g][h] = sum_t softmax_t(scale * l[g][h][t]) * nu_t Pi_v^T chat_t,
// with l the unbiased logit estimate of the keys (the scoring kernels write it, or, for the
// d = 128 scorer's shapes, the block kernel computes it).  Pi_v^T is
// linear, so the weighted sum runs in the values' rotated coordinates and one inverse
// rotation per head finishes it:  o = Pi_v^T a,  a = sum_t p_t nu_t chat_t / sum_t p_t.
//
// attn_block_kernel: one workgroup per (group, pass of AH heads, block of KB keys), 64 keys per
//   wave.  Lanes first hold one key each: scaled logits, the block maximum per head, the
//   weights p = exp(l - max) and p nu.  The weighted sum of the keys' centroids then runs on
//   the integer MFMA through the Walsh form of the codebook (value_block): the weights as
//   exact integer digits, the value codes' bit planes as 0/1 bytes.  Out: per block and head
//   the maximum, the sum of p and the weighted sum of centroids.
// attn_fused_kernel: the same block work for d = 128 keys scored by the int8 scorer, with the
//   logits of the block's keys computed in the workgroup (score_tile.h) from the query operands
//   of the scorer's query prep instead of read from memory: per wave 4 tiles of 16 keys, lane l
//   holding head l / 16 of the quad for key l % 16 of each tile, so the block maxima, the sums
//   of p and the weights' scales are reductions over 16-lane rows, and the weights land in the
//   layout of the value MFMA's output (lane l: head l / 16).
// attn_combine_kernel: one workgroup per (group, head): merges the blocks (log-sum-exp) and
//   applies Pi_v^T; threads split both sums into slices of independent float4 loads (rows
//   of Pi_v are contiguous, so a slice reads coalesced columns), the first loads of both
//   issued before the maximum and the sum are reduced (DPP wave reductions, four waves up to
//   d = 1024).
#include "score_tile.h"

#include <algorithm>
#include <type_traits>
#include <cmath>

namespace tq {
namespace {

constexpr int AH = 4;      // query heads per pass
constexpr int KB = 256;    // keys per workgroup (64 per wave)
constexpr int CT = 1024;   // threads of a combine workgroup for d > 1024 (256 below)

// The value operands of one channel group for the block kernel.
struct BlockGroup {
  const unsigned char* params_v;
  const uint32_t* vcodes;
  const float* vnu;
  int d;
  float* part_m;
  float* part_s;
  float* part_acc;
};

// The key operands of the fused block kernel: the d = 128 key cache (4 coordinate groups of
// BITS plane words per key, nu, gamma) and the query operands of the scorer's query prep, one
// block per quad of query heads.
struct KeyOps {
  const uint32_t* codes;
  const float* nu;
  const float* gamma;
  const unsigned char* qws;
};

// One workgroup's block (256 keys) of one value channel group.  BV: index planes of a value
// (1..3); NC: 64-coordinate steps per chunk (NC divides d / 64).
// With the Walsh form of the odd-symmetric codebook, chat_tc = sum_P e_P (2 B_P,tc - 1) over
// the index bit planes B_P (three index bits add the plane b0 ^ b1 ^ b2), so for head h and
// coordinate c
//   sum_t w_ht chat_tc = sum_P e_P (2 sum_t w_ht B_P,tc - sum_t w_ht).
// Per wave and head the weights become integers v = round(w (2^21 - 1) / max_t w), three
// 7-bit digits each, and v_mfma_i32_16x16x64_i8 sums them exactly over the keys whose plane bit
// is set: A = 16 rows (head h: rows 4 h + {digit 0, 1, 2, zero}) over the wave's 64 keys, B =
// those keys' bits of 16 coordinates as bytes 0/1.  In the 16x16 accumulator layout lane l
// ends with head l / 16 and the tile's column l % 16, its three digit sums in registers 0..2.
// The value codes are staged in LDS byte-transposed, [plane][32-coordinate group][byte of the
// word][key], so one 16-byte read gives a lane one byte (8 coordinates) of 16 keys.  For a
// chunk of 128 coordinates per plane (NC even) column n is byte n and MFMA j takes bit j, so
// one read feeds the plane's 8 MFMAs and lane l ends with coordinates 8 (l % 16) .. + 7; for
// NC odd column n is coordinate n of a 16-coordinate tile (one read per MFMA).  Lanes hold their keys in the same order in A and B, so the MFMA's own
// order within K does not matter.  The first chunk's code words are loaded before anything
// waits, so their latency overlaps the logits and the softmax prologue.
// Row and wave-wide reductions without LDS: within each 16-lane row by DPP rotations (every
// lane of the row ends with the row's result), then, for a wave, across the four rows from
// lanes 0, 16, 32, 48 (wave uniform results).
template <int K>
__device__ __forceinline__ int dpp_ror(int v) {   // row_ror:K
  return __builtin_amdgcn_update_dpp(v, v, 0x120 + K, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_quad(uint32_t v) {   // quad_perm CTRL
  return uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_max_dpp(float v) {
  v = fmaxf(v, __int_as_float(dpp_ror<8>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_ror<4>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_ror<2>(__float_as_int(v))));
  return fmaxf(v, __int_as_float(dpp_ror<1>(__float_as_int(v))));
}
__device__ __forceinline__ float row_sum_dpp(float v) {
  v += __int_as_float(dpp_ror<8>(__float_as_int(v)));
  v += __int_as_float(dpp_ror<4>(__float_as_int(v)));
  v += __int_as_float(dpp_ror<2>(__float_as_int(v)));
  return v + __int_as_float(dpp_ror<1>(__float_as_int(v)));
}
__device__ __forceinline__ int row_sum_int(int v) {
  v += dpp_ror<8>(v);
  v += dpp_ror<4>(v);
  v += dpp_ror<2>(v);
  return v + dpp_ror<1>(v);
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = row_max_dpp(v);
  const int i = __float_as_int(v);
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(i, 0)), __int_as_float(__builtin_amdgcn_readlane(i, 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(i, 32)), __int_as_float(__builtin_amdgcn_readlane(i, 48))));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = row_sum_dpp(v);
  const int i = __float_as_int(v);
  return (__int_as_float(__builtin_amdgcn_readlane(i, 0)) + __int_as_float(__builtin_amdgcn_readlane(i, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(i, 32)) + __int_as_float(__builtin_amdgcn_readlane(i, 48)));
}
__device__ __forceinline__ int wave_sum_int(int v) {
  v = row_sum_int(v);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// The weighted sums of one chunk of value coordinates (c0 .. c0 + 64 NC - 1) over the wave's
// 64 keys, and the block's partial sums of the chunk: the keys' plane words pw (the lane's key,
// the chunk's 2 NC coordinate groups) are staged byte-transposed in the wave's LDS rows kb, the
// value MFMAs run against the weight digits A, and the workgroup's four waves are summed into
// part_acc.  e: the codebook's Walsh coefficients; tsum_l, inv_l: the sum of the integer weights
// of the lane's head and their scale.
template <int BV, int NC>
__device__ __forceinline__ void value_chunk(const BlockGroup& bg, const uint32_t (&pw)[2 * NC][BV], const v4i& A,
                                            const float (&e)[BV == 3 ? 4 : BV], int tsum_l, float inv_l,
                                            long prow, long nh, long nkb, long kblk, int c0,
                                            float (*accs)[AH][64 * NC], unsigned char* kb) {
  constexpr int NE = BV == 3 ? 4 : BV;      // Walsh planes: b0 [, b1 [, b2, b0^b1^b2]]
  constexpr int NG = 2 * NC;                // 32-coordinate groups per chunk
  const int d = bg.d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 4;                     // this lane's head in the MFMA output
  const int ksl = 16 * hl;                      // first of this lane's 16 keys in A and B
  const uint32_t sh = lane & 7;                 // bit of the byte for coordinate lane % 16
  const int qi = lane & 3;                      // the lane's byte in the quad transpose
  // byte selectors of the two transpose steps (v_perm: 0..3 own bytes, 4..7 the partner's)
  const uint32_t sel_a = (qi & 2) ? 0x03020706u : 0x05040100u;
  const uint32_t sel_b = (qi & 1) ? 0x03070105u : 0x06020400u;
  // stage the chunk's words byte-transposed (the xor plane formed here): a 4 x 4 byte
  // transpose within each lane quad (16-bit halves with the lane two apart, then bytes with
  // the neighbour) leaves lane 4 j + i with byte i of keys 4 j .. 4 j + 3, one dword store
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    uint32_t word[NE];
#pragma unroll
    for (int p = 0; p < BV; ++p) word[p] = pw[gg][p];
    if constexpr (BV == 3) word[3] = pw[gg][0] ^ pw[gg][1] ^ pw[gg][2];
#pragma unroll
    for (int pp = 0; pp < NE; ++pp) {
      const uint32_t x = __builtin_amdgcn_perm(dpp_quad<0x4E>(word[pp]), word[pp], sel_a);
      const uint32_t y = __builtin_amdgcn_perm(dpp_quad<0xB1>(x), x, sel_b);
      *reinterpret_cast<uint32_t*>(kb + ((pp * NG + gg) * 4 + qi) * 64 + (lane & ~3)) = y;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

  float acc[2 * NG];
#pragma unroll
  for (int i = 0; i < 2 * NG; ++i) acc[i] = 0.f;
  if constexpr (NC % 2 == 0) {
    // MFMA column n = byte n of 16 consecutive bytes of the keys' plane (byte n of the chunk
    // holds coordinates 8 n .. 8 n + 7), MFMA j = bit j: one 16-byte read per lane feeds the
    // plane's 8 MFMAs of a 128-coordinate slice, and the lane ends with coordinates
    // 8 (16 rr + lane % 16) + j of its head
#pragma unroll
    for (int pp = 0; pp < NE; ++pp) {
      v4i r[2 * NG];
#pragma unroll
      for (int rr = 0; rr < NC / 2; ++rr) {
        const uint4 q = *reinterpret_cast<const uint4*>(kb + (pp * NG * 4 + 16 * rr + (lane & 15)) * 64 + ksl);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const v4i B = {int((q.x >> j) & 0x01010101u), int((q.y >> j) & 0x01010101u),
                         int((q.z >> j) & 0x01010101u), int((q.w >> j) & 0x01010101u)};
          r[8 * rr + j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, v4i{0, 0, 0, 0}, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 2 * NG; ++i) {
        const int S = r[i][2] * 16384 + r[i][1] * 128 + r[i][0];
        acc[i] = fmaf(e[pp], float(2 * S - tsum_l), acc[i]);
      }
    }
#pragma unroll
    for (int rr = 0; rr < NC / 2; ++rr) {
      float4* dst = reinterpret_cast<float4*>(&accs[wave][hl][8 * (16 * rr + (lane & 15))]);
      dst[0] = make_float4(acc[8 * rr] * inv_l, acc[8 * rr + 1] * inv_l, acc[8 * rr + 2] * inv_l,
                           acc[8 * rr + 3] * inv_l);
      dst[1] = make_float4(acc[8 * rr + 4] * inv_l, acc[8 * rr + 5] * inv_l, acc[8 * rr + 6] * inv_l,
                           acc[8 * rr + 7] * inv_l);
    }
  } else {
#pragma unroll
    for (int pp = 0; pp < NE; ++pp) {
      // the plane's MFMAs first, then their results (the MFMA latency overlaps the gathers)
      v4i r[2 * NG];
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          // coordinate 32 gg + 16 half + lane % 16: byte 2 half + (lane % 16) / 8 of the word
          const int by = 2 * half + ((lane & 15) >> 3);
          const uint4 q = *reinterpret_cast<const uint4*>(kb + ((pp * NG + gg) * 4 + by) * 64 + ksl);
          const v4i B = {int((q.x >> sh) & 0x01010101u), int((q.y >> sh) & 0x01010101u),
                         int((q.z >> sh) & 0x01010101u), int((q.w >> sh) & 0x01010101u)};
          r[2 * gg + half] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, v4i{0, 0, 0, 0}, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 2 * NG; ++i) {
        const int S = r[i][2] * 16384 + r[i][1] * 128 + r[i][0];
        acc[i] = fmaf(e[pp], float(2 * S - tsum_l), acc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 2 * NG; ++i) accs[wave][hl][16 * i + (lane & 15)] = acc[i] * inv_l;
  }
  __syncthreads();
  for (int ei = tid; ei < AH * 64 * NC; ei += 256) {
    const int hh = ei / (64 * NC), c = ei % (64 * NC);
    if (hh < nh)
      bg.part_acc[((prow + hh) * nkb + kblk) * d + c0 + c] =
          (accs[0][hh][c] + accs[1][hh][c]) + (accs[2][hh][c] + accs[3][hh][c]);
  }
  __syncthreads();
}

// KBITS = 0: the logits come from memory (one per (head, key)); KBITS = b of d = 128 keys: the
// workgroup scores its keys itself (PROD: the inner-product estimate, else the MSE one).
// red: 8 rows of AH floats (the block maxima of the waves, then their sums of p).
template <int BV, int NC, int KBITS = 0, bool PROD = true>
__device__ __forceinline__ void value_block(const BlockGroup& bg, const KeyOps& ko, const float* __restrict__ logits,
                                            long G, long T, long nkb, long passes, float scale,
                                            long blk, float (*red)[AH], float (*accs)[AH][64 * NC],
                                            unsigned char* kb_all, unsigned char* ab_all) {
  static_assert(BV >= 1 && BV <= 3, "one to three index planes");
  constexpr int NE = BV == 3 ? 4 : BV;      // Walsh planes: b0 [, b1 [, b2, b0^b1^b2]]
  constexpr int NG = 2 * NC;                // 32-coordinate groups per chunk
  constexpr float kVMax = 2097151.f;        // 2^21 - 1: three 7-bit digits
  const unsigned char* __restrict__ params_v = bg.params_v;
  const uint32_t* __restrict__ vcodes = bg.vcodes;
  const float* __restrict__ vnu = bg.vnu;
  const int d = bg.d;
  const Header* hdr = reinterpret_cast<const Header*>(params_v);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  unsigned char* kb = kb_all + wave * (NE * NG * 4 * 64);   // [plane][group][byte][key]
  unsigned char* ab = ab_all + wave * (16 * 64);            // [row][key] weight digits

  const long kblk = blk % nkb;
  const long gp = blk / nkb;
  const long g = gp / passes;
  const long h0 = (gp % passes) * AH;
  const long nh = G - h0 < AH ? G - h0 : AH;
  const long tw0 = kblk * KB + wave * 64;
  const long t = tw0 + lane;
  const bool valid = t < T;
  const int W = d / 32;

  // the lane's key's plane words of one chunk; lanes past the end read the last key's words
  // (their weights are zero, so their bits add nothing), which keeps the loads unconditional
  uint32_t pw[NG][BV];
  const long tc = valid ? t : T - 1;
  auto load_words = [&](int c0) {
    const uint32_t* kc = vcodes + (size_t(g * T + tc) * W + c0 / 32) * BV;
#pragma unroll
    for (int gg = 0; gg < NG; ++gg)
#pragma unroll
      for (int p = 0; p < BV; ++p) pw[gg][p] = kc[gg * BV + p];
  };
  // loads complete in issue order, so the operands needed first are loaded first: with logits
  // from memory, the value words (their latency overlaps the softmax prologue); when the block
  // scores its keys, the key words (the value words follow them, below)
  if constexpr (KBITS == 0) load_words(0);

  float e[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) e[i] = hdr->e[i];

  float inv_l = 0.f;      // this lane's head (lane / 16): 1 / scale
  int tsum_l = 0;         // this lane's head: sum of its integer weights over the wave
  const long prow = g * G + h0;                 // partial rows of this pass: prow + hh
  if constexpr (KBITS == 0) {
    // scaled logits of the lane's key, block maximum per head, weights p nu, sums of p
    float l[AH];
#pragma unroll
    for (int hh = 0; hh < AH; ++hh) {
      const long h = h0 + (hh < nh ? hh : nh - 1);
      l[hh] = valid ? scale * logits[size_t(g * G + h) * T + t] : -INFINITY;
      const float m = wave_max_dpp(l[hh]);
      if (lane == 0) red[wave][hh] = m;
    }
    __syncthreads();
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
      const float sp = wave_sum_dpp(p);
      if (lane == 0) red[wave][hh] = sp;
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < AH; ++hh) {
      if (tid == hh && hh < nh) {
        bg.part_m[(prow + hh) * nkb + kblk] = M[hh];
        bg.part_s[(prow + hh) * nkb + kblk] = (red[0][hh] + red[1][hh]) + (red[2][hh] + red[3][hh]);
      }
    }

    // integer weights of the wave's keys and the A operand (rows 4 hh + j: digit j of head hh)
#pragma unroll
    for (int hh = 0; hh < AH; ++hh) {
      const float wm = wave_max_dpp(w[hh]);
      const float sc = wm > 0.f ? kVMax / wm : 0.f;
      int v = int(rintf(w[hh] * sc));
      v = v < 2097151 ? v : 2097151;
      const int ts = wave_sum_int(v);
      if ((lane >> 4) == hh) {
        inv_l = wm * (1.f / kVMax);
        tsum_l = ts;
      }
      ab[(4 * hh + 0) * 64 + lane] = (unsigned char)(v & 127);
      ab[(4 * hh + 1) * 64 + lane] = (unsigned char)((v >> 7) & 127);
      ab[(4 * hh + 2) * 64 + lane] = (unsigned char)(v >> 14);
      ab[(4 * hh + 3) * 64 + lane] = 0;
    }
  } else {
    // the block's logits: 4 tiles of 16 keys per wave, lane l holding head l / 16 of the quad
    // for key 16 u + l % 16 of the wave (tile u)
    constexpr int NW = score_words(KBITS);
    constexpr int NWU = PROD ? NW : NW - 1;
    const int hs = lane >> 4;
    const unsigned char* qb = ko.qws + size_t(gp) * score_ws_per_group(KBITS);
    v4i QA[2 * NW];
#pragma unroll
    for (int m = 0; m < 2 * NWU; ++m) QA[m] = reinterpret_cast<const v4i*>(qb)[m * 64 + lane];
    const float4 cst = reinterpret_cast<const float4*>(qb + size_t(2 * NW) * 64 * 16)[hs];
    const uint32_t* kc = ko.codes + size_t(g) * T * 4 * KBITS;
    uint32_t kw[4][KBITS];
    float nk[4], gk[4], nv[4];
    bool ok[4];
    // keys past the end read the last key (their logits are replaced by -inf below), so that
    // no load sits under a branch
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long key = tw0 + 16 * u + (lane & 15);
      ok[u] = key < T;
      const long kr = ok[u] ? key : T - 1;
      const uint32_t* src = kc + (size_t(kr) * 4 + hs) * KBITS;
      if constexpr (KBITS == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(src);
        kw[u][0] = v.x; kw[u][1] = v.y; kw[u][2] = v.z; kw[u][3] = v.w;
      } else if constexpr (KBITS == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(src);
        kw[u][0] = v.x; kw[u][1] = v.y;
      } else {
#pragma unroll
        for (int p = 0; p < KBITS; ++p) kw[u][p] = src[p];
      }
      nk[u] = ko.nu[g * T + kr];
      gk[u] = PROD ? ko.gamma[g * T + kr] : 0.f;
      nv[u] = vnu[g * T + kr];
    }
    load_words(0);   // in flight while the logits and the softmax are formed
    // every load is issued before the first use (the scheduler would otherwise move the later
    // tiles' loads down to their uses, one round trip each)
    __builtin_amdgcn_sched_barrier(0);
    float l[4], mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float lv = scale * score_tile_logit<KBITS, PROD>(QA, cst, kw[u], nk[u], gk[u]);
      l[u] = ok[u] ? lv : -INFINITY;
      mx = fmaxf(mx, l[u]);
    }
    mx = row_max_dpp(mx);
    if ((lane & 15) == 0) red[wave][hs] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0][hs], red[1][hs]), fmaxf(red[2][hs], red[3][hs]));
    float w[4], sp = 0.f, wmx = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float p = ok[u] ? __expf(l[u] - M) : 0.f;
      sp += p;
      w[u] = p * nv[u];
      wmx = fmaxf(wmx, w[u]);
    }
    sp = row_sum_dpp(sp);
    if ((lane & 15) == 0) red[4 + wave][hs] = sp;
    // integer weights (the lane's head is also its head in the value MFMA's output) and the
    // A operand rows 4 hs + j: digit j of head hs
    const float wm = row_max_dpp(wmx);
    const float sc = wm > 0.f ? kVMax / wm : 0.f;
    int vs = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int v = int(rintf(w[u] * sc));
      v = v < 2097151 ? v : 2097151;
      vs += v;
      const int key = 16 * u + (lane & 15);
      ab[(4 * hs + 0) * 64 + key] = (unsigned char)(v & 127);
      ab[(4 * hs + 1) * 64 + key] = (unsigned char)((v >> 7) & 127);
      ab[(4 * hs + 2) * 64 + key] = (unsigned char)(v >> 14);
      ab[(4 * hs + 3) * 64 + key] = 0;
    }
    tsum_l = row_sum_int(vs);
    inv_l = wm * (1.f / kVMax);
    __syncthreads();
    if (tid < nh) {
      bg.part_m[(prow + tid) * nkb + kblk] =
          fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
      bg.part_s[(prow + tid) * nkb + kblk] = (red[4][tid] + red[5][tid]) + (red[6][tid] + red[7][tid]);
    }
  }

  // the staging writes and the reads below use other types: order them explicitly
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  const v4i A = *reinterpret_cast<const v4i*>(ab + (lane & 15) * 64 + 16 * (lane >> 4));

  for (int c0 = 0; c0 < d; c0 += 64 * NC) {
    if (c0 > 0) load_words(c0);
    value_chunk<BV, NC>(bg, pw, A, e, tsum_l, inv_l, prow, nh, nkb, kblk, c0, accs, kb);
  }
}

// grid: the blocks of value channel group 0, then those of group 1 (BV1 > 0: a fractional
// rate's second value group with the same chunk shape).
template <int BV0, int BV1, int NC>
__global__ __launch_bounds__(256) void attn_block_kernel(BlockGroup b0, BlockGroup b1, long blocks0,
                                                         const float* __restrict__ logits, long G,
                                                         long T, long nkb, long passes, float scale) {
  __shared__ float red[8][AH];
  __shared__ __align__(16) float accs[4][AH][64 * NC];
  __shared__ uint4 kbytes[4 * 4 * 2 * NC * 4 * 64 / 16];   // [wave][plane][group][byte][key]
  __shared__ uint4 abytes[4 * 16 * 64 / 16];               // [wave][row][key] weight digits
  unsigned char* kb = reinterpret_cast<unsigned char*>(kbytes);
  unsigned char* ab = reinterpret_cast<unsigned char*>(abytes);
  const long blk = blockIdx.x;
  if constexpr (BV1 > 0) {
    if (blk >= blocks0) {
      value_block<BV1, NC>(b1, KeyOps{}, logits, G, T, nkb, passes, scale, blk - blocks0, red, accs, kb, ab);
      return;
    }
  }
  value_block<BV0, NC>(b0, KeyOps{}, logits, G, T, nkb, passes, scale, blk, red, accs, kb, ab);
}

// d = 128 keys and values: the block's logits computed in the workgroup (grid: groups x quads
// of heads x key blocks, as attn_block_kernel's).  At most 128 VGPRs, so that four workgroups
// (one wave per SIMD each) stay resident per CU: a decode layer's whole grid in one round.
template <int KBITS, bool PROD, int BV>
__global__ __launch_bounds__(256, 4) void attn_fused_kernel(KeyOps ko, BlockGroup bg, long G, long T, long nkb,
                                                         long passes, float scale) {
  constexpr int NC = 2;
  __shared__ float red[8][AH];
  __shared__ __align__(16) float accs[4][AH][64 * NC];
  __shared__ uint4 kbytes[4 * 4 * 2 * NC * 4 * 64 / 16];   // [wave][plane][group][byte][key]
  __shared__ uint4 abytes[4 * 16 * 64 / 16];               // [wave][row][key] weight digits
  value_block<BV, NC, KBITS, PROD>(bg, ko, nullptr, G, T, nkb, passes, scale, blockIdx.x, red, accs,
                                   reinterpret_cast<unsigned char*>(kbytes),
                                   reinterpret_cast<unsigned char*>(abytes));
}

// ------------------------------------------------- fused blocks of a 64 + 64 split cache
// The key operands of the fused split block kernel: the two channel groups' key caches (each
// [groups][T] keys of 2 coordinate groups x b plane words, nu, gamma) and the query operands
// that the split scorer's query prep wrote (score_split_ws_per_group bytes per quad of heads).
struct SplitKeyOps {
  const uint32_t* codes0;
  const float* nu0;
  const float* gamma0;
  const uint32_t* codes1;
  const float* nu1;
  const float* gamma1;
  const unsigned char* qws;
};

// A key's BITS plane words of one coordinate group (one vector load where the size allows).
template <int BITS>
__device__ __forceinline__ void load_plane_words(const uint32_t* src, uint32_t* w) {
  if constexpr (BITS == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(src);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (BITS == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(src);
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int p = 0; p < BITS; ++p) w[p] = src[p];
  }
}

// The block work of attn_fused_kernel for keys and values held as two 64-channel groups (keys
// at KB0, KB1 bits, values at BV0, BV1 index planes), inner-product keys.  The logits are the
// split scorer's (score_split_tile_sums per key group, the two estimates added); the softmax is
// shared, and each value group then forms its own weights p nu_v,g, digits and 64-coordinate
// value sums into its own partials (both groups' partials carry the same maxima and sums of p).
// At most 168 VGPRs (three waves per SIMD).
template <int KB0, int KB1, int BV0, int BV1>
__global__ __launch_bounds__(256, 3) void attn_fused_split_kernel(SplitKeyOps ko, BlockGroup bg0, BlockGroup bg1,
                                                                long G, long T, long nkb, long passes,
                                                                float scale) {
  constexpr int NW0 = score_words(KB0), NW1 = score_words(KB1);
  constexpr int NE0 = BV0 == 3 ? 4 : BV0, NE1 = BV1 == 3 ? 4 : BV1;
  constexpr int NEM = NE0 > NE1 ? NE0 : NE1;
  constexpr float kVMax = 2097151.f;        // 2^21 - 1: three 7-bit digits
  __shared__ float red[8][AH];
  __shared__ __align__(16) float accs[4][AH][64];
  __shared__ uint4 kbytes[4 * NEM * 2 * 4 * 64 / 16];      // [wave][plane][group][byte][key]
  __shared__ uint4 abytes[4 * 16 * 64 / 16];               // [wave][row][key] weight digits
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  unsigned char* kb = reinterpret_cast<unsigned char*>(kbytes) + wave * (NEM * 2 * 4 * 64);
  unsigned char* ab = reinterpret_cast<unsigned char*>(abytes) + wave * (16 * 64);
  const long blk = blockIdx.x;
  const long kblk = blk % nkb;
  const long gp = blk / nkb;
  const long g = gp / passes;
  const long h0 = (gp % passes) * AH;
  const long tw0 = kblk * KB + wave * 64;
  const long prow = g * G + h0;
  const int hs = lane >> 4;                 // the lane's head (rows of the MFMA outputs)
  const int cg = lane >> 5;                 // B operand: coordinate group of the channel group
  const uint32_t mj = 0x01010101u << ((lane >> 4) & 1);   // and bit parity

  // the quad's query operands, then every key and value load of the block
  const unsigned char* qb = ko.qws + size_t(gp) * score_split_ws_per_group(KB0, KB1);
  v4i A0[NW0], A1[NW1];
#pragma unroll
  for (int m = 0; m < NW0; ++m) A0[m] = reinterpret_cast<const v4i*>(qb)[m * 64 + lane];
#pragma unroll
  for (int m = 0; m < NW1; ++m) A1[m] = reinterpret_cast<const v4i*>(qb + size_t(NW0) * 64 * 16)[m * 64 + lane];
  const float4* cst = reinterpret_cast<const float4*>(qb + size_t(NW0 + NW1) * 64 * 16);
  const float4 c0 = cst[hs], c1 = cst[AH + hs];
  const uint32_t* kc0 = ko.codes0 + size_t(g) * T * 2 * KB0;
  const uint32_t* kc1 = ko.codes1 + size_t(g) * T * 2 * KB1;
  uint32_t kw0[4][KB0], kw1[4][KB1];
  float nk0[4], nk1[4], gk0[4], gk1[4], nv0[4], nv1[4];
  // keys past the end read the last key (their logits are replaced by -inf below), so that no
  // load sits under a branch
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const long key = tw0 + 16 * u + (lane & 15);
    const long kr = key < T ? key : T - 1;
    load_plane_words<KB0>(kc0 + (size_t(kr) * 2 + cg) * KB0, kw0[u]);
    load_plane_words<KB1>(kc1 + (size_t(kr) * 2 + cg) * KB1, kw1[u]);
    nk0[u] = ko.nu0[g * T + kr];
    nk1[u] = ko.nu1[g * T + kr];
    gk0[u] = ko.gamma0[g * T + kr];
    gk1[u] = ko.gamma1[g * T + kr];
    nv0[u] = bg0.vnu[g * T + kr];
    nv1[u] = bg1.vnu[g * T + kr];
    // loads return in issue order: a tile's loads stay together, ahead of the next tile's
    __builtin_amdgcn_sched_barrier(0);
  }
  // the value words of key tw0 + lane (both groups' 2 coordinate groups), in flight while the
  // logits and the softmax are formed
  const long t = tw0 + lane;
  const long tc = t < T ? t : T - 1;
  uint32_t pw0[2][BV0], pw1[2][BV1];
  {
    const uint32_t* v0 = bg0.vcodes + size_t(g * T + tc) * 2 * BV0;
    const uint32_t* v1 = bg1.vcodes + size_t(g * T + tc) * 2 * BV1;
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
#pragma unroll
      for (int p = 0; p < BV0; ++p) pw0[gg][p] = v0[gg * BV0 + p];
#pragma unroll
      for (int p = 0; p < BV1; ++p) pw1[gg][p] = v1[gg * BV1 + p];
    }
  }
  // every load is issued before the first use
  __builtin_amdgcn_sched_barrier(0);

  float l[4], mx = -INFINITY;
  bool ok[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    ok[u] = tw0 + 16 * u + (lane & 15) < T;
    const v4i s0 = score_split_tile_sums<KB0, true>(A0, kw0[u], mj);
    const v4i s1 = score_split_tile_sums<KB1, true>(A1, kw1[u], mj);
    const float lv = scale * (score_tile_estimate<true>(s0, c0, nk0[u], gk0[u]) +
                              score_tile_estimate<true>(s1, c1, nk1[u], gk1[u]));
    l[u] = ok[u] ? lv : -INFINITY;
    mx = fmaxf(mx, l[u]);
  }
  mx = row_max_dpp(mx);
  if ((lane & 15) == 0) red[wave][hs] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0][hs], red[1][hs]), fmaxf(red[2][hs], red[3][hs]));
  float p[4], sp = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    p[u] = ok[u] ? __expf(l[u] - M) : 0.f;
    sp += p[u];
  }
  sp = row_sum_dpp(sp);
  if ((lane & 15) == 0) red[4 + wave][hs] = sp;
  __syncthreads();
  if (tid < AH) {
    const float bm = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
    const float bs = (red[4][tid] + red[5][tid]) + (red[6][tid] + red[7][tid]);
    bg0.part_m[(prow + tid) * nkb + kblk] = bm;
    bg0.part_s[(prow + tid) * nkb + kblk] = bs;
    bg1.part_m[(prow + tid) * nkb + kblk] = bm;
    bg1.part_s[(prow + tid) * nkb + kblk] = bs;
  }

  // one value group: weights p nu_v, their digits as the A operand (rows 4 hs + j: digit j of
  // head hs; the lane's head is also its head in the value MFMA's output), the value sums
  auto value_group_sums = [&](const BlockGroup& bg, const float (&nv)[4], auto& pw, auto bv_tag) {
    constexpr int BV = decltype(bv_tag)::value;
    constexpr int NE = BV == 3 ? 4 : BV;
    const Header* hdr = reinterpret_cast<const Header*>(bg.params_v);
    float e[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) e[i] = hdr->e[i];
    float w[4], wmx = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      w[u] = p[u] * nv[u];
      wmx = fmaxf(wmx, w[u]);
    }
    const float wm = row_max_dpp(wmx);
    const float sc = wm > 0.f ? kVMax / wm : 0.f;
    int vs = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int v = int(rintf(w[u] * sc));
      v = v < 2097151 ? v : 2097151;
      vs += v;
      const int key = 16 * u + (lane & 15);
      ab[(4 * hs + 0) * 64 + key] = (unsigned char)(v & 127);
      ab[(4 * hs + 1) * 64 + key] = (unsigned char)((v >> 7) & 127);
      ab[(4 * hs + 2) * 64 + key] = (unsigned char)(v >> 14);
      ab[(4 * hs + 3) * 64 + key] = 0;
    }
    const int tsum_l = row_sum_int(vs);
    const float inv_l = wm * (1.f / kVMax);
    // the staging writes and the reads below use other types: order them explicitly
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const v4i A = *reinterpret_cast<const v4i*>(ab + (lane & 15) * 64 + 16 * (lane >> 4));
    value_chunk<BV, 1>(bg, pw, A, e, tsum_l, inv_l, prow, AH, nkb, kblk, 0, accs, kb);
  };
  value_group_sums(bg0, nv0, pw0, std::integral_constant<int, BV0>{});
  // (value_chunk ends with a barrier: the wave's digit and staging rows are free again)
  value_group_sums(bg1, nv1, pw1, std::integral_constant<int, BV1>{});
}

// The block partials and output columns of one value channel group.
struct CombineGroup {
  const unsigned char* params_v;
  size_t off_pi;
  int d;
  const float* part_m;
  const float* part_s;
  const float* part_acc;
  float* out;                        // the group's first output column
};

// grid: the rows (group * G + head) of channel group 0, then those of group 1 (a fractional
// rate's second value group; none otherwise).  out rows are opitch floats apart (a channel
// group of wider output rows: its columns only).  CTT threads, CTT / 4 >= d / 4 of the
// larger group (256 up to d = 1024, else 1024): a thread owns one float4 column of a slice.
template <int CTT>
__global__ __launch_bounds__(CTT) void attn_combine_kernel(CombineGroup c0, CombineGroup c1, long rows0,
                                                           long nkb, long opitch) {
  constexpr int NW = CTT / 64;
  constexpr int PF = CTT <= 256 ? 16 : 8;   // loads of each sum issued before the reductions
  extern __shared__ float4 lds4[];   // [slices][d / 4] partial sums, then a[d / 4]
  __shared__ float red[2][NW];
  const bool second = long(blockIdx.x) >= rows0;
  const CombineGroup& cg = second ? c1 : c0;
  const long row = second ? long(blockIdx.x) - rows0 : long(blockIdx.x);
  const unsigned char* params_v = cg.params_v;
  const size_t off_pi = cg.off_pi;
  const int d = cg.d;
  const float* part_m = cg.part_m;
  const float* part_s = cg.part_s;
  const float* part_acc = cg.part_acc;
  float* out = cg.out;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* pm = part_m + row * nkb;
  const float* ps = part_s + row * nkb;
  // threads = (float4 column q4, slice sl): a slice sums every nsl-th block (and, for the
  // inverse rotation, every nsl-th row of Pi_v)
  const int d4 = d / 4;
  const int cols = d4 < CTT ? d4 : CTT;
  const int nsl = CTT / cols;
  const int q4 = tid % cols, sl = tid / cols;
  const bool act = sl < nsl;
  const float4* pa = reinterpret_cast<const float4*>(part_acc) + row * nkb * d4;
  const float4* P4 = reinterpret_cast<const float4*>(params_v + off_pi);
  float4 pacc[PF], ppi[PF];
  float pmk[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const long k = sl + long(i) * nsl;
    const int r = sl + i * nsl;
    const bool okk = act && k < nkb, okr = act && r < d;
    pacc[i] = okk ? pa[k * d4 + q4] : make_float4(0.f, 0.f, 0.f, 0.f);
    pmk[i] = okk ? pm[k] : -INFINITY;
    ppi[i] = okr ? P4[size_t(r) * d4 + q4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  // this thread's first block maximum and sum, in the same round trip as the loads above;
  // wave reductions by DPP, then one value per wave through LDS
  const float pm0 = tid < nkb ? pm[tid] : -INFINITY;
  const float ps0 = tid < nkb ? ps[tid] : 0.f;
  float mx = pm0;
  for (long k = tid + CTT; k < nkb; k += CTT) mx = fmaxf(mx, pm[k]);
  mx = wave_max_dpp(mx);
  if (lane == 0) red[0][wave] = mx;
  __syncthreads();
  float M = red[0][0];
#pragma unroll
  for (int i = 1; i < NW; ++i) M = fmaxf(M, red[0][i]);
  float sum = tid < nkb ? __expf(pm0 - M) * ps0 : 0.f;
  for (long k = tid + CTT; k < nkb; k += CTT) sum += __expf(pm[k] - M) * ps[k];
  sum = wave_sum_dpp(sum);
  if (lane == 0) red[1][wave] = sum;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) tot += red[1][i];
  const float inv = 1.f / tot;

  float4* part = lds4;                    // [nsl][d4]
  float4* av = lds4 + size_t(nsl) * d4;   // a / sum, d4 float4
  if (act) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const float e = __expf(pmk[i] - M);   // 0 for the slots past nkb
      v.x = fmaf(e, pacc[i].x, v.x);
      v.y = fmaf(e, pacc[i].y, v.y);
      v.z = fmaf(e, pacc[i].z, v.z);
      v.w = fmaf(e, pacc[i].w, v.w);
    }
#pragma unroll 8
    for (long k = sl + long(PF) * nsl; k < nkb; k += nsl) {
      const float e = __expf(pm[k] - M);
      const float4 x = pa[k * d4 + q4];
      v.x = fmaf(e, x.x, v.x);
      v.y = fmaf(e, x.y, v.y);
      v.z = fmaf(e, x.z, v.z);
      v.w = fmaf(e, x.w, v.w);
    }
    part[sl * d4 + q4] = v;
  }
  __syncthreads();
  // slice sums: the reads of a column's slices are independent, so they go out together
  for (int c4 = tid; c4 < d4; c4 += CTT) {
    float4 v = part[c4];
#pragma unroll 8
    for (int t = 1; t < nsl; ++t) {
      const float4 x = part[t * d4 + c4];
      v.x += x.x; v.y += x.y; v.z += x.z; v.w += x.w;
    }
    v.x *= inv; v.y *= inv; v.z *= inv; v.w *= inv;
    av[c4] = v;
  }
  __syncthreads();
  // out = Pi_v^T a: thread (float4 of outputs q4, slice of rows sl); rows of Pi_v contiguous
  const float* a = reinterpret_cast<const float*>(av);
  if (act) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int r = sl + i * nsl;
      const float ai = r < d ? a[r] : 0.f;
      v.x = fmaf(ppi[i].x, ai, v.x);
      v.y = fmaf(ppi[i].y, ai, v.y);
      v.z = fmaf(ppi[i].z, ai, v.z);
      v.w = fmaf(ppi[i].w, ai, v.w);
    }
#pragma unroll 8
    for (int r = sl + PF * nsl; r < d; r += nsl) {
      const float ai = a[r];
      const float4 x = P4[size_t(r) * d4 + q4];
      v.x = fmaf(x.x, ai, v.x);
      v.y = fmaf(x.y, ai, v.y);
      v.z = fmaf(x.z, ai, v.z);
      v.w = fmaf(x.w, ai, v.w);
    }
    part[sl * d4 + q4] = v;
  }
  __syncthreads();
  float4* o4 = reinterpret_cast<float4*>(out + row * opitch);
  for (int j4 = tid; j4 < d4; j4 += CTT) {
    float4 v = part[j4];
#pragma unroll 8
    for (int t = 1; t < nsl; ++t) {
      const float4 x = part[t * d4 + j4];
      v.x += x.x; v.y += x.y; v.z += x.z; v.w += x.w;
    }
    o4[j4] = v;
  }
}

}  // namespace

// Block partials in the workspace: maxima, sums, weighted centroid sums, each 256-aligned.
size_t attention_part_bytes(int d, int64_t groups, int64_t G, int64_t T) {
  const size_t rk = size_t(groups) * G * size_t((T + KB - 1) / KB);
  return 2 * align256(rk * 4) + align256(rk * size_t(d) * 4);
}

namespace {

// The operands of one value channel group: its partials in part, its output columns at out.
struct ValueGroup {
  BlockGroup blk;
  CombineGroup comb;
  int bv;       // index planes (b_v - 1)
  int nc;       // 64-coordinate steps per chunk of the block kernel
};

ValueGroup value_group(const void* params_v, int d, int b_v, const uint32_t* vcodes, const float* vnu,
                       int64_t groups, int64_t G, int64_t T, float* out, void* part) {
  const unsigned char* pv = static_cast<const unsigned char*>(params_v);
  const long nkb = (T + KB - 1) / KB;
  const size_t rows = size_t(groups) * G;
  unsigned char* pb = static_cast<unsigned char*>(part);
  float* part_m = reinterpret_cast<float*>(pb);
  float* part_s = reinterpret_cast<float*>(pb + align256(rows * nkb * 4));
  float* part_acc = reinterpret_cast<float*>(pb + 2 * align256(rows * nkb * 4));
  const int steps = d / 64;
  const int nc = steps % 4 == 0 ? 4 : steps % 3 == 0 ? 3 : steps % 2 == 0 ? 2 : 1;
  const Layout lay(d, b_v);
  return ValueGroup{BlockGroup{pv, vcodes, vnu, d, part_m, part_s, part_acc},
                    CombineGroup{pv, lay.off_pi, d, part_m, part_s, part_acc, out}, b_v - 1, nc};
}

template <int BV0, int BV1, int NC>
void launch_blocks_t(const ValueGroup& v0, const ValueGroup& v1, long blocks0, long blocks1,
                     const float* logits, int64_t G, int64_t T, float scale, hipStream_t s) {
  const long nkb = (T + KB - 1) / KB;
  const long passes = (G + AH - 1) / AH;
  hipLaunchKernelGGL((attn_block_kernel<BV0, BV1, NC>), dim3(unsigned(blocks0 + blocks1)), dim3(256), 0, s,
                     v0.blk, v1.blk, blocks0, logits, long(G), long(T), nkb, passes, scale);
}

template <int BV0, int NC>
hipError_t launch_blocks_b1(const ValueGroup& v0, const ValueGroup* v1, long blocks, const float* logits,
                            int64_t G, int64_t T, float scale, hipStream_t s) {
  if (!v1) {
    launch_blocks_t<BV0, 0, NC>(v0, v0, blocks, 0, logits, G, T, scale, s);
    return hipSuccess;
  }
  if constexpr (NC <= 2) {
    switch (v1->bv) {
      case 1: launch_blocks_t<BV0, 1, NC>(v0, *v1, blocks, blocks, logits, G, T, scale, s); break;
      case 2: launch_blocks_t<BV0, 2, NC>(v0, *v1, blocks, blocks, logits, G, T, scale, s); break;
      case 3: launch_blocks_t<BV0, 3, NC>(v0, *v1, blocks, blocks, logits, G, T, scale, s); break;
      default: return hipErrorInvalidValue;
    }
    return hipSuccess;
  } else {
    return hipErrorInvalidValue;   // two groups share a grid only with NC <= 2
  }
}

// Block kernel launch for one group (v1 NULL) or for two groups of the same chunk shape with
// NC <= 2 (a fractional rate's value groups of up to 128 channels each), in one grid.
template <int NC>
hipError_t launch_blocks_nc(const ValueGroup& v0, const ValueGroup* v1, long blocks, const float* logits,
                            int64_t G, int64_t T, float scale, hipStream_t s) {
  switch (v0.bv) {
    case 1: return launch_blocks_b1<1, NC>(v0, v1, blocks, logits, G, T, scale, s);
    case 2: return launch_blocks_b1<2, NC>(v0, v1, blocks, logits, G, T, scale, s);
    case 3: return launch_blocks_b1<3, NC>(v0, v1, blocks, logits, G, T, scale, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_blocks_one(const ValueGroup& v, long blocks, const float* logits, int64_t G, int64_t T,
                             float scale, hipStream_t s) {
  hipError_t e;
  switch (v.nc) {
    case 4: e = launch_blocks_nc<4>(v, nullptr, blocks, logits, G, T, scale, s); break;
    case 3: e = launch_blocks_nc<3>(v, nullptr, blocks, logits, G, T, scale, s); break;
    case 2: e = launch_blocks_nc<2>(v, nullptr, blocks, logits, G, T, scale, s); break;
    default: e = launch_blocks_nc<1>(v, nullptr, blocks, logits, G, T, scale, s); break;
  }
  return e != hipSuccess ? e : hipGetLastError();
}

// One combine launch over rows (rows0 of group c0, then rows - rows0 of c1); the thread count
// follows the larger group's d.
hipError_t launch_combine(const CombineGroup& c0, const CombineGroup& c1, long rows, long rows0, long nkb,
                          long opitch, hipStream_t s) {
  const int dmax = std::max(c0.d, rows > rows0 ? c1.d : c0.d);
  const int ct = dmax / 4 <= 256 ? 256 : CT;
  size_t lds = 0;
  for (const int d : {c0.d, rows > rows0 ? c1.d : c0.d}) {
    const int d4 = d / 4, cols = d4 < ct ? d4 : ct, nsl = ct / cols;
    lds = std::max(lds, (size_t(nsl) * d4 + d4) * 16);
  }
  if (ct == 256)
    hipLaunchKernelGGL(attn_combine_kernel<256>, dim3(unsigned(rows)), dim3(256), lds, s, c0, c1, rows0, nkb, opitch);
  else
    hipLaunchKernelGGL(attn_combine_kernel<CT>, dim3(unsigned(rows)), dim3(CT), lds, s, c0, c1, rows0, nkb, opitch);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_values(const void* params_v, int d, int b_v, const float* logits,
                                   const uint32_t* vcodes, const float* vnu, int64_t groups,
                                   int64_t G, int64_t T, float scale, float* out, void* part,
                                   hipStream_t s, int64_t opitch) {
  if (b_v < 2 || b_v > 4) return hipErrorInvalidValue;
  const ValueGroup v = value_group(params_v, d, b_v, vcodes, vnu, groups, G, T, out, part);
  const long nkb = (T + KB - 1) / KB;
  const long blocks = long(groups) * ((G + AH - 1) / AH) * nkb;
  hipError_t e = launch_blocks_one(v, blocks, logits, G, T, scale, s);
  if (e != hipSuccess) return e;
  const long rows = long(groups) * G;
  return launch_combine(v.comb, v.comb, rows, rows, nkb, long(opitch > 0 ? opitch : d), s);
}

namespace {

template <int KBITS, bool PROD>
hipError_t launch_fused_kb(const KeyOps& ko, const ValueGroup& v, long blocks, int64_t G, int64_t T,
                           float scale, hipStream_t s) {
  const long nkb = (T + KB - 1) / KB;
  const long passes = G / AH;
  switch (v.bv) {
    case 1: hipLaunchKernelGGL((attn_fused_kernel<KBITS, PROD, 1>), dim3(unsigned(blocks)), dim3(256), 0, s,
                               ko, v.blk, long(G), long(T), nkb, passes, scale); break;
    case 2: hipLaunchKernelGGL((attn_fused_kernel<KBITS, PROD, 2>), dim3(unsigned(blocks)), dim3(256), 0, s,
                               ko, v.blk, long(G), long(T), nkb, passes, scale); break;
    case 3: hipLaunchKernelGGL((attn_fused_kernel<KBITS, PROD, 3>), dim3(unsigned(blocks)), dim3(256), 0, s,
                               ko, v.blk, long(G), long(T), nkb, passes, scale); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KBITS>
hipError_t launch_fused_k(bool prod, const KeyOps& ko, const ValueGroup& v, long blocks, int64_t G,
                          int64_t T, float scale, hipStream_t s) {
  return prod ? launch_fused_kb<KBITS, true>(ko, v, blocks, G, T, scale, s)
              : launch_fused_kb<KBITS, false>(ko, v, blocks, G, T, scale, s);
}

}  // namespace

hipError_t launch_attention_fused(const void* params_v, int b_k, bool prod, const uint32_t* codes_k,
                                  const float* nu_k, const float* gamma_k, const void* qws, int b_v,
                                  const uint32_t* vcodes, const float* vnu, int64_t groups, int64_t G,
                                  int64_t T, float scale, float* out, void* part, hipStream_t s) {
  constexpr int d = 128;
  if (b_v < 2 || b_v > 4 || G % AH != 0) return hipErrorInvalidValue;
  const ValueGroup v = value_group(params_v, d, b_v, vcodes, vnu, groups, G, T, out, part);
  if (v.nc != 2) return hipErrorInvalidValue;
  const KeyOps ko{codes_k, nu_k, gamma_k, static_cast<const unsigned char*>(qws)};
  const long nkb = (T + KB - 1) / KB;
  const long blocks = long(groups) * (G / AH) * nkb;
  hipError_t e;
  switch (b_k) {
    case 2: e = launch_fused_k<2>(prod, ko, v, blocks, G, T, scale, s); break;
    case 3: e = launch_fused_k<3>(prod, ko, v, blocks, G, T, scale, s); break;
    case 4: e = launch_fused_k<4>(prod, ko, v, blocks, G, T, scale, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const long rows = long(groups) * G;
  return launch_combine(v.comb, v.comb, rows, rows, nkb, long(d), s);
}

hipError_t launch_attention_values_split(const void* params_v0, const void* params_v1, int d0, int d1,
                                         int bv0, int bv1, const float* logits,
                                         const uint32_t* vcodes0, const float* vnu0,
                                         const uint32_t* vcodes1, const float* vnu1, int64_t groups,
                                         int64_t G, int64_t T, float scale, float* out, void* part,
                                         hipStream_t s) {
  if (bv0 < 2 || bv0 > 4 || bv1 < 2 || bv1 > 4) return hipErrorInvalidValue;
  void* part1 = static_cast<unsigned char*>(part) + align256(attention_part_bytes(d0, groups, G, T));
  const ValueGroup v0 = value_group(params_v0, d0, bv0, vcodes0, vnu0, groups, G, T, out, part);
  const ValueGroup v1 = value_group(params_v1, d1, bv1, vcodes1, vnu1, groups, G, T, out + d0, part1);
  const long nkb = (T + KB - 1) / KB;
  const long blocks = long(groups) * ((G + AH - 1) / AH) * nkb;
  hipError_t e;
  if (v0.nc == v1.nc && v0.nc <= 2) {   // both groups' blocks in one grid
    e = v0.nc == 2 ? launch_blocks_nc<2>(v0, &v1, blocks, logits, G, T, scale, s)
                   : launch_blocks_nc<1>(v0, &v1, blocks, logits, G, T, scale, s);
    if (e == hipSuccess) e = hipGetLastError();
  } else {
    e = launch_blocks_one(v0, blocks, logits, G, T, scale, s);
    if (e == hipSuccess) e = launch_blocks_one(v1, blocks, logits, G, T, scale, s);
  }
  if (e != hipSuccess) return e;
  const long rows = long(groups) * G;
  return launch_combine(v0.comb, v1.comb, 2 * rows, rows, nkb, long(d0) + d1, s);
}

namespace {

template <int KB0, int KB1, int BV0, int BV1>
void launch_fused_split_t(const SplitKeyOps& ko, const ValueGroup& v0, const ValueGroup& v1, long blocks,
                          int64_t G, int64_t T, float scale, hipStream_t s) {
  const long nkb = (T + KB - 1) / KB;
  hipLaunchKernelGGL((attn_fused_split_kernel<KB0, KB1, BV0, BV1>), dim3(unsigned(blocks)), dim3(256), 0, s, ko,
                     v0.blk, v1.blk, long(G), long(T), nkb, long(G / AH), scale);
}

// value index planes (BV0, BV1) of the instantiated kernels: equal, or group 0 one above
template <int KB0, int KB1>
hipError_t launch_fused_split_k(const SplitKeyOps& ko, const ValueGroup& v0, const ValueGroup& v1, long blocks,
                                int64_t G, int64_t T, float scale, hipStream_t s) {
  const int p = v0.bv * 4 + v1.bv;
  switch (p) {
    case 1 * 4 + 1: launch_fused_split_t<KB0, KB1, 1, 1>(ko, v0, v1, blocks, G, T, scale, s); break;
    case 2 * 4 + 1: launch_fused_split_t<KB0, KB1, 2, 1>(ko, v0, v1, blocks, G, T, scale, s); break;
    case 2 * 4 + 2: launch_fused_split_t<KB0, KB1, 2, 2>(ko, v0, v1, blocks, G, T, scale, s); break;
    case 3 * 4 + 2: launch_fused_split_t<KB0, KB1, 3, 2>(ko, v0, v1, blocks, G, T, scale, s); break;
    case 3 * 4 + 3: launch_fused_split_t<KB0, KB1, 3, 3>(ko, v0, v1, blocks, G, T, scale, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool attention_fused_split_applies(int bk0, int bk1, int bv0, int bv1) {
  // the instantiated kernels: group 0's bits equal to group 1's or one above, for keys and for
  // values (a fractional rate puts the extra bit in the first group)
  auto pair = [](int a, int b, int lo, int hi) { return b >= lo && a <= hi && (a == b || a == b + 1); };
  return pair(bk0, bk1, 2, 4) && pair(bv0, bv1, 2, 4);
}

hipError_t launch_attention_fused_split(const void* params_v0, const void* params_v1, int bk0, int bk1,
                                        const uint32_t* codes_k0, const float* nu_k0, const float* gamma_k0,
                                        const uint32_t* codes_k1, const float* nu_k1, const float* gamma_k1,
                                        const void* qws, int bv0, int bv1, const uint32_t* vcodes0,
                                        const float* vnu0, const uint32_t* vcodes1, const float* vnu1,
                                        int64_t groups, int64_t G, int64_t T, float scale, float* out, void* part,
                                        hipStream_t s) {
  constexpr int d0 = 64, d1 = 64;
  if (!attention_fused_split_applies(bk0, bk1, bv0, bv1) || G % AH != 0) return hipErrorInvalidValue;
  void* part1 = static_cast<unsigned char*>(part) + align256(attention_part_bytes(d0, groups, G, T));
  const ValueGroup v0 = value_group(params_v0, d0, bv0, vcodes0, vnu0, groups, G, T, out, part);
  const ValueGroup v1 = value_group(params_v1, d1, bv1, vcodes1, vnu1, groups, G, T, out + d0, part1);
  const SplitKeyOps ko{codes_k0, nu_k0, gamma_k0, codes_k1, nu_k1, gamma_k1, static_cast<const unsigned char*>(qws)};
  const long nkb = (T + KB - 1) / KB;
  const long blocks = long(groups) * (G / AH) * nkb;
  hipError_t e;
  switch (bk0 * 8 + bk1) {
    case 2 * 8 + 2: e = launch_fused_split_k<2, 2>(ko, v0, v1, blocks, G, T, scale, s); break;
    case 3 * 8 + 2: e = launch_fused_split_k<3, 2>(ko, v0, v1, blocks, G, T, scale, s); break;
    case 3 * 8 + 3: e = launch_fused_split_k<3, 3>(ko, v0, v1, blocks, G, T, scale, s); break;
    case 4 * 8 + 3: e = launch_fused_split_k<4, 3>(ko, v0, v1, blocks, G, T, scale, s); break;
    case 4 * 8 + 4: e = launch_fused_split_k<4, 4>(ko, v0, v1, blocks, G, T, scale, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const long rows = long(groups) * G;
  return launch_combine(v0.comb, v1.comb, 2 * rows, rows, nkb, long(d0) + d1, s);
}

bool attention_grid_fits(int64_t groups, int64_t G, int64_t T) {
  const int64_t nkb = (T + KB - 1) / KB;
  // a fractional rate's two value groups share the block and combine grids: twice the sizes
  return 2 * groups * G < (int64_t(1) << 31) && 2 * groups * ((G + AH - 1) / AH) * nkb < (int64_t(1) << 31);
}

}  // namespace tq
