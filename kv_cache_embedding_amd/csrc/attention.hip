// One decode step of attention over a TurboQuant KV cache: keys carry the inner-product
// quantizer, values the MSE quantizer alone ([review, problem statement]: the two
// quantizers; [news, KV-cache paragraph]: KV caches compressed to about 3 bits):
//   o[g][h] = sum_t softmax_t(scale * l[g][h][t]) * nu_t Pi_v^T chat_t,
// with l the unbiased logit estimate of the keys (the scoring kernels write it).  Pi_v^T is
// linear, so the weighted sum runs in the values' rotated coordinates and one inverse
// rotation per head finishes it:  o = Pi_v^T a,  a = sum_t p_t nu_t chat_t / sum_t p_t.
//
// attn_block_kernel: one workgroup per (group, pass of AH heads, block of KB keys).  Lanes
//   first hold one key each: scaled logits, the block maximum per head, the weights
//   p = exp(l - max) and p nu, which go to LDS as one float4 per key.  Then each wave walks
//   its 64 keys with the lanes over the coordinates (64 per step): the wave's keys are first
//   staged in LDS, lane j turning key j's plane words of each 32-coordinate group into one
//   16-byte slot of 4-bit indices (coordinate 8 q + i in bits 4 i .. of dword q), so that
//   per key a lane reads the weights (a broadcast) and its coordinate's dword, extracts the
//   index with one bit-field op, looks the centroid up in LDS and accumulates it times the
//   key's weight for every head.  Out: per block and head the maximum, the sum of p and the
//   weighted sum of centroids.
// attn_combine_kernel: one workgroup per (group, head): merges the blocks (log-sum-exp) and
//   applies Pi_v^T; threads split both sums into slices of independent float4 loads (rows
//   of Pi_v are contiguous, so a slice reads coalesced columns), the first loads of both
//   issued before the maximum and the sum are reduced.
#include "tq_internal.h"

#include <algorithm>
#include <cmath>

namespace tq {
namespace {

constexpr int AH = 4;      // query heads per pass
constexpr int KB = 256;    // keys per workgroup (64 per wave)
constexpr int CT = 1024;   // threads of a combine workgroup (one per (group, head))

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Bits 0..7 of x to bits 0, 4, .., 28.
__device__ __forceinline__ uint32_t spread_nibbles(uint32_t x) {
  x &= 0xffu;
  x = (x | (x << 12)) & 0x000f000fu;
  x = (x | (x << 6)) & 0x03030303u;
  return (x | (x << 3)) & 0x11111111u;
}

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

// One workgroup's block (256 keys) of one value channel group.  BV: index planes of a value
// (1..3); NC: 64-coordinate steps per chunk (NC divides d / 64).  The LDS arrays come from
// the kernel, sized for the largest codebook.
template <int BV, int NC>
__device__ __forceinline__ void value_block(const BlockGroup& bg, const float* __restrict__ logits,
                                            long G, long T, long nkb, long passes, float scale,
                                            long blk, float* cen, float (*red)[AH],
                                            float (*accs)[AH][64 * NC], uint4 (*kw)[64][2 * NC],
                                            float4 (*wsh)[64]) {
  static_assert(BV >= 1 && BV <= 3, "a value's index fits one 4-bit field");
  constexpr int L = 1 << BV;
  const unsigned char* __restrict__ params_v = bg.params_v;
  const uint32_t* __restrict__ vcodes = bg.vcodes;
  const float* __restrict__ vnu = bg.vnu;
  const int d = bg.d;
  float* __restrict__ part_m = bg.part_m;
  float* __restrict__ part_s = bg.part_s;
  float* __restrict__ part_acc = bg.part_acc;
  const Header* hdr = reinterpret_cast<const Header*>(params_v);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar code loads
  if (tid < L) cen[tid] = hdr->cen[tid];

  const long kb = blk % nkb;
  const long gp = blk / nkb;
  const long g = gp / passes;
  const long h0 = (gp % passes) * AH;
  const long nh = G - h0 < AH ? G - h0 : AH;   // heads of this pass
  const long tw0 = kb * KB + wave * 64;        // first key of this wave
  const long t = tw0 + lane;                   // the lane's key in the prologue
  const bool valid = t < T;

  // prologue: scaled logits of the lane's key, block maximum per head
  float l[AH];
#pragma unroll
  for (int hh = 0; hh < AH; ++hh) {
    const long h = h0 + (hh < nh ? hh : nh - 1);
    l[hh] = valid ? scale * logits[size_t(g * G + h) * T + t] : -INFINITY;
    const float m = wave_max(l[hh]);
    if (lane == 0) red[wave][hh] = m;
  }
  __syncthreads();   // also publishes cen
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
    const float sp = wave_sum(p);
    if (lane == 0) red[wave][hh] = sp;
  }
  wsh[wave][lane] = make_float4(w[0], w[1], w[2], w[3]);
  __syncthreads();
  const long prow = g * G + h0;                 // partial rows of this pass: prow + hh
#pragma unroll
  for (int hh = 0; hh < AH; ++hh) {
    if (tid == hh && hh < nh) {
      part_m[(prow + hh) * nkb + kb] = M[hh];
      part_s[(prow + hh) * nkb + kb] = (red[0][hh] + red[1][hh]) + (red[2][hh] + red[3][hh]);
    }
  }

  // weighted sum of the centroids of the wave's keys, 64 NC coordinates per chunk
  const int W = d / 32;
  const long nk = T - tw0 < 64 ? (T - tw0 > 0 ? T - tw0 : 0) : 64;
  for (int c0 = 0; c0 < d; c0 += 64 * NC) {
    // the chunk's plane words of the wave's keys: lane j loads those of key j (one pass of
    // contiguous loads instead of a dependent scalar load per key)
    if (lane < nk) {
      const uint32_t* kc = vcodes + (size_t(g * T + tw0 + lane) * W + c0 / 32) * BV;
#pragma unroll
      for (int e = 0; e < 2 * NC; ++e) {
        const uint32_t p0 = kc[e * BV], p1 = BV > 1 ? kc[e * BV + 1] : 0u, p2 = BV > 2 ? kc[e * BV + 2] : 0u;
        uint32_t nib[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          nib[q] = spread_nibbles(p0 >> (8 * q)) | (spread_nibbles(p1 >> (8 * q)) << 1) |
                   (spread_nibbles(p2 >> (8 * q)) << 2);
        kw[wave][lane][e] = make_uint4(nib[0], nib[1], nib[2], nib[3]);
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    float acc[AH][NC];
#pragma unroll
    for (int hh = 0; hh < AH; ++hh)
#pragma unroll
      for (int i = 0; i < NC; ++i) acc[hh][i] = 0.f;
    // this lane's coordinate within a 32-coordinate group: dword q of the slot, field i
    const int q = (lane & 31) >> 3, fsh = 4 * (lane & 7);
    const uint32_t* kwd = reinterpret_cast<const uint32_t*>(&kw[wave][0][0]) + q;
#pragma unroll 4
    for (int j = 0; j < nk; ++j) {
      const float4 wj = wsh[wave][j];
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const uint32_t dw = kwd[(j * 2 * NC + 2 * i + (lane >> 5)) * 4];
        const float c = cen[(dw >> fsh) & 0xfu];
        acc[0][i] = fmaf(wj.x, c, acc[0][i]);
        acc[1][i] = fmaf(wj.y, c, acc[1][i]);
        acc[2][i] = fmaf(wj.z, c, acc[2][i]);
        acc[3][i] = fmaf(wj.w, c, acc[3][i]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < AH; ++hh)
#pragma unroll
      for (int i = 0; i < NC; ++i) accs[wave][hh][64 * i + lane] = acc[hh][i];
    __syncthreads();
    for (int e = tid; e < AH * 64 * NC; e += 256) {
      const int hh = e / (64 * NC), c = e % (64 * NC);
      if (hh < nh)
        part_acc[((prow + hh) * nkb + kb) * d + c0 + c] =
            (accs[0][hh][c] + accs[1][hh][c]) + (accs[2][hh][c] + accs[3][hh][c]);
    }
    __syncthreads();
  }
}


// grid: the blocks of value channel group 0, then those of group 1 (BV1 > 0: a fractional
// rate's second value group with the same chunk shape).
template <int BV0, int BV1, int NC>
__global__ __launch_bounds__(256) void attn_block_kernel(BlockGroup b0, BlockGroup b1, long blocks0,
                                                         const float* __restrict__ logits, long G,
                                                         long T, long nkb, long passes, float scale) {
  __shared__ float cen[8];
  __shared__ float red[4][AH];
  __shared__ float accs[4][AH][64 * NC];
  __shared__ uint4 kw[4][64][2 * NC];   // a chunk's 4-bit indices: [wave][key][32-coordinate group]
  __shared__ float4 wsh[4][64];         // p nu of the wave's keys for the 4 heads
  const long blk = blockIdx.x;
  if constexpr (BV1 > 0) {
    if (blk >= blocks0) {
      value_block<BV1, NC>(b1, logits, G, T, nkb, passes, scale, blk - blocks0, cen, red, accs, kw, wsh);
      return;
    }
  }
  value_block<BV0, NC>(b0, logits, G, T, nkb, passes, scale, blk, cen, red, accs, kw, wsh);
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
// group of wider output rows: its columns only).
__global__ __launch_bounds__(CT) void attn_combine_kernel(CombineGroup c0, CombineGroup c1, long rows0,
                                                          long nkb, long opitch) {
  constexpr int NW = CT / 64;
  constexpr int PF = 8;              // loads of each sum issued before the reductions
  extern __shared__ float4 lds4[];   // [slices][d / 4] partial sums, then a[d / 4]
  __shared__ float red[NW];
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
  // inverse rotation, every nsl-th row of Pi_v); d / 4 <= CT, so a thread owns one column
  const int d4 = d / 4;
  const int cols = d4 < CT ? d4 : CT;
  const int nsl = CT / cols;
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

  float mx = -INFINITY;
  for (long k = tid; k < nkb; k += CT) mx = fmaxf(mx, pm[k]);
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) M = fmaxf(M, red[i]);
  __syncthreads();
  float sum = 0.f;
  for (long k = tid; k < nkb; k += CT) sum += __expf(pm[k] - M) * ps[k];
  sum = wave_sum(sum);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) tot += red[i];
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
  for (int c4 = tid; c4 < d4; c4 += CT) {
    float4 v = part[c4];
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
  for (int j4 = tid; j4 < d4; j4 += CT) {
    float4 v = part[j4];
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

size_t combine_lds_bytes(int d) {
  const int d4 = d / 4, cols = d4 < CT ? d4 : CT, nsl = CT / cols;
  return (size_t(nsl) * d4 + d4) * 16;
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
  hipLaunchKernelGGL(attn_combine_kernel, dim3(unsigned(rows)), dim3(CT), combine_lds_bytes(d), s, v.comb,
                     v.comb, rows, nkb, long(opitch > 0 ? opitch : d));
  return hipGetLastError();
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
  hipLaunchKernelGGL(attn_combine_kernel, dim3(unsigned(2 * rows)), dim3(CT),
                     std::max(combine_lds_bytes(d0), combine_lds_bytes(d1)), s, v0.comb, v1.comb, rows,
                     nkb, long(d0) + d1);
  return hipGetLastError();
}

bool attention_grid_fits(int64_t groups, int64_t G, int64_t T) {
  const int64_t nkb = (T + KB - 1) / KB;
  // a fractional rate's two value groups share the block and combine grids: twice the sizes
  return 2 * groups * G < (int64_t(1) << 31) && 2 * groups * ((G + AH - 1) / AH) * nkb < (int64_t(1) << 31);
}

}  // namespace tq
