// Attention logits over a TurboQuant key cache for the shapes the d = 128 kernel does not
// take: any d that is a multiple of 64, any number G of query heads per group.
//
// Estimate ([review, problem statement]: the query is exact, the key quantized, unbiased;
// [tldr, step 2]):
//   l = nu (<Pi q, chat> + alpha gamma <S q, 2z - 1>),  alpha from the parameter header,
// with <S q, 2z - 1> = 2 sum_{t : z_t = 1} (S q)_t - sum_t (S q)_t, so per coordinate a key
// needs one centroid times (Pi q)_t and one sign-bit-selected (S q)_t for each head.
//
// generic_qprep_kernel: qh = Pi q and sh = S q in float32, a tiled NT product of the query
//   rows with the stacked rows of Pi and S.
// generic_score_kernel: one lane per key and HB heads per pass.  The key's plane words of a
//   32-coordinate group come in with one vector load and are turned into 4-bit fields; per
//   coordinate one LDS read gives the centroid and the sign bit that weights sh.  The query
//   values are the same for every lane of a workgroup: staged in LDS and read as
//   broadcasts; the workgroup also sums the staged sh for the -sum_t (S q)_t term.
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int HB = 4;        // query heads per pass of the scoring kernel
constexpr int KEYS = 256;    // keys per workgroup (one per lane)

constexpr int QR = 16;       // query prep tile: query rows
constexpr int QO = 64;       //                  outputs (rows of the stacked [Pi; S])
constexpr int QK = 64;       //                  K staged per round

// qs[row][o] = <M_o, q_row> for the stacked M = [Pi; S] (o < d: Pi q, o >= d: S q): an
// Query operands of one channel group (qs[row][2][d]: Pi q then S q of each query row).
struct QprepGroup {
  const unsigned char* params;
  size_t off_pi, off_s;
  int d;
  const void* q;          // the group's first query value (row stride qpitch elements)
  float* qs;
  long blocks;            // workgroups of this group: query row tiles x output tiles
};

// Codes and query operands of one channel group for the scoring kernel.
struct ScoreGroup {
  const unsigned char* params;
  const float* qs;        // [groups * G][2][d] from the query prep
  const uint32_t* codes;
  const float* nu;
  const float* gamma;
  int d;
};

// NT product of the query rows with the rows of M, one workgroup per QR x QO tile (64
// outputs never straddle Pi and S since d is a multiple of 64).  Thread t accumulates
// output t % 64 of rows 4 (t / 64) .. +3 over K, both operands staged in LDS with padded
// rows (the M rows are read at a stride of QK + 1 words: conflict-free).
// grid: the blocks of group 0, then those of group 1 (none for a single group)
__global__ __launch_bounds__(256) void generic_qprep_kernel(QprepGroup g0, QprepGroup g1, long qpitch,
                                                            int q_f32, long rows) {
  __shared__ float Qs[QR][QK + 1];
  __shared__ float Ms[QO][QK + 1];
  const bool second = long(blockIdx.x) >= g0.blocks;
  const QprepGroup& gr = second ? g1 : g0;
  const long blk = second ? long(blockIdx.x) - g0.blocks : long(blockIdx.x);
  const unsigned char* params = gr.params;
  const int d = gr.d;
  const void* q = gr.q;
  float* qs = gr.qs;
  const int tid = threadIdx.x;
  const long ntile_o = 2 * d / QO;
  const long r0 = (blk / ntile_o) * QR;
  const int o0 = int(blk % ntile_o) * QO;
  const float* M = o0 < d ? reinterpret_cast<const float*>(params + gr.off_pi) + size_t(o0) * d
                          : reinterpret_cast<const float*>(params + gr.off_s) + size_t(o0 - d) * d;
  const int o = tid & 63, rq = tid >> 6;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  constexpr int NQ = QR * QK / 256, NM = QO * QK / 256;   // staged values per thread
  for (int k0 = 0; k0 < d; k0 += QK) {
    // all of this round's loads are issued before the first LDS store
    float qv[NQ], mv[NM];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int i = tid + 256 * j, r = i / QK, k = i % QK;
      const long row = r0 + r;
      const size_t at = size_t(row < rows ? row : rows - 1) * qpitch + k0 + k;
      const float v = q_f32 ? static_cast<const float*>(q)[at]
                            : __uint_as_float(uint32_t(static_cast<const uint16_t*>(q)[at]) << 16);
      qv[j] = row < rows ? v : 0.f;
    }
#pragma unroll
    for (int j = 0; j < NM; ++j) {
      const int i = tid + 256 * j;
      mv[j] = M[size_t(i / QK) * d + k0 + i % QK];
    }
    __syncthreads();                       // the previous round's tiles are no longer read
#pragma unroll
    for (int j = 0; j < NQ; ++j) Qs[(tid + 256 * j) / QK][(tid + 256 * j) % QK] = qv[j];
#pragma unroll
    for (int j = 0; j < NM; ++j) Ms[(tid + 256 * j) / QK][(tid + 256 * j) % QK] = mv[j];
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < QK; ++k) {
      const float m = Ms[o][k];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fmaf(m, Qs[4 * rq + j][k], acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const long row = r0 + 4 * rq + j;
    if (row < rows) qs[size_t(row) * 2 * d + o0 + o] = acc[j];
  }
}

// Bits 0..7 of x to bits 0, 4, .., 28.
__device__ __forceinline__ uint32_t spread_nibbles(uint32_t x) {
  x &= 0xffu;
  x = (x | (x << 12)) & 0x000f000fu;
  x = (x | (x << 6)) & 0x03030303u;
  return (x | (x << 3)) & 0x11111111u;
}

// One channel group's part of the estimate for this thread's key and the pass's heads:
// l[hh] += n_k (<Pi q, chat> + alpha gamma_k <S q, 2z - 1>).  The pass's query values (HB
// heads of Pi q and S q) are staged in LDS, CH coordinates at a time, as one float4 per
// coordinate and matrix: every lane reads the same address, a broadcast.  A key's plane
// words of a 32-coordinate group are turned into 4-bit fields (index bits, QJL sign in bit
// 3), so that per coordinate one bit-field op and one LDS read of (centroid, sign) from a
// 16-entry table decode it.  Every thread of the workgroup calls it (it synchronizes).
template <int BITS, bool PROD>
__device__ __forceinline__ void add_group_estimate(
    const unsigned char* __restrict__ params, const float* __restrict__ qs,
    const uint32_t* __restrict__ codes, const float* __restrict__ nu,
    const float* __restrict__ gamma, int d, long G, long T, long g, long h0, long nh, long t,
    bool valid, float4 (*qsh)[KEYS], float4* red, float2* tab, float* l) {
  static_assert(HB == 4, "one float4 of query values per coordinate");
  constexpr int L = 1 << (BITS - 1);
  constexpr int CH = KEYS;                 // coordinates staged per round (one per thread)
  const Header* hdr = reinterpret_cast<const Header*>(params);
  const float alpha = hdr->alpha;
  const int tid = threadIdx.x;
  __syncthreads();                         // a previous group's table and sums are read
  if (tid < 16) tab[tid] = make_float2(hdr->cen[(tid & 7) < L ? (tid & 7) : L - 1], float(tid >> 3));

  const long key = g * T + (valid ? t : T - 1);  // ragged block: read a valid key, store nothing
  const int words = d / 32;
  const uint32_t* kc = codes + size_t(key) * words * BITS;
  // query rows of the pass; heads past G repeat the last one (results not stored)
  const float* qrow[HB];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    const long h = h0 + (hh < nh ? hh : nh - 1);
    qrow[hh] = qs + size_t(g * G + h) * 2 * d;
  }
  // a word's BITS planes (one vector load where the size allows)
  auto load_word = [&](int wi, uint32_t* pl) {
    const uint32_t* src = kc + size_t(wi) * BITS;
    if constexpr (BITS == 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(src);
      pl[0] = v.x; pl[1] = v.y; pl[2] = v.z; pl[3] = v.w;
    } else if constexpr (BITS == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(src);
      pl[0] = v.x; pl[1] = v.y; pl[2] = 0u; pl[3] = 0u;
    } else {
      pl[0] = src[0]; pl[1] = src[1]; pl[2] = src[2]; pl[3] = 0u;
    }
  };
  // loads in flight before the first barrier: the key's nu and gamma and the first word;
  // later words are loaded one word ahead
  const float n_k = nu[key], g_k = gamma[key];
  uint32_t cur[4];
  load_word(0, cur);
  float4 mse = make_float4(0.f, 0.f, 0.f, 0.f), zs = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 spart = make_float4(0.f, 0.f, 0.f, 0.f);   // this thread's staged S q values, summed
  for (int c0 = 0; c0 < d; c0 += CH) {
    const int cn = d - c0 < CH ? d - c0 : CH;
    __syncthreads();                       // the previous round's values are no longer read
    if (tid < cn) {
      const int c = c0 + tid;
      qsh[0][tid] = make_float4(qrow[0][c], qrow[1][c], qrow[2][c], qrow[3][c]);
      if constexpr (PROD) {
        const float4 sv = make_float4(qrow[0][d + c], qrow[1][d + c], qrow[2][d + c], qrow[3][d + c]);
        qsh[1][tid] = sv;
        spart.x += sv.x;
        spart.y += sv.y;
        spart.z += sv.z;
        spart.w += sv.w;
      }
    }
    __syncthreads();
    for (int w = 0; w < cn / 32; ++w) {
      const int wi = c0 / 32 + w;
      uint32_t pl[4] = {cur[0], cur[1], cur[2], cur[3]};
      if (wi + 1 < words) load_word(wi + 1, cur);
      // fields: index bits 0 .. BITS-2, the QJL sign in bit 3 (coordinate 8 q + i in bits
      // 4 i .. of nib[q])
      uint32_t nib[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t v = spread_nibbles(pl[0] >> (8 * q));
        if constexpr (BITS > 2) v |= spread_nibbles(pl[1] >> (8 * q)) << 1;
        if constexpr (BITS > 3) v |= spread_nibbles(pl[2] >> (8 * q)) << 2;
        if constexpr (PROD) v |= spread_nibbles(pl[BITS - 1] >> (8 * q)) << 3;
        nib[q] = v;
      }
#pragma unroll 8
      for (int e = 0; e < 32; ++e) {
        const float2 cz = tab[(nib[e >> 3] >> (4 * (e & 7))) & 0xfu];
        const float4 a = qsh[0][32 * w + e];
        mse.x = fmaf(a.x, cz.x, mse.x);
        mse.y = fmaf(a.y, cz.x, mse.y);
        mse.z = fmaf(a.z, cz.x, mse.z);
        mse.w = fmaf(a.w, cz.x, mse.w);
        if constexpr (PROD) {
          const float4 b = qsh[1][32 * w + e];
          zs.x = fmaf(b.x, cz.y, zs.x);
          zs.y = fmaf(b.y, cz.y, zs.y);
          zs.z = fmaf(b.z, cz.y, zs.z);
          zs.w = fmaf(b.w, cz.y, zs.w);
        }
      }
    }
  }
  float s4[HB] = {0.f, 0.f, 0.f, 0.f};    // sum_t (S q)_t of the 4 heads (same order everywhere)
  if constexpr (PROD) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      spart.x += __shfl_xor(spart.x, off);
      spart.y += __shfl_xor(spart.y, off);
      spart.z += __shfl_xor(spart.z, off);
      spart.w += __shfl_xor(spart.w, off);
    }
    if ((tid & 63) == 0) red[tid >> 6] = spart;
    __syncthreads();
    const float4 a = red[0], b = red[1], c = red[2], e = red[3];
    s4[0] = (a.x + b.x) + (c.x + e.x);
    s4[1] = (a.y + b.y) + (c.y + e.y);
    s4[2] = (a.z + b.z) + (c.z + e.z);
    s4[3] = (a.w + b.w) + (c.w + e.w);
  }
  const float m4[HB] = {mse.x, mse.y, mse.z, mse.w};
  const float z4[HB] = {zs.x, zs.y, zs.z, zs.w};
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    float v = m4[hh];
    if constexpr (PROD) v = fmaf(alpha * g_k, 2.f * z4[hh] - s4[hh], v);
    l[hh] += n_k * v;
  }
}

// grid: one workgroup per (group, head pass, block of KEYS keys), flattened into x.  B1 > 0:
// a fractional rate's second channel group (its own parameters, codes and query operands),
// whose estimate is added to the first one's in registers before the single store.
template <int B0, int B1, bool PROD>
__global__ __launch_bounds__(KEYS) void generic_score_kernel(ScoreGroup s0, ScoreGroup s1, long G, long T,
                                                             long kblocks, long passes,
                                                             float* __restrict__ logits) {
  __shared__ float4 qsh[2][KEYS];          // [0]: Pi q, [1]: S q of the pass's 4 heads
  __shared__ float4 red[KEYS / 64];        // sum_t (S q)_t: per-wave partial sums
  __shared__ float2 tab[16];               // field -> (centroid, QJL sign bit as 0 / 1)
  const long blk = blockIdx.x;
  const long kb = blk % kblocks;
  const long gp = blk / kblocks;           // group * passes + pass
  const long g = gp / passes;
  const long h0 = (gp % passes) * HB;
  const long nh = G - h0 < HB ? G - h0 : HB;   // heads of this pass
  const long t = kb * KEYS + threadIdx.x;
  const bool valid = t < T;
  float l[HB] = {0.f, 0.f, 0.f, 0.f};
  add_group_estimate<B0, PROD>(s0.params, s0.qs, s0.codes, s0.nu, s0.gamma, s0.d, G, T, g, h0, nh,
                               t, valid, qsh, red, tab, l);
  if constexpr (B1 > 0)
    add_group_estimate<B1, PROD>(s1.params, s1.qs, s1.codes, s1.nu, s1.gamma, s1.d, G, T, g, h0,
                                 nh, t, valid, qsh, red, tab, l);
  if (!valid) return;
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    if (hh >= nh) break;
    logits[size_t(g * G + h0 + hh) * T + t] = l[hh];
  }
}

// Query prep of one or two channel groups in one launch, then the scoring kernel.
template <int B0, int B1>
hipError_t launch_b(const void* params0, int d0, const void* params1, int d1, const void* q,
                    int q_dtype, long qpitch, const uint32_t* codes0, const float* nu0,
                    const float* gamma0, const uint32_t* codes1, const float* nu1,
                    const float* gamma1, int64_t groups, int64_t G, int64_t T, int mode,
                    float* logits, void* ws, hipStream_t s, int phases) {
  const long rows = long(groups) * G;
  const size_t esz = q_dtype == 0 ? 4 : 2;
  const Layout lay0(d0, B0);
  float* qs0 = static_cast<float*>(ws);
  QprepGroup g0{static_cast<const unsigned char*>(params0), lay0.off_pi, lay0.off_s, d0, q, qs0,
                (rows + QR - 1) / QR * (2 * d0 / QO)};
  QprepGroup g1{};
  ScoreGroup s1{};
  if constexpr (B1 > 0) {
    const Layout lay1(d1, B1);
    float* qs1 = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) +
                                          align256(score_generic_ws_bytes(d0, groups, G)));
    g1 = QprepGroup{static_cast<const unsigned char*>(params1), lay1.off_pi, lay1.off_s, d1,
                    q ? static_cast<const unsigned char*>(q) + size_t(d0) * esz : nullptr, qs1,
                    (rows + QR - 1) / QR * (2 * d1 / QO)};
    s1 = ScoreGroup{g1.params, qs1, codes1, nu1, gamma1, d1};
  }
  if (phases & kScorePrep) {
    hipLaunchKernelGGL(generic_qprep_kernel, dim3(unsigned(g0.blocks + g1.blocks)), dim3(256), 0, s, g0,
                       g1, qpitch, q_dtype == 0 ? 1 : 0, rows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(phases & kScoreScan)) return hipSuccess;
  const ScoreGroup s0{g0.params, qs0, codes0, nu0, gamma0, d0};
  const long kblocks = (T + KEYS - 1) / KEYS;
  const long passes = (G + HB - 1) / HB;
  const dim3 grid(unsigned(groups * passes * kblocks));
  if (mode == 0)
    hipLaunchKernelGGL((generic_score_kernel<B0, B1, true>), grid, dim3(KEYS), 0, s, s0, s1, long(G),
                       long(T), kblocks, passes, logits);
  else
    hipLaunchKernelGGL((generic_score_kernel<B0, B1, false>), grid, dim3(KEYS), 0, s, s0, s1, long(G),
                       long(T), kblocks, passes, logits);
  return hipGetLastError();
}

template <int B0>
hipError_t launch_b1(int b1, const void* params0, int d0, const void* params1, int d1, const void* q,
                     int q_dtype, long qpitch, const uint32_t* codes0, const float* nu0,
                     const float* gamma0, const uint32_t* codes1, const float* nu1,
                     const float* gamma1, int64_t groups, int64_t G, int64_t T, int mode,
                     float* logits, void* ws, hipStream_t s, int phases) {
  switch (b1) {
#define TQ_GEN_CASE(B1)                                                                           \
  case B1:                                                                                        \
    return launch_b<B0, B1>(params0, d0, params1, d1, q, q_dtype, qpitch, codes0, nu0, gamma0,    \
                            codes1, nu1, gamma1, groups, G, T, mode, logits, ws, s, phases);
    TQ_GEN_CASE(0)
    TQ_GEN_CASE(2)
    TQ_GEN_CASE(3)
    TQ_GEN_CASE(4)
#undef TQ_GEN_CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_groups(const void* params0, int d0, int b0, const void* params1, int d1, int b1,
                         const void* q, int q_dtype, long qpitch, const uint32_t* codes0,
                         const float* nu0, const float* gamma0, const uint32_t* codes1,
                         const float* nu1, const float* gamma1, int64_t groups, int64_t G,
                         int64_t T, int mode, float* logits, void* ws, hipStream_t s, int phases) {
  switch (b0) {
    case 2: return launch_b1<2>(b1, params0, d0, params1, d1, q, q_dtype, qpitch, codes0, nu0, gamma0,
                                codes1, nu1, gamma1, groups, G, T, mode, logits, ws, s, phases);
    case 3: return launch_b1<3>(b1, params0, d0, params1, d1, q, q_dtype, qpitch, codes0, nu0, gamma0,
                                codes1, nu1, gamma1, groups, G, T, mode, logits, ws, s, phases);
    case 4: return launch_b1<4>(b1, params0, d0, params1, d1, q, q_dtype, qpitch, codes0, nu0, gamma0,
                                codes1, nu1, gamma1, groups, G, T, mode, logits, ws, s, phases);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t score_generic_ws_bytes(int d, int64_t groups, int64_t G) {
  return size_t(groups) * G * 2 * size_t(d) * 4;
}

size_t score_generic_split_ws_bytes(int d0, int d1, int64_t groups, int64_t G) {
  return align256(score_generic_ws_bytes(d0, groups, G)) + score_generic_ws_bytes(d1, groups, G);
}

bool score_generic_grid_fits(int64_t groups, int64_t G, int64_t T) {
  const int64_t blocks = groups * ((G + HB - 1) / HB) * ((T + KEYS - 1) / KEYS);
  // query prep of one or two channel groups, at most 4096 coordinates in all
  const int64_t qblocks = (groups * G + QR - 1) / QR * (2 * 4096 / QO);
  return groups * G < (int64_t(1) << 31) && blocks < (int64_t(1) << 31) && qblocks < (int64_t(1) << 31);
}

hipError_t launch_score_generic(const void* params, int d, int b, const void* q, int q_dtype,
                                const uint32_t* codes, const float* nu, const float* gamma,
                                int64_t groups, int64_t G, int64_t T, int mode, float* logits,
                                void* ws, hipStream_t s, int64_t qpitch, int phases) {
  const long qp = qpitch > 0 ? long(qpitch) : long(d);
  return launch_groups(params, d, b, nullptr, 0, 0, q, q_dtype, qp, codes, nu, gamma, nullptr, nullptr,
                       nullptr, groups, G, T, mode, logits, ws, s, phases);
}

hipError_t launch_score_generic_split(const void* params0, const void* params1, int d0, int d1, int b0,
                                      int b1, const void* q, int q_dtype, const uint32_t* codes0,
                                      const float* nu0, const float* gamma0, const uint32_t* codes1,
                                      const float* nu1, const float* gamma1, int64_t groups, int64_t G,
                                      int64_t T, int mode, float* logits, void* ws, hipStream_t s,
                                      int phases) {
  if (b1 < 2) return hipErrorInvalidValue;
  return launch_groups(params0, d0, b0, params1, d1, b1, q, q_dtype, long(d0) + d1, codes0, nu0,
                       gamma0, codes1, nu1, gamma1, groups, G, T, mode, logits, ws, s, phases);
}

}  // namespace tq
