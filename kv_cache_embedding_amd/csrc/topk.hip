// Flat-scan top-k search over TurboQuant codes ([news, vector-search paragraph]: the index
// is the codes themselves, so there is nothing to build).
//
// Score of query a against key j ([review, problem statement]; [explainer, step 2]):
//   l_aj = |q_a| nu_j ( <Pi q_a, chat_j> + alpha gamma_j <S q_a, 2 z_j - 1> ) / |q_a|
//        = |q_a| nu_j < [Pi q_a | S q_a / sqrt(d)] / |q_a| , [chat_j | alpha sqrt(d) gamma_j (2 z_j - 1)] >,
// a dense contraction over K = 2d between a query operand Q~ (fp16, prepared once per call)
// and a key operand that is decoded from the packed bit planes inside the scan kernel: the
// codes are the only per-key bytes read from HBM (b d / 8 + 8 per key).
//
// Kernels:
//   topk_qprep_kernel   Pi q and S q on v_mfma_f32_32x32x2f32 (float32 operands, exact
//                       products), scaled and written in fp16 MFMA fragment order;
//   topk_scan_kernel    one workgroup per (32 RT-query tile, key range): 4 waves, one per
//                       SIMD, each scores 32 RT queries x 32 KT keys per 128 KT-key block on
//                       v_mfma_f32_32x32x16_f16 (RT x KT tiles, every query fragment feeds
//                       KT MFMAs) with its key operand built in registers (byte-permute
//                       lookup of the codebook magnitude + sign-bit insert), then filters
//                       the block's scores against each query's running k-th best and
//                       merges the survivors into per-query lists in LDS;
//   topk_merge_kernel   merges the lists of all key ranges of a query.
// Order: decreasing score, equal scores by increasing key index.
#include "tq_internal.h"

#include <cfloat>
#include <cmath>

namespace tq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const void* gptr;   // global
typedef __attribute__((address_space(3))) void* lptr;         // LDS

// Tile shape: every wave holds RT x KT = 16 accumulator tiles of 32 x 32 (all 256 AGPRs).
// Each query fragment read from LDS feeds KT MFMAs and each decoded key operand feeds RT,
// so RT trades the query-operand traffic (DMA + LDS reads per MFMA, ~1/KT) against the key
// decode (VALU per MFMA, ~1/RT); on gfx950 about four independent VALU ops issue in the
// shadow of one 32x32x16 MFMA, further VALU work adds to the time.
#ifndef TQ_TOPK_RT
#define TQ_TOPK_RT 8
#endif
constexpr int RT = TQ_TOPK_RT;                // MFMA row tiles (32 queries each) per query tile
constexpr int KT = 16 / RT;                   // MFMA key tiles (32 keys each) per wave
constexpr int NW = (KT + 1) / 2;              // pending-bit words per row tile (16 bits per key tile)
constexpr int QROWS = 32 * RT;                // queries per tile
constexpr int KEYS = 4 * 32 * KT;             // keys per block (4 waves)
constexpr int KMAX = 32;                      // largest k held in the per-query lists
// candidate slots per query for lists of KM entries (LDS of a workgroup stays <= 160 KiB)
constexpr int cand_slots(int km) { return RT >= 8 ? (km <= 16 ? 24 : 8) : 32; }
constexpr int STEP_HALVES = RT * 4 * 64 * 8;  // query operand of one 32-coordinate group (16 KiB)
#ifndef TQ_TOPK_PF
#define TQ_TOPK_PF 3
#endif
constexpr int PF = TQ_TOPK_PF;                // A fragments in flight ahead of the MFMAs

// The fp16 scan keeps kk >= k + KMARGIN candidates per query; their float32 estimates decide
// the final k.  Larger k take the float32 score-and-select path.
constexpr int KMARGIN = 6;
constexpr int KFUSED = KMAX - KMARGIN;        // largest k of the fused path
constexpr int list_len(int k) { return k + KMARGIN <= 16 ? 16 : KMAX; }

struct Plan {
  long nq, n, qt, nb, rb, nsplit;
  int kk;
  size_t off_q, off_qn, off_qx, off_cand, off_top, off_ovf, total;
};

Plan plan(int d, int64_t nq, int64_t n, int k) {
  Plan p;
  p.kk = list_len(k);
  p.nq = nq;
  p.n = n;
  p.qt = (nq + QROWS - 1) / QROWS;
  p.nb = (n + KEYS - 1) / KEYS;
  // one workgroup per CU over the whole scan: each key range as long as the CUs allow (a
  // range's candidate rate falls as its thresholds rise, so fewer, longer ranges queue fewer
  // candidates; a second round of workgroups cost 6% at 10^6 keys)
  long want = device_cu_count() / (p.qt > 0 ? p.qt : 1);
  if (want < 1) want = 1;
  p.rb = (p.nb + want - 1) / want;
  if (p.rb < 1) p.rb = 1;
  p.nsplit = (p.nb + p.rb - 1) / p.rb;
  p.off_q = 0;
  p.off_qn = align256(size_t(p.qt) * (d / 32) * STEP_HALVES * 2);
  p.off_qx = p.off_qn + align256(size_t(p.qt) * QROWS * 4);
  p.off_cand = p.off_qx + align256(size_t(nq) * 2 * d * 4);
  p.off_top = p.off_cand + align256(size_t(nq) * p.nsplit * p.kk * 8);
  p.off_ovf = p.off_top + align256(size_t(nq) * p.kk * 8);
  p.total = p.off_ovf + align256(size_t(p.qt) * p.nsplit * QROWS * KEYS * 8);
  return p;
}

// Position of (query a, coordinate t, half) in the fragment-ordered query operand.  Within a
// 32-coordinate group, MFMA K position 16 s + 8 h + 2 i + e (s: K16 substep, h: lane half,
// i: dword, e: half of the dword) holds coordinate 8 s + 4 h + i + 16 e, so that the two
// halves of one B dword come from bits p and p + 16 of a packed plane word.
__device__ __forceinline__ size_t qfrag_offset(long a, int t, int sign, int G) {
  const int w = t >> 5, c = t & 31;
  const int e = c >> 4, p = c & 15;
  const int sub = p >> 3, hh = (p >> 2) & 1, ii = p & 3;
  const long qt = a / QROWS;
  const int ar = int(a % QROWS);
  const int i = ar >> 5, lrow = ar & 31;
  const int s = sub + 2 * sign;
  const int lane = lrow + 32 * hh;
  return ((((size_t(qt) * G + w) * RT + i) * 4 + s) * 64 + lane) * 8 + 2 * ii + e;
}

// ------------------------------------------------------------------ query operands
// One wave per (32 queries, 32 output rows of [Pi ; S]).  Lane (row r, half h) reads 4
// consecutive float32 of its query and of its matrix row; MFMA j of a K8 step pairs
// coordinates k0 + j (h = 0) and k0 + 4 + j (h = 1), so every coordinate is summed once.
__global__ __launch_bounds__(256) void topk_qprep_kernel(const unsigned char* __restrict__ params,
                                                          size_t off_pi, size_t off_s, int d,
                                                          const void* __restrict__ q, int q_f32,
                                                          long nq, long rows_pad,
                                                          _Float16* __restrict__ qf,
                                                          float* __restrict__ qn,
                                                          float* __restrict__ qx) {
  const int lane = threadIdx.x & 63, h = lane >> 5, nl = lane & 31;
  const long wid = long(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const long rho_tiles = 2 * d / 32;
  const long a0 = (wid / rho_tiles) * 32;
  const int rho0 = int(wid % rho_tiles) * 32;
  if (a0 >= rows_pad) return;
  const long a = a0 + nl;
  const bool aok = a < nq;
  const int rho = rho0 + nl;
  const float* m = reinterpret_cast<const float*>(params + (rho < d ? off_pi : off_s)) +
                   size_t(rho % d) * d;
  f32x16 acc = f32x16{};
  float ssq = 0.f;
  for (int k0 = 0; k0 < d; k0 += 8) {
    float4 qv = make_float4(0.f, 0.f, 0.f, 0.f);
    if (aok) {
      const size_t off = size_t(a) * d + k0 + 4 * h;
      if (q_f32) {
        qv = *reinterpret_cast<const float4*>(static_cast<const float*>(q) + off);
      } else {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(q) + off);
        qv = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                         __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
      }
    }
    const float4 mv = *reinterpret_cast<const float4*>(m + k0 + 4 * h);
    ssq = fmaf(qv.x, qv.x, fmaf(qv.y, qv.y, fmaf(qv.z, qv.z, fmaf(qv.w, qv.w, ssq))));
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv.x, mv.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv.y, mv.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv.z, mv.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv.w, mv.w, acc, 0, 0, 0);
  }
  // |q| of row nl: both lane halves hold half of the coordinates
  ssq += __shfl_xor(ssq, 32);
  const float norm = sqrtf(ssq);
  if (rho0 == 0 && h == 0 && a < rows_pad) qn[a] = aok ? norm : 0.f;
  const float rsd = 1.0f / sqrtf(float(d));
  // accumulator register r of lane l: query row 8 (r / 4) + 4 h + r % 4, output row nl
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 8 * (r >> 2) + 4 * h + (r & 3);
    const float nr = __shfl(norm, row);
    const long ar = a0 + row;
    float v = 0.f;
    if (ar < nq && nr > 0.f) v = acc[r] / nr * (rho < d ? 1.0f : rsd);
    qf[qfrag_offset(ar, rho % d, rho >= d ? 1 : 0, d / 32)] = (_Float16)v;
    if (ar < nq) qx[size_t(ar) * 2 * d + rho] = acc[r];   // [Pi q | S q], float32
  }
}

// ---------------------------------------------------------------- key operand decode
// B dword i of substep s (coordinates p = 8 s + i and p + 16 after the lane-half shift).
// Sign plane: fp16 pair +-v with the sign bit inserted from the complemented plane word.
__device__ __forceinline__ uint32_t sign_pair(uint32_t nplane_sh, int p, uint32_t base) {
  const uint32_t sb = nplane_sh << (15 - p);
  return (sb & 0x80008000u) | (base & 0x7fff7fffu);
}

// Codebook value of two coordinates (bits p and p + 16 of the shifted planes): the fp16
// bytes of the magnitude are looked up with v_perm_b32 in the 4-entry table, the sign comes
// from the top index bit.  b = 4 reads the 2-bit magnitude index from a word holding the two
// index bits of even coordinates side by side (ev) or of odd coordinates (od).
template <int B>
__device__ __forceinline__ uint32_t mse_pair(uint32_t ev, uint32_t od, uint32_t nsg, int p,
                                             uint32_t tab_lo, uint32_t tab_hi) {
  uint32_t mag;
  if constexpr (B == 2) {
    mag = tab_lo;   // one magnitude, already a packed pair
  } else {
    uint32_t t;
    if constexpr (B == 4)
      t = (p & 1) ? (od >> (p - 1)) & 0x00030003u : (ev >> p) & 0x00030003u;
    else
      t = (ev >> p) & 0x00010001u;
    const uint32_t sel = t * 0x0101u + 0x04000400u;
    mag = __builtin_amdgcn_perm(tab_hi, tab_lo, sel);
  }
  return sign_pair(nsg, p, mag);
}

// v from lane ctrl(lane) of its row (a DPP move; every source lane is inside the row here)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ uint32_t f16_bits(float v) {
  return uint32_t(__builtin_bit_cast(uint16_t, (_Float16)v));
}

// ------------------------------------------------------------- scan + running top-k

template <int B, bool PROD, int KM>
__global__ __launch_bounds__(256, 1) void topk_scan_kernel(
    const unsigned char* __restrict__ params, const _Float16* __restrict__ qf,
    const uint32_t* __restrict__ codes, const float* __restrict__ nu,
    const float* __restrict__ gamma, int G, float s_unscale, long n, int QT, long RB,
    long nsplit, int k, long nq, const float* __restrict__ qn, int* __restrict__ cand_idx,
    float* __restrict__ cand_score, float2* __restrict__ ovf_all) {
  // two operand buffers as distinct objects, selected at compile time, so the compiler can
  // tell reads of one from the direct loads in flight into the other
  __shared__ __attribute__((aligned(16))) _Float16 Abuf0[STEP_HALVES];
  __shared__ __attribute__((aligned(16))) _Float16 Abuf1[STEP_HALVES];
  __shared__ __attribute__((aligned(16))) float theta[QROWS];   // score of each query's k-th entry
  __shared__ __attribute__((aligned(16))) int thidx[QROWS];     // its key (INT_MAX until k held)
  __shared__ int cnt[QROWS];
  constexpr int CAND = cand_slots(KM);
  constexpr int CSTRIDE = CAND + 1;                             // padded: conflict-free both ways
  __shared__ float Ls[KM * QROWS];                              // lists, entry e of row r at e * QROWS + r
  __shared__ int Li[KM * QROWS];
  __shared__ float Cs[QROWS * CSTRIDE];                         // candidates, slot c of row r at r * CSTRIDE + c
  __shared__ int Ci[QROWS * CSTRIDE];
  __shared__ float nus[KEYS];                                   // nu of the block's keys
  __shared__ int hbase[64];                                     // 4 h of each lane (see below)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, nl = lane & 31;
  const int qt = int(blockIdx.x % unsigned(QT));
  const long split = long(blockIdx.x / unsigned(QT));
  const long NB = (n + KEYS - 1) / KEYS;
  const long blk0 = split * RB;
  const long blk1 = blk0 + RB < NB ? blk0 + RB : NB;
  const _Float16* qsrc = qf + size_t(qt) * G * STEP_HALVES;
  float2* ovf = ovf_all + size_t(blockIdx.x) * QROWS * KEYS;   // this workgroup's overflow log

  // positive half of the codebook as fp16 bytes (v_perm_b32 table)
  const Header* hdr = reinterpret_cast<const Header*>(params);
  const float ag_unit = s_unscale * hdr->alpha;                 // key side: ag_unit gamma_j (2 z - 1)
  constexpr int L = 1 << (B - 1);
  uint32_t tab_lo = 0, tab_hi = 0;
  if constexpr (B == 2) {
    const uint32_t hv = f16_bits(hdr->cen[1]);
    tab_lo = hv | (hv << 16);
  } else {
#pragma unroll
    for (int m = 0; m < L / 2; ++m) {
      const uint32_t hv = f16_bits(hdr->cen[L / 2 + m]);
      tab_lo |= (hv & 0xffu) << (8 * m);
      tab_hi |= (hv >> 8) << (8 * m);
    }
  }

  if (tid < QROWS) {
    theta[tid] = -INFINITY;
    thidx[tid] = 0x7fffffff;
    cnt[tid] = 0;
  }
  if (tid < 64) hbase[tid] = 4 * (tid >> 5);
  int lcount = 0;   // entries in the list of query row tid (tid < QROWS)

  // query operand of coordinate group w -> buf by direct global -> LDS loads: wave-instruction
  // m writes 1 KiB (64 lanes x 16 bytes) at LDS chunk 4 m + wave
  constexpr int DMA_PER_WAVE = STEP_HALVES * 2 / 1024 / 4;
  auto stage = [&](int w, _Float16* buf) {
    const u32x4* src = reinterpret_cast<const u32x4*>(qsrc + size_t(w) * STEP_HALVES);
#pragma unroll
    for (int m = 0; m < DMA_PER_WAVE; ++m) {
      const int chunk = 4 * m + wave;
      __builtin_amdgcn_global_load_lds((gptr)(src + chunk * 64 + lane),
                                       (lptr)(reinterpret_cast<u32x4*>(buf) + chunk * 64),
                                       16, 0, 0);
    }
  };
  stage(0, Abuf0);
  __syncthreads();

  auto better = [](float s1, int i1, float s2, int i2) { return s1 > s2 || (s1 == s2 && i1 < i2); };
  auto insert = [&](float sc, int j) {
    if (lcount == k && !better(sc, j, Ls[(k - 1) * QROWS + tid], Li[(k - 1) * QROWS + tid])) return;
    int pos = lcount < k ? lcount : k - 1;
    while (pos > 0) {
      const float ps = Ls[(pos - 1) * QROWS + tid];
      const int pi = Li[(pos - 1) * QROWS + tid];
      if (!better(sc, j, ps, pi)) break;
      Ls[pos * QROWS + tid] = ps;
      Li[pos * QROWS + tid] = pi;
      --pos;
    }
    Ls[pos * QROWS + tid] = sc;
    Li[pos * QROWS + tid] = j;
    if (lcount < k) ++lcount;
  };

  // Packed plane words of one key and coordinate group, one buffer load per key through a
  // resource spanning one block (keys past n read as 0).  Their count is exact: each step
  // ends by waiting until at most this step's KT code loads are outstanding, which covers
  // its direct LDS loads (vector-memory loads complete in issue order).
  const size_t blk_words = size_t(KEYS) * G * B;
  auto block_rsrc = [&](long blk) {
    const long nk = n - blk * KEYS;
    const int bytes = nk <= 0 ? 0 : int((nk < KEYS ? nk : KEYS) * G * B * 4);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(codes) + size_t(blk) * blk_words,
                                             0, bytes, 0x00020000);
  };
  auto load_codes = [&](uint32_t* P, __amdgpu_buffer_rsrc_t rs, int key, int w) {
    const int off = (key * G + w) * B * 4;
    if constexpr (B == 4) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
      P[0] = v[0]; P[1] = v[1]; P[2] = v[2]; P[3] = v[3];
    } else if constexpr (B == 3) {
      const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rs, off, 0, 0);
      P[0] = v[0]; P[1] = v[1]; P[2] = v[2]; P[3] = 0u;
    } else {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
      P[0] = v[0]; P[1] = v[1]; P[2] = P[3] = 0u;
    }
  };
  // two-step-ahead ring of code words: pw[w & 1] holds group w of the current block's keys
  uint32_t pw[2][KT][4];
  {
    const __amdgpu_buffer_rsrc_t rs = block_rsrc(blk0);
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) load_codes(pw[par][kt], rs, wave * 32 * KT + 32 * kt + nl, par);
  }

  for (long blk = blk0; blk < blk1; ++blk) {
    long jk[KT];
    bool ok[KT];
    uint32_t agp[KT];
    float nuv[KT];   // loaded here, used by the selection after the block's MFMAs
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      jk[kt] = blk * KEYS + wave * 32 * KT + 32 * kt + nl;
      ok[kt] = jk[kt] < n;
      const uint32_t hv = (PROD && ok[kt]) ? f16_bits(ag_unit * gamma[jk[kt]]) : 0u;
      agp[kt] = hv | (hv << 16);
      nuv[kt] = ok[kt] ? nu[jk[kt]] : 0.f;
    }
    f32x16 acc[RT][KT];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) acc[i][kt] = f32x16{};

    // one step: coordinate group w from buffer ab while the next group streams into nxt
    // (G is even, so even groups always read Abuf0 and odd groups Abuf1)
    auto step = [&](const int w, const int par, const _Float16* ab, _Float16* nxt) {
      // every step (and the prologue) leaves at most KT loads in flight; restating it lets
      // the compiler see that this step's plane words, loaded two steps ago, are ready
      __builtin_amdgcn_s_waitcnt(vmcnt_only(KT));
      // key operands: plane words -> magnitude-index bits and complemented sign planes,
      // pre-shifted by the lane half (4 h) so that bit 8 s + i is coordinate p
      uint32_t ev[KT], od[KT], nsg[KT], nz[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const uint32_t* P = pw[par][kt];
        const int sh = 4 * h;
        ev[kt] = od[kt] = 0u;
        if constexpr (B == 2) {
          nsg[kt] = (~P[0]) >> sh;
        } else if constexpr (B == 3) {
          ev[kt] = (P[0] ^ ~P[1]) >> sh;
          nsg[kt] = (~P[1]) >> sh;
        } else {
          const uint32_t m0 = (P[0] ^ ~P[2]) >> sh, m1 = (P[1] ^ ~P[2]) >> sh;
          ev[kt] = (m0 & 0x55555555u) | ((m1 & 0x55555555u) << 1);
          od[kt] = ((m0 >> 1) & 0x55555555u) | (m1 & 0xaaaaaaaau);
          nsg[kt] = (~P[2]) >> sh;
        }
        nz[kt] = (~P[B - 1]) >> sh;
      }
      __builtin_amdgcn_sched_barrier(0);
      // Loads of this step, spread over the first MFMA iterations so that the four waves do
      // not queue them all at once: the next group's query operand (DMA_PER_WAVE direct LDS
      // loads), then the code words two steps ahead (group w + 2, or the next block's group
      // w + 2 - G), which must stay the newest loads for the wait at the end of the step.
      const bool last = w + 1 == G;
      const bool dostage = !last || blk + 1 < blk1;
      const u32x4* dsrc = reinterpret_cast<const u32x4*>(qsrc + size_t(last ? 0 : w + 1) * STEP_HALVES);
      const bool wrap = w + 2 >= G;
      const __amdgpu_buffer_rsrc_t crs = block_rsrc(wrap ? blk + 1 : blk);
      const int cw = wrap ? w + 2 - G : w + 2;
      auto issue = [&](int f) {
        if (f < DMA_PER_WAVE) {
          if (dostage) {
            const int chunk = 4 * f + wave;
            __builtin_amdgcn_global_load_lds((gptr)(dsrc + chunk * 64 + lane),
                                             (lptr)(reinterpret_cast<u32x4*>(nxt) + chunk * 64),
                                             16, 0, 0);
          }
        } else if (f < DMA_PER_WAVE + KT) {
          const int kt = f - DMA_PER_WAVE;
          load_codes(pw[par][kt], crs, wave * 32 * KT + 32 * kt + nl, cw);
        }
      };
      constexpr int NS = PROD ? 4 : 2;   // K16 substeps: 2 codebook + 2 sign
      constexpr int NF = NS * RT;        // A fragments (substep-major, row tile minor)
      auto dec = [&](int s, int kt, int dw) -> uint32_t {
        const int p = 8 * (s & 1) + dw;
        return s < 2 ? mse_pair<B>(ev[kt], od[kt], nsg[kt], p, tab_lo, tab_hi)
                     : sign_pair(nz[kt], p, agp[kt]);
      };
      auto frag = [&](int f) {
        return *reinterpret_cast<const f16x8*>(ab + (((f % RT) * 4 + f / RT) * 64 + lane) * 8);
      };
      u32x4 bc[KT], bn[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int dw = 0; dw < 4; ++dw) bc[kt][dw] = dec(0, kt, dw);
      // f -> (substep f / RT, row tile f % RT): A fragments prefetched PF ahead, each feeding
      // KT MFMAs; the next substep's key operands are decoded KT dwords per fragment
      f16x8 fq[PF];
#pragma unroll
      for (int f = 0; f < PF; ++f) fq[f] = frag(f);
      static_assert(NF >= DMA_PER_WAVE + KT, "every load is issued inside the step");
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int s = f / RT, i = f % RT;
        issue(f);
        const f16x8 fa = fq[f % PF];
        if (f + PF < NF) fq[f % PF] = frag(f + PF);
        if (s + 1 < NS) {
          constexpr int DPI = KT * 4 / RT;       // next-operand dwords decoded per iteration
          static_assert(DPI * RT == KT * 4, "decode spread");
#pragma unroll
          for (int q = 0; q < DPI; ++q) {
            const int d = i * DPI + q;             // dword d of the KT x 4 next operands
            bn[d >> 2][d & 3] = dec(s + 1, d >> 2, d & 3);
          }
        }
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
          acc[i][kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa, __builtin_bit_cast(f16x8, bc[kt]),
                                                              acc[i][kt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (i == RT - 1) {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) bc[kt] = bn[kt];
        }
      }
      // this wave's direct LDS loads are complete once at most its KT newest loads (the code
      // words just issued) are outstanding
      __builtin_amdgcn_s_waitcnt(vmcnt_only(KT));
      __builtin_amdgcn_s_barrier();
    };
    for (int w = 0; w < G; w += 2) {
      step(w, 0, Abuf0, Abuf1);
      step(w + 1, 1, Abuf1, Abuf0);
    }

    // ---- selection: accumulator register r of tile (i, kt) in lane l is query row
    //      32 i + 8 (r / 4) + 4 h + r % 4 and key jk[kt]; score = nu * acc (the |q| factor is
    //      applied on output).  Pending bit 16 (kt & 1) + r of word NW i + kt / 2.
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) nus[wave * 32 * KT + 32 * kt + nl] = nuv[kt];
    // The lane's row offset 4 h, read back from LDS here (after the last step's barrier):
    // as a value of this block it keeps the compiler from precomputing the 128 row addresses
    // of the epilogue once for the whole loop, which would hold them in registers throughout.
    const int hb = hbase[lane];
    // First block of the range: seed every row's threshold with a lower bound of its k-th
    // best score, the k-th largest of the maxima over 16 KT disjoint 8-key groups (k
    // distinct keys reach it).  Without it every key of the block would queue for a slot.
    // A group's 8 keys sit in 8 consecutive lanes: quad swaps and a half-row mirror (DPP)
    // leave the group maximum in each of them.
    constexpr int NGRP = 16 * KT;
    if (blk == blk0 && k <= NGRP) {
      float* gm = reinterpret_cast<float*>(Abuf1);   // idle here; [QROWS][NGRP]
      static_assert(QROWS * NGRP * 4 <= STEP_HALVES * 2, "group maxima fit the idle buffer");
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float v = ok[kt] ? acc[i][kt][r] * nuv[kt] : -INFINITY;
            v = fmaxf(v, dpp_f<0xB1>(v));    // quad_perm [1, 0, 3, 2]
            v = fmaxf(v, dpp_f<0x4E>(v));    // quad_perm [2, 3, 0, 1]
            v = fmaxf(v, dpp_f<0x141>(v));   // row_half_mirror
            if ((lane & 7) == 0) {
              const int row = 32 * i + 8 * (r >> 2) + hb + (r & 3);
              gm[row * NGRP + (wave * KT + kt) * 4 + ((lane >> 3) & 3)] = v;
            }
          }
      __syncthreads();
      if (tid < QROWS) {
        // the value whose rank (larger first, ties by position) is k - 1; read from LDS as
        // compared (once per key range), so that no register array is live beside the
        // accumulators
        const float* gr = gm + tid * NGRP;
        float th = -INFINITY;
#pragma unroll 1
        for (int a2 = 0; a2 < NGRP; ++a2) {
          const float ga = gr[a2];
          int rank = 0;
#pragma unroll 8
          for (int b2 = 0; b2 < NGRP; ++b2) {
            const float gb = gr[b2];
            rank += (gb > ga || (gb == ga && b2 < a2)) ? 1 : 0;
          }
          if (rank == k - 1) th = ga;
        }
        theta[tid] = th;
        thidx[tid] = 0x7fffffff;
      }
      __syncthreads();
    }
    // pass 1: exact (score, key) test against each row's k-th entry as of the last merge
    uint32_t pend[NW * RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      uint32_t mk[NW] = {};
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 th = *reinterpret_cast<const float4*>(&theta[32 * i + 8 * g + hb]);
        const int4 ti = *reinterpret_cast<const int4*>(&thidx[32 * i + 8 * g + hb]);
        const float tv[4] = {th.x, th.y, th.z, th.w};
        const int tj[4] = {ti.x, ti.y, ti.z, ti.w};
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            if (ok[kt] && better(acc[i][kt][4 * g + rr] * nuv[kt], int(jk[kt]), tv[rr], tj[rr]))
              mk[kt >> 1] |= 1u << (16 * (kt & 1) + 4 * g + rr);
      }
#pragma unroll
      for (int q = 0; q < NW; ++q) pend[NW * i + q] = mk[q];
    }
    // Candidates wait in per-row LDS slots across blocks; one that finds its row's slots
    // full goes to the row's overflow log in the workspace (only under massive ties: the
    // seeded thresholds keep the counts near k).  The lists are merged (raising the
    // thresholds) when a row's slots are half used or overflowed, and at the end of the
    // range.  A row receives at most KEYS candidates between merges beyond its CAND slots.
    const bool last_blk = blk + 1 == blk1;
    {
      float nua[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) nua[kt] = nus[wave * 32 * KT + 32 * kt + nl];
#pragma unroll
      for (int q = 0; q < NW * RT; ++q) {
        if (__builtin_amdgcn_ballot_w64(pend[q] != 0) == 0) continue;
        const int i = q / NW;
#pragma unroll
        for (int hk = 0; hk < 2 && 2 * (q % NW) + hk < KT; ++hk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kt = 2 * (q % NW) + hk;
            if (pend[q] & (1u << (16 * hk + r))) {
              const int row = 32 * i + 8 * (r >> 2) + hb + (r & 3);
              const int pos = atomicAdd(&cnt[row], 1);
              if (pos < CAND) {
                Cs[row * CSTRIDE + pos] = acc[i][kt][r] * nua[kt];
                Ci[row * CSTRIDE + pos] = int(jk[kt]);
              } else {
                ovf[size_t(row) * KEYS + (pos - CAND)] =
                    make_float2(acc[i][kt][r] * nua[kt], __int_as_float(int(jk[kt])));
              }
            }
          }
      }
    }
    __syncthreads();
    const bool need = __syncthreads_or(tid < QROWS && cnt[tid] >= CAND / 2) != 0;
    if (need || last_blk) {
      if (tid < QROWS) {
        const int mc = cnt[tid];
        for (int e = 0; e < mc; ++e) {
          if (e < CAND) {
            insert(Cs[tid * CSTRIDE + e], Ci[tid * CSTRIDE + e]);
          } else {
            const float2 o = ovf[size_t(tid) * KEYS + (e - CAND)];
            insert(o.x, __float_as_int(o.y));
          }
        }
        cnt[tid] = 0;
        if (lcount == k) {   // (a seeded threshold stays until the list is full)
          theta[tid] = Ls[(k - 1) * QROWS + tid];
          thidx[tid] = Li[(k - 1) * QROWS + tid];
        }
      }
      __syncthreads();
    }
  }

  const long a = long(qt) * QROWS + tid;
  if (tid < QROWS && a < nq) {
    const size_t base = (size_t(a) * nsplit + split) * k;
    const float qa = qn[a];
    for (int e = 0; e < k; ++e) {
      cand_score[base + e] = e < lcount ? Ls[e * QROWS + tid] * qa : -FLT_MAX;
      cand_idx[base + e] = e < lcount ? Li[e * QROWS + tid] : -1;
    }
  }
}

// ------------------------------------------------------------------ final merge
// One workgroup per query: k rounds of a block-wide arg-max over the candidate lists
// (larger score first, then smaller index; empty slots carry index -1 and lose).
__device__ __forceinline__ bool better_c(float s1, int i1, float s2, int i2) {
  if (i2 < 0) return i1 >= 0;
  if (i1 < 0) return false;
  return s1 > s2 || (s1 == s2 && i1 < i2);
}

__global__ __launch_bounds__(256) void topk_merge_kernel(int* __restrict__ cand_idx,
                                                          const float* __restrict__ cand_score,
                                                          long per_query, int k,
                                                          int32_t* __restrict__ out_idx,
                                                          float* __restrict__ out_score) {
  __shared__ float rs[256];
  __shared__ int ri[256];
  __shared__ long rp[256];
  const long a = blockIdx.x;
  int* ci = cand_idx + size_t(a) * per_query;
  const float* cs = cand_score + size_t(a) * per_query;
  for (int e = 0; e < k; ++e) {
    float bs = -FLT_MAX;
    int bi = -1;
    long bp = -1;
    for (long p = threadIdx.x; p < per_query; p += 256) {
      const int i = ci[p];
      const float s = cs[p];
      if (better_c(s, i, bs, bi)) {
        bs = s;
        bi = i;
        bp = p;
      }
    }
    rs[threadIdx.x] = bs;
    ri[threadIdx.x] = bi;
    rp[threadIdx.x] = bp;
    __syncthreads();
    for (int hh = 128; hh > 0; hh >>= 1) {
      if (threadIdx.x < hh &&
          better_c(rs[threadIdx.x + hh], ri[threadIdx.x + hh], rs[threadIdx.x], ri[threadIdx.x])) {
        rs[threadIdx.x] = rs[threadIdx.x + hh];
        ri[threadIdx.x] = ri[threadIdx.x + hh];
        rp[threadIdx.x] = rp[threadIdx.x + hh];
      }
      __syncthreads();
    }
    if (threadIdx.x == 0) {
      out_idx[size_t(a) * k + e] = ri[0];
      out_score[size_t(a) * k + e] = rs[0];
      if (rp[0] >= 0) ci[rp[0]] = -1;   // taken
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ float32 rescore
// One workgroup per query: the float32 estimate of each of the kk candidates that the fp16
// scan kept, l = nu_j (<Pi q, chat_j> + alpha gamma_j <S q, 2 z_j - 1>) from the float32
// products Pi q, S q of the query prep (the formula of the general scoring path), then the k
// best by decreasing estimate, equal estimates by increasing key index.
template <int B, bool PROD>
__global__ __launch_bounds__(256) void topk_rescore_kernel(const unsigned char* __restrict__ params, int d,
                                                            const uint32_t* __restrict__ codes,
                                                            const float* __restrict__ nu,
                                                            const float* __restrict__ gamma,
                                                            const float* __restrict__ qx,
                                                            const int* __restrict__ top_idx, int kk, int k,
                                                            int32_t* __restrict__ out_idx,
                                                            float* __restrict__ out_score) {
  __shared__ float qs[2 * 4096];     // Pi q, S q of this query
  __shared__ float cs[KMAX];
  __shared__ int ci[KMAX];
  const long a = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = d / 32;
  for (int t = tid; t < 2 * d; t += 256) qs[t] = qx[size_t(a) * 2 * d + t];
  const Header* hdr = reinterpret_cast<const Header*>(params);
  constexpr int L = 1 << (B - 1);
  float cen[L];
#pragma unroll
  for (int i = 0; i < L; ++i) cen[i] = hdr->cen[i];
  const float alpha = hdr->alpha;
  __syncthreads();
  for (int c = wave; c < kk; c += 4) {
    const int j = top_idx[size_t(a) * kk + c];   // uniform over the wave
    float mse = 0.f, qjl = 0.f;
    if (j >= 0) {
      for (int g = lane; g < G; g += 64) {
        const uint32_t* w = codes + (size_t(j) * G + g) * B;
        uint32_t pl[B];
#pragma unroll
        for (int p = 0; p < B; ++p) pl[p] = w[p];
#pragma unroll 8
        for (int t = 0; t < 32; ++t) {
          int idx = 0;
#pragma unroll
          for (int p = 0; p < B - 1; ++p) idx |= int((pl[p] >> t) & 1u) << p;
          float cv = cen[0];
#pragma unroll
          for (int i = 1; i < L; ++i) cv = idx == i ? cen[i] : cv;
          mse = fmaf(qs[32 * g + t], cv, mse);
          if constexpr (PROD) {
            const float sv = qs[d + 32 * g + t];
            qjl += ((pl[B - 1] >> t) & 1u) ? sv : -sv;
          }
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      mse += __shfl_xor(mse, o);
      qjl += __shfl_xor(qjl, o);
    }
    if (lane == 0) {
      ci[c] = j;
      cs[c] = j >= 0 ? nu[j] * (PROD ? mse + alpha * gamma[j] * qjl : mse) : -FLT_MAX;
    }
  }
  __syncthreads();
  if (tid == 0) {
    // insertion sort of the kk (<= 32) candidates, best first; empty slots (key -1) last
    for (int e = 1; e < kk; ++e) {
      const float sv = cs[e];
      const int iv = ci[e];
      int pos = e;
      while (pos > 0 && better_c(sv, iv, cs[pos - 1], ci[pos - 1])) {
        cs[pos] = cs[pos - 1];
        ci[pos] = ci[pos - 1];
        --pos;
      }
      cs[pos] = sv;
      ci[pos] = iv;
    }
    for (int e = 0; e < k; ++e) {
      out_idx[size_t(a) * k + e] = ci[e];
      out_score[size_t(a) * k + e] = cs[e];
    }
  }
}

template <int B, int KM>
hipError_t launch_scan_km(bool prod, dim3 grid, const unsigned char* params, const _Float16* qf,
                          const uint32_t* codes, const float* nu, const float* gamma, int G,
                          float s_unscale, long n, int QT, long RB, long nsplit, int k, long nq,
                          const float* qn, int* cand_idx, float* cand_score, float2* ovf,
                          hipStream_t s) {
  if (prod)
    hipLaunchKernelGGL((topk_scan_kernel<B, true, KM>), grid, dim3(256), 0, s, params, qf, codes,
                       nu, gamma, G, s_unscale, n, QT, RB, nsplit, k, nq, qn, cand_idx, cand_score,
                       ovf);
  else
    hipLaunchKernelGGL((topk_scan_kernel<B, false, KM>), grid, dim3(256), 0, s, params, qf, codes,
                       nu, gamma, G, s_unscale, n, QT, RB, nsplit, k, nq, qn, cand_idx, cand_score,
                       ovf);
  return hipGetLastError();
}

template <int B>
hipError_t launch_scan(bool prod, dim3 grid, const unsigned char* params, const _Float16* qf,
                       const uint32_t* codes, const float* nu, const float* gamma, int G,
                       float s_unscale, long n, int QT, long RB, long nsplit, int k, long nq,
                       const float* qn, int* cand_idx, float* cand_score, float2* ovf,
                       hipStream_t s) {
  // lists of 16 entries leave room for more candidate slots (fewer merges)
  if (k <= 16)
    return launch_scan_km<B, 16>(prod, grid, params, qf, codes, nu, gamma, G, s_unscale, n, QT, RB,
                                 nsplit, k, nq, qn, cand_idx, cand_score, ovf, s);
  return launch_scan_km<B, KMAX>(prod, grid, params, qf, codes, nu, gamma, G, s_unscale, n, QT, RB,
                                 nsplit, k, nq, qn, cand_idx, cand_score, ovf, s);
}

}  // namespace

size_t topk_ws_bytes(int d, int b, int64_t nq, int64_t n, int k) {
  (void)b;
  if (k > KFUSED) return topk_large_ws_bytes(d, nq, n);
  return plan(d, nq, n, k).total;
}

hipError_t launch_topk(const void* params_v, int d, int b, const void* q, int q_dtype, int64_t nq,
                       const uint32_t* codes, const float* nu, const float* gamma, int64_t n,
                       int k, int mode, int32_t* idx, float* score, void* ws, hipStream_t s) {
  if (d % 32 != 0) return hipErrorNotSupported;
  if (k > KFUSED)
    return launch_topk_large(params_v, d, b, q, q_dtype, nq, codes, nu, gamma, n, k, mode, idx, score,
                             ws, s);
  const unsigned char* params = static_cast<const unsigned char*>(params_v);
  const Layout lay(d, b);
  const Plan p = plan(d, nq, n, k);
  unsigned char* w = static_cast<unsigned char*>(ws);
  _Float16* qf = reinterpret_cast<_Float16*>(w + p.off_q);
  float* qn = reinterpret_cast<float*>(w + p.off_qn);
  float* qx = reinterpret_cast<float*>(w + p.off_qx);
  const int kk = p.kk;
  int* cand_idx = reinterpret_cast<int*>(w + p.off_cand);
  float* cand_score = reinterpret_cast<float*>(w + p.off_cand + size_t(nq) * p.nsplit * kk * 4);
  int* top_idx = reinterpret_cast<int*>(w + p.off_top);
  float* top_score = reinterpret_cast<float*>(w + p.off_top + size_t(nq) * kk * 4);
  float2* ovf = reinterpret_cast<float2*>(w + p.off_ovf);
  const int G = d / 32;

  // query operands: (padded query tiles / 32) x (2d / 32) waves, 4 per workgroup
  const long rows_pad = p.qt * QROWS;
  const long waves = (rows_pad / 32) * (2 * d / 32);
  hipLaunchKernelGGL(topk_qprep_kernel, dim3(unsigned((waves + 3) / 4)), dim3(256), 0, s, params,
                     lay.off_pi, lay.off_s, d, q, q_dtype == 0 ? 1 : 0, long(nq), rows_pad, qf, qn, qx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // workgroup x -> (query tile x % QT, key range x / QT): consecutive workgroups land on
  // different XCDs, so with QT dividing 8 each XCD keeps reading one query tile from its L2
  // the query operand carries S q / sqrt(d); the kernel multiplies the key side back by
  // sqrt(d) alpha gamma_j, alpha from the parameter header
  const float s_unscale = std::sqrt(float(d));
  const dim3 grid(unsigned(p.qt * p.nsplit));
  const bool prod = mode == 0;
  switch (b) {
    case 2: e = launch_scan<2>(prod, grid, params, qf, codes, nu, gamma, G, s_unscale, n, int(p.qt), p.rb,
                               p.nsplit, kk, nq, qn, cand_idx, cand_score, ovf, s); break;
    case 3: e = launch_scan<3>(prod, grid, params, qf, codes, nu, gamma, G, s_unscale, n, int(p.qt), p.rb,
                               p.nsplit, kk, nq, qn, cand_idx, cand_score, ovf, s); break;
    default: e = launch_scan<4>(prod, grid, params, qf, codes, nu, gamma, G, s_unscale, n, int(p.qt), p.rb,
                                p.nsplit, kk, nq, qn, cand_idx, cand_score, ovf, s); break;
  }
  if (e != hipSuccess) return e;
  // the kk best fp16 candidates over all key ranges, then their float32 estimates decide
  hipLaunchKernelGGL(topk_merge_kernel, dim3(unsigned(nq)), dim3(256), 0, s, cand_idx, cand_score,
                     long(p.nsplit) * kk, kk, top_idx, top_score);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
#define TQ_RESCORE(BB)                                                                              \
  if (prod)                                                                                         \
    hipLaunchKernelGGL((topk_rescore_kernel<BB, true>), dim3(unsigned(nq)), dim3(256), 0, s, params, d, \
                       codes, nu, gamma, qx, top_idx, kk, k, idx, score);                             \
  else                                                                                              \
    hipLaunchKernelGGL((topk_rescore_kernel<BB, false>), dim3(unsigned(nq)), dim3(256), 0, s, params, d, \
                       codes, nu, gamma, qx, top_idx, kk, k, idx, score);
  switch (b) {
    case 2: TQ_RESCORE(2) break;
    case 3: TQ_RESCORE(3) break;
    default: TQ_RESCORE(4) break;
  }
#undef TQ_RESCORE
  return hipGetLastError();
}

}  // namespace tq
