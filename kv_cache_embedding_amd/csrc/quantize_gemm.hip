// TurboQuant encoder for any d != 128 that is a multiple of 64 (e.g. 1536-dimensional
// embeddings)
// ([review, inner-product paragraph]; [tldr, steps 1-2]), per chunk of vectors:
//   split:    nu = |x| per vector; float32 x is split into bf16 rows x_hi + x_lo (RNE);
//   phase 1:  U = X Pi^T (rows = vectors, columns = rotated coordinates); its epilogue
//             divides by nu, bucketizes, packs the index planes, writes the residual
//             r' = u - chat as bf16 hi/lo rows to a scratch buffer and its partial sum of
//             squares per (vector, column tile);
//   phase 2:  Y = R' S'^T with S' = S Pi^T; its epilogue packs the QJL sign plane and sums
//             the partials into gamma = |r'|.
// Both GEMMs run on v_mfma_f32_32x32x16_bf16 with hi/lo operand splits (Pi_hi x_hi +
// Pi_lo x_hi + Pi_hi x_lo, the last pass only for float32 inputs; S'_hi r_hi + S'_lo r_hi +
// S'_hi r_lo), float32 accumulation.  In the 32x32 accumulator layout (row = 8(r/4) +
// 4(lane/32) + r%4, column = lane % 32) a wave ballot over one accumulator register is
// exactly two packed words of the canonical layout (32 consecutive coordinates of two
// vectors).
//
// Tiling.  A workgroup computes a 256 x 256 output tile with 8 waves (two per SIMD) of
// 128 x 64: 4 x 2 accumulator tiles of 32 x 32, so every A fragment read from LDS feeds two
// MFMAs per pass and every B fragment four.  K advances 32 per stage; the operands of a
// stage come into LDS by direct global -> LDS loads, each 64-lane instruction filling one
// 1 KiB MFMA fragment in register order (lane l: row l % 32, K offset 8 (l / 32)),
// double-buffered with one barrier per stage.  Workgroups of one row block run on one XCD
// (dispatch is round-robin over the 8 XCDs), so its d / 256 column tiles share that XCD's
// L2 for the rows of X.
#include "tq_internal.h"

#include <type_traits>

namespace tq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(1))) const void* gptr;   // global
typedef __attribute__((address_space(3))) void* lptr;         // LDS

constexpr int WT = 256;          // workgroup tile: vectors x coordinates
constexpr int BK = 32;           // K per stage (two MFMA K steps, 64 bytes of a bf16 row)
constexpr int WAVES = 8;
constexpr long CHUNK = 32768;    // vectors per pass at d = 1536 (float32 rows)
// Scratch of one pass (bf16 hi/lo planes of r' and, for float32 rows, of x) is held to the
// d = 1536 float32 footprint; smaller d take proportionally more vectors per pass, so that
// one launch still fills the chip.
constexpr size_t SCRATCH_BUDGET = size_t(CHUNK) * 1536 * 2 * 4;

// Vectors per pass for rows of d (pitch xpitch) with `planes` bf16 scratch planes per row;
// at least CHUNK, and small enough that every byte offset of a pass fits 30 bits.
long chunk_rows(int64_t n, int d, long xpitch, int planes) {
  long ch = long(SCRATCH_BUDGET / (size_t(d) * 2 * planes));
  if (ch < CHUNK) ch = CHUNK;
  const long pitch = xpitch > d ? xpitch : long(d);
  const long cap = long((size_t(1) << 30) / size_t(pitch));
  if (ch > cap) ch = cap;
  return n < ch ? long(n) : ch;
}
constexpr int NXCD = 8;

// LDS blocks (1 KiB) of one stage: 16 rows x 32 K of one operand part.  B blocks
// [part][16-column block 0..15] (32), then A blocks [part][16-row block] (32, or 16 when A
// has no low part).  Row q of a block holds its 64 bytes as four 16-byte pieces, piece p
// at slot p ^ ((q / 4) % 4): a direct load fills the block from whole 64-byte row segments
// (lane L: row L / 4, slot L % 4), and an MFMA fragment read (lane l: row l % 32, piece
// 2 ks + l / 32) hits 16 distinct bank groups per 16 lanes.
template <bool ALO>
struct StageShape {
  static constexpr int NB = 32;
  static constexpr int NA = ALO ? 32 : 16;
  static constexpr int NF = NB + NA;
  static constexpr int U4 = NF * 64;     // uint4 per stage
};

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_bits(float v) {
  return uint32_t(__builtin_bit_cast(uint16_t, (__bf16)v));
}

// ------------------------------------------------------------------------------ split
// One wave per vector: nu = |x| (float32 sum of squares), and for float32 inputs the bf16
// rows x_hi = RNE(x), x_lo = RNE(x - x_hi).  Lane l covers coordinates 8 (l + 64 i) .. +7.
// Input rows are xpitch elements apart (a channel group of wider rows); x_hi, x_lo are
// written d apart.
template <bool F32IN>
__global__ __launch_bounds__(256) void qsplit_kernel(const void* __restrict__ x, long rows, int d,
                                                      long xpitch, uint16_t* __restrict__ xh,
                                                      uint16_t* __restrict__ xl, long v0,
                                                      float* __restrict__ nu_out) {
  const int lane = threadIdx.x & 63;
  const long row = long(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  float ss = 0.f;
  for (int c = 8 * lane; c < d; c += 512) {
    const size_t off = size_t(row) * d + c;
    const size_t in = size_t(row) * xpitch + c;
    if constexpr (F32IN) {
      const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + in);
      const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + in + 4);
      const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      uint32_t h[4], l[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        ss = fmaf(f[e], f[e], ss);
        ss = fmaf(f[e + 1], f[e + 1], ss);
        const uint32_t h0 = bf16_bits(f[e]), h1 = bf16_bits(f[e + 1]);
        h[e / 2] = h0 | (h1 << 16);
        l[e / 2] = bf16_bits(f[e] - __uint_as_float(h0 << 16)) |
                   (bf16_bits(f[e + 1] - __uint_as_float(h1 << 16)) << 16);
      }
      *reinterpret_cast<uint4*>(xh + off) = make_uint4(h[0], h[1], h[2], h[3]);
      *reinterpret_cast<uint4*>(xl + off) = make_uint4(l[0], l[1], l[2], l[3]);
    } else {
      const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + in);
      const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(w4[e] << 16), hi = __uint_as_float(w4[e] & 0xffff0000u);
        ss = fmaf(lo, lo, fmaf(hi, hi, ss));
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if (lane == 0) nu_out[v0 + row] = sqrtf(ss);
}

// ------------------------------------------------------------------------------- GEMMs
// Direct buffer -> LDS loads of one stage.  Block f = 8 m + wave of the stage is loaded by
// this wave: m < 4 are B blocks (part f / 16 = m / 2, column block f % 16), the rest A
// blocks.  Each source is a buffer resource (matrix part) plus the stage's K offset (the
// scalar offset) plus a per-lane byte offset (row or column times the row pitch, plus the
// K offset of the lane's piece) that does not change from stage to stage.  Buffer loads
// rather than global ones: the compiler takes a global load that writes LDS as a pending
// access to both memories, which turns every later partial wait for LDS reads into a full
// one.
constexpr int RSRC_WORD3 = 0x00020000;         // raw (untyped) buffer resource, gfx9 family

template <bool ALO>
struct DmaPlan {
  static constexpr int NA = ALO ? 4 : 2;     // A blocks per wave
  void* b[2];                                // B parts [hi, lo], bbytes each
  void* a[ALO ? 2 : 1];                      // A parts, abytes each
  int bbytes, abytes;
  uint32_t bo[4];
  uint32_t ao[NA];
};

// Loads blocks m0 and m0 + 1 of one part: block f = 8 m + wave lands at LDS block base + f.
__device__ __forceinline__ void dma_pair(__amdgpu_buffer_rsrc_t r, const uint32_t* vo, int m0,
                                         int k0, uint4* base, int wave) {
#pragma unroll
  for (int m = m0; m < m0 + 2; ++m)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lptr)(base + (WAVES * m + wave) * 64), 16, vo[m],
                                             k0 * 2, 0, 0);
}

template <bool ALO>
__device__ __forceinline__ void stage_dma(const DmaPlan<ALO>& p, int k0, uint4* dst, int wave) {
  dma_pair(__builtin_amdgcn_make_buffer_rsrc(p.b[0], 0, p.bbytes, RSRC_WORD3), p.bo, 0, k0, dst, wave);
  dma_pair(__builtin_amdgcn_make_buffer_rsrc(p.b[1], 0, p.bbytes, RSRC_WORD3), p.bo, 2, k0, dst, wave);
  dma_pair(__builtin_amdgcn_make_buffer_rsrc(p.a[0], 0, p.abytes, RSRC_WORD3), p.ao, 0, k0, dst + 32 * 64,
           wave);
  if constexpr (ALO)
    dma_pair(__builtin_amdgcn_make_buffer_rsrc(p.a[1], 0, p.abytes, RSRC_WORD3), p.ao, 2, k0,
             dst + 32 * 64, wave);
}

// The operand fragments of one MFMA K step (16 of a stage's 32) for the wave tile (rows
// 128 wm .., columns 64 wn ..): B hi/lo of its two 32-column tiles, A hi[/lo] of its four
// 32-row tiles.
template <bool ALO>
struct Frags {
  bf16x8 bh[2], bl[2], ah[4], al[ALO ? 4 : 1];
};

// b is the stage buffer plus the lane's byte offset of the K step within a pair of blocks
// (see the block layout above).
template <bool ALO>
__device__ __forceinline__ void read_b(Frags<ALO>& f, const char* b, int wn) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int cb = 2 * (2 * wn + j);           // first 16-column block of the column tile
    f.bh[j] = *reinterpret_cast<const bf16x8*>(b + cb * 1024);
    f.bl[j] = *reinterpret_cast<const bf16x8*>(b + (16 + cb) * 1024);
  }
}

template <bool ALO>
__device__ __forceinline__ void read_a(Frags<ALO>& f, const char* b, int wm, int i) {
  const int rb = 2 * (4 * wm + i);             // first 16-row block of the row tile
  f.ah[i] = *reinterpret_cast<const bf16x8*>(b + (32 + rb) * 1024);
  if constexpr (ALO) f.al[i] = *reinterpret_cast<const bf16x8*>(b + (48 + rb) * 1024);
}

// B is the MFMA's first operand, so acc[i][j] holds the transposed 32 x 32 tile: lane l
// has row (vector) 32 i + l % 32 and columns (coordinates) 32 j + 8 (r / 4) + 4 (l / 32) +
// r % 4 in its register r.
template <bool ALO>
__device__ __forceinline__ void mfma_row(f32x16 (&acc)[4][2], const Frags<ALO>& f, int i) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    acc[i][j] = mfma(f.bh[j], f.ah[i], acc[i][j]);
    acc[i][j] = mfma(f.bl[j], f.ah[i], acc[i][j]);
    if constexpr (ALO) acc[i][j] = mfma(f.bh[j], f.al[i], acc[i][j]);
  }
}

// The MFMAs of one K step (fragments f) while the next K step's fragments g come in from
// LDS: g's B fragments first, then its A fragments of each row tile once f's of that row
// tile are consumed, so the two sets share registers (the scheduling barriers keep that
// order).
template <bool ALO>
__device__ __forceinline__ void mfma_and_read(f32x16 (&acc)[4][2], const Frags<ALO>& f,
                                              Frags<ALO>& g, const char* b, int wm, int wn) {
  read_b(g, b, wn);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    mfma_row(acc, f, i);
    __builtin_amdgcn_sched_barrier(0);
    read_a(g, b, wm, i);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Stage s, held in cur, with its first K step's fragments already in f0: the first K
// step's MFMAs run while the second one's fragments come in; then (NEXT: stage s + 1
// exists), once every wave's loads of stage s + 1 (into nxt) have landed and every wave
// has read cur, the loads of stage s + 2 into cur start (DMA: it exists) and the second K
// step's MFMAs run while stage s + 1's first fragments come in.  The MFMAs after the
// barrier find their operands in registers.  The stage kinds are template arguments so
// that the loop body has no branches and every LDS access keeps its own buffer.
template <bool ALO, bool NEXT, bool DMA>
__device__ __forceinline__ void kstage(f32x16 (&acc)[4][2], Frags<ALO>& f0, Frags<ALO>& f1,
                                       uint4* cur, const uint4* nxt, const DmaPlan<ALO>& plan,
                                       const uint32_t (&off)[2], int wm, int wn, int wave, int s) {
  mfma_and_read(acc, f0, f1, reinterpret_cast<const char*>(cur) + off[1], wm, wn);
  // this wave's direct LDS loads of stage s + 1 and its reads of cur are complete before
  // the barrier (the compiler orders neither against the barrier by itself)
  __builtin_amdgcn_s_waitcnt(0);
  if constexpr (NEXT) {
    __syncthreads();
    if constexpr (DMA) stage_dma(plan, (s + 2) * BK, cur, wave);
    mfma_and_read(acc, f1, f0, reinterpret_cast<const char*>(nxt) + off[0], wm, wn);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) mfma_row(acc, f1, i);
  }
}

// Residual rows of one 32 x 64 wave tile through LDS (sb: 32 rows of 144 bytes, padded
// against bank conflicts), so that every global store is 16 bytes and eight lanes write a
// row's whole 128-byte segment.  Lane (row l % 32, half h) holds, per 32-column tile j and
// group g, the bf16 pairs of columns 32 j + 8 g + 4 h .. +3.
__device__ __forceinline__ void store_residual(char* sb, const uint32_t (&v)[2][4][2], int lane,
                                               uint16_t* dst, long row0, long rows_left, int d,
                                               int col0, bool okc0, bool okc1) {
  const int vr = lane & 31, h = lane >> 5;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<uint2*>(sb + vr * 144 + 64 * j + 16 * g + 8 * h) = make_uint2(v[j][g][0], v[j][g][1]);
  const int piece = lane & 7;                   // 16-byte piece: columns 8 piece .. +7
  const bool okc = piece < 4 ? okc0 : okc1;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int row = 8 * k + (lane >> 3);
    const uint4 w = *reinterpret_cast<const uint4*>(sb + row * 144 + 16 * piece);
    if (okc && row < rows_left)
      *reinterpret_cast<uint4*>(dst + size_t(row0 + row) * d + col0 + 8 * piece) = w;
  }
}

// PHASE 1: A = x (hi[/lo]) bf16 rows, B = Pi (hi/lo). PHASE 2: A = r' (hi/lo), B = S' (hi/lo).
// A rows are apitch elements apart (d, or the caller's row pitch for bf16 rows read in place).
// PHASE 3: phase 1 for the MSE quantizer alone: the b-1 index planes (a code stride of b-1
// words per coordinate group) and nothing for a phase 2.
// UOUT (diagnostic, phase 1 only): u = Pi x / nu of every vector is also written to u_out
// [rows of the call][d] float32 (row v0 + r of the call at u_out + (v0 + r) d), the values the
// bucketize reads.
template <int PHASE, int BITS, bool ALO, bool UOUT = false>
__global__ __launch_bounds__(WAVES * 64, 1) void qgemm_kernel(
    const unsigned char* __restrict__ params, const uint16_t* __restrict__ ahi,
    const uint16_t* __restrict__ alo, long rows, const uint16_t* __restrict__ bhi,
    const uint16_t* __restrict__ blo, int d, long apitch, long v0, int nrb, uint32_t* __restrict__ codes,
    const float* __restrict__ nu, float* __restrict__ gamma_out, uint16_t* __restrict__ rhi,
    uint16_t* __restrict__ rlo, float* __restrict__ gpart, float* __restrict__ u_out) {
  static_assert(!UOUT || PHASE == 1, "rotation output from phase 1 only");
  __shared__ uint4 buf0[StageShape<ALO>::U4];
  __shared__ uint4 buf1[StageShape<ALO>::U4];
  __shared__ float rowscale[WT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: branches stay scalar
  const int wm = wave >> 2, wn = wave & 3;     // wave tile: rows 128 wm .., columns 64 wn ..
  const int nct = (d + WT - 1) / WT;
  // block -> (row block, column tile): the column tiles of a row block share an XCD
  const int xcd = blockIdx.x % NXCD, slot = blockIdx.x / NXCD;
  const int rb = (slot / nct) * NXCD + xcd, ct = slot % nct;
  if (rb >= nrb) return;
  const long r0 = long(rb) * WT;               // first row (vector) of the tile in the chunk
  const int c0 = ct * WT;                      // first output coordinate of the tile

  // DMA plan of this wave (ragged rows and columns past d are clamped: they read valid
  // data whose results are discarded); lane L loads piece (L % 4) ^ ((L / 16) % 4) of row
  // L / 4 of its blocks
  const int q = lane >> 2, piece = (lane & 3) ^ ((lane >> 4) & 3);
  DmaPlan<ALO> plan;
  plan.b[0] = const_cast<uint16_t*>(bhi);
  plan.b[1] = const_cast<uint16_t*>(blo);
  plan.a[0] = const_cast<uint16_t*>(ahi);
  if constexpr (ALO) plan.a[1] = const_cast<uint16_t*>(alo);
  plan.bbytes = int(size_t(d) * d * 2);
  plan.abytes = int((size_t(rows - 1) * apitch + d) * 2);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int f = WAVES * m + wave;
    int col = c0 + 16 * (f & 15) + q;
    col = col < d ? col : d - 1;
    plan.bo[m] = uint32_t((size_t(col) * d + 8 * piece) * 2);
  }
#pragma unroll
  for (int m = 0; m < DmaPlan<ALO>::NA; ++m) {
    const int fa = WAVES * m + wave;
    long row = r0 + 16 * (fa & 15) + q;
    row = row < rows ? row : rows - 1;
    plan.ao[m] = uint32_t((size_t(row) * apitch + 8 * piece) * 2);
  }
  // fragment read offsets: lane l reads row l % 32 of a 32-row pair of blocks, piece
  // 2 ks + l / 32
  uint32_t off[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int rr = lane & 31, qq = rr & 15, pp = 2 * ks + (lane >> 5);
    off[ks] = uint32_t((rr >> 4) * 1024 + qq * 64 + 16 * (pp ^ ((qq >> 2) & 3)));
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // K loop: stage s is read from buffer s % 2 while stage s + 1 lands in the other one.
  // d is a multiple of 64, so the number of stages is even (at least 2).
  const int ns = d / BK;
  stage_dma(plan, 0, buf0, wave);
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  __syncthreads();
  stage_dma(plan, BK, buf1, wave);
  // The epilogue's arguments are loaded now: a scalar load still in flight during the loop
  // would turn every partial wait for LDS reads into a full one.
  asm volatile("" ::"s"(params), "s"(codes), "s"(nu), "s"(gamma_out), "s"(rhi), "s"(rlo),
               "s"(gpart), "s"(rows), "s"(v0));
  if constexpr (UOUT) asm volatile("" ::"s"(u_out));
  Frags<ALO> f0, f1;
  read_b(f0, reinterpret_cast<const char*>(buf0) + off[0], wn);
#pragma unroll
  for (int i = 0; i < 4; ++i) read_a(f0, reinterpret_cast<const char*>(buf0) + off[0], wm, i);
  for (int s = 0; s < ns - 2; s += 2) {
    kstage<ALO, true, true>(acc, f0, f1, buf0, buf1, plan, off, wm, wn, wave, s);
    kstage<ALO, true, true>(acc, f0, f1, buf1, buf0, plan, off, wm, wn, wave, s + 1);
  }
  kstage<ALO, true, false>(acc, f0, f1, buf0, buf1, plan, off, wm, wn, wave, ns - 2);
  kstage<ALO, false, false>(acc, f0, f1, buf1, buf0, plan, off, wm, wn, wave, ns - 1);

  const int groups = d / 32;
  if constexpr (PHASE == 1 || PHASE == 3) {
    constexpr bool MSE = PHASE == 3;
    constexpr int CB = MSE ? BITS - 1 : BITS;   // code words per coordinate group
    if (tid < WT) {
      const long row = r0 + tid < rows ? r0 + tid : rows - 1;
      const float nrm = nu[v0 + row];
      rowscale[tid] = nrm > 0.f ? 1.f / nrm : 0.f;   // zero vector: u is taken as 0
    }
    __syncthreads();   // also: every wave is done with buf0 before it holds the partials
    const Header* hdr = reinterpret_cast<const Header*>(params);
    constexpr int L = 1 << (BITS - 1);
    float T[L / 2 > 1 ? L / 2 - 1 : 1], M[L / 2];
#pragma unroll
    for (int k = 0; k < L / 2 - 1; ++k) T[k] = hdr->tpos[k];
#pragma unroll
    for (int k = 0; k < L / 2; ++k) M[k] = hdr->mpos[k];
    float* gsum = reinterpret_cast<float*>(buf0);   // [4 wn][256 rows] partial |r'|^2
    static_assert(WAVES * 32 * 144 <= StageShape<ALO>::U4 * 16, "transpose areas fit in buf1");
    char* sb = reinterpret_cast<char*>(buf1) + wave * (32 * 144);   // residual transpose area
    const int h = lane >> 5;
    // one row tile at a time (a compile-time index keeps the accumulators in registers)
    auto row_tile = [&](auto it) {
      constexpr int i = decltype(it)::value;
      const int vr = 128 * wm + 32 * i + (lane & 31);   // tile row (vector) of this lane
      const bool okr = r0 + vr < rows;
      const float rs = rowscale[vr];
      float g2 = 0.f;
      uint32_t hq[2][4][2], lq[2][4][2];         // residual bf16 pairs, stored after both tiles
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int cb = c0 + 64 * wn + 32 * j;    // first coordinate of this 32-column tile
        const bool okc = cb < d;                 // uniform: padding columns past d
        const int w = cb / 32;                   // coordinate group of this tile
        // index bits of the lane's 16 coordinates at their positions 8 g + e (+ 4 h below)
        uint32_t word[BITS - 1];
#pragma unroll
        for (int p = 0; p < BITS - 1; ++p) word[p] = 0u;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if constexpr (UOUT) {
            // coordinates cb + 8 g + 4 h + e, e = 0..3, of this lane's vector
            if (okc && okr)
              *reinterpret_cast<float4*>(u_out + size_t(v0 + r0 + vr) * d + cb + 8 * g + 4 * h) =
                  make_float4(acc[i][j][4 * g] * rs, acc[i][j][4 * g + 1] * rs, acc[i][j][4 * g + 2] * rs,
                              acc[i][j][4 * g + 3] * rs);
          }
          uint32_t hp[2] = {0u, 0u}, lp[2] = {0u, 0u};   // bf16 pairs of coordinates 4 h + e
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float u = acc[i][j][4 * g + e] * rs;
            // magnitude index k of |u| against the positive thresholds (a tie goes to the
            // outer cell), the level's side from the sign of u (0 to the positive side):
            // index = L/2 + k for u >= 0, L/2 - 1 - k for u < 0, so the low index bits are
            // the bits of k, complemented on the negative side
            const float a = fabsf(u);
            const bool pos = u >= 0.f;
            bool bit[3] = {false, false, false};
            float mag;
            if constexpr (BITS == 2) {
              bit[0] = pos;
              mag = M[0];
            } else if constexpr (BITS == 3) {
              const bool k0 = a >= T[0];
              bit[1] = pos;
              bit[0] = k0 == pos;
              mag = k0 ? M[1] : M[0];
            } else {
              const bool k1 = a >= T[1];
              const bool k0 = a >= (k1 ? T[2] : T[0]);
              bit[2] = pos;
              bit[1] = k1 == pos;
              bit[0] = k0 == pos;
              mag = k1 ? (k0 ? M[3] : M[2]) : (k0 ? M[1] : M[0]);
            }
            const float c = pos ? mag : -mag;
            const float rv = u - c;
            const uint32_t hb = bf16_bits(rv);
            const uint32_t lb = bf16_bits(rv - __uint_as_float(hb << 16));
            const float rq = __uint_as_float(hb << 16) + __uint_as_float(lb << 16);
            if (okc) g2 = fmaf(rq, rq, g2);      // the residual phase 2 will see
            hp[e / 2] |= hb << (16 * (e % 2));
            lp[e / 2] |= lb << (16 * (e % 2));
#pragma unroll
            for (int p = 0; p < BITS - 1; ++p) word[p] |= uint32_t(bit[p]) << (8 * g + e);
          }
          // 4 consecutive coordinates: lanes l and l + 32 write 16 contiguous bytes of a row
          hq[j][g][0] = hp[0];
          hq[j][g][1] = hp[1];
          lq[j][g][0] = lp[0];
          lq[j][g][1] = lp[1];
        }
        // lanes l and l + 32 hold the two nibble halves of each byte of the vector's words
#pragma unroll
        for (int p = 0; p < BITS - 1; ++p) {
          word[p] <<= 4 * h;
          word[p] |= __shfl_xor(word[p], 32);
        }
        if (okc && lane < 32 && okr) {
#pragma unroll
          for (int p = 0; p < BITS - 1; ++p) codes[(size_t(v0 + r0 + vr) * groups + w) * CB + p] = word[p];
        }
      }
      // residual rows 128 wm + 32 i .. +31, columns 64 wn .. +63 of the tile
      if constexpr (!MSE) {
        const long row0 = r0 + 128 * wm + 32 * i;
        const int col0 = c0 + 64 * wn;
        store_residual(sb, hq, lane, rhi, row0, rows - row0, d, col0, col0 < d, col0 + 32 < d);
        store_residual(sb, lq, lane, rlo, row0, rows - row0, d, col0, col0 < d, col0 + 32 < d);
      }
      // row sum over this wave's 64 columns: lanes l and l + 32 share the row
      if constexpr (!MSE) {
        g2 += __shfl_xor(g2, 32);
        if (lane < 32) gsum[wn * WT + vr] = g2;
      }
    };
    row_tile(std::integral_constant<int, 0>{});
    row_tile(std::integral_constant<int, 1>{});
    row_tile(std::integral_constant<int, 2>{});
    row_tile(std::integral_constant<int, 3>{});
    if constexpr (!MSE) {
      __syncthreads();
      if (tid < WT && r0 + tid < rows)
        gpart[size_t(r0 + tid) * nct + ct] =
            gsum[tid] + gsum[WT + tid] + gsum[2 * WT + tid] + gsum[3 * WT + tid];
    }
  } else {
    const int h = lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int vr = 128 * wm + 32 * i + (lane & 31);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int cb = c0 + 64 * wn + 32 * j;
        const bool okc = cb < d;
        const int w = cb / 32;
        uint32_t word = 0u;                      // sign bits of the lane's 16 coordinates
#pragma unroll
        for (int r = 0; r < 16; ++r) word |= uint32_t(acc[i][j][r] >= 0.f) << (8 * (r / 4) + r % 4);
        word <<= 4 * h;
        word |= __shfl_xor(word, 32);
        if (okc && lane < 32 && r0 + vr < rows)
          codes[(size_t(v0 + r0 + vr) * groups + w) * BITS + BITS - 1] = word;
      }
    }
    // gamma = |r'| from the per-column-tile partial sums of phase 1, in column order
    if (ct == 0 && tid < WT && r0 + tid < rows) {
      float g = 0.f;
      for (int t = 0; t < nct; ++t) g += gpart[size_t(r0 + tid) * nct + t];
      gamma_out[v0 + r0 + tid] = sqrtf(g);
    }
  }
}

template <int BITS, bool F32IN>
hipError_t run(const unsigned char* params, const Layout& lay, const void* x, long xpitch, int64_t n,
               uint32_t* codes, float* nu, float* gamma, hipStream_t s, float* u) {
  const int d = lay.d;
  const uint16_t* pih = reinterpret_cast<const uint16_t*>(params + lay.off_gmat);
  const uint16_t* pil = pih + size_t(d) * d;
  const uint16_t* sph = pil + size_t(d) * d;
  const uint16_t* spl = sph + size_t(d) * d;
  const long ch = chunk_rows(n, d, xpitch, F32IN ? 4 : 2);
  const int nct = (d + WT - 1) / WT;
  // scratch: r' hi, r' lo and (float32 input) x hi, x lo, each (chunk rows) x d bf16; then
  // the partial sums of |r'|^2, (chunk rows) x (d / 256) float32
  const size_t plane = size_t(ch) * d;
  const size_t bytes = plane * 2 * (F32IN ? 4 : 2) + size_t(ch) * nct * 4;
  uint16_t* scratch = nullptr;
  hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&scratch), bytes, s);
  if (e != hipSuccess) return e;
  uint16_t* rhi = scratch;
  uint16_t* rlo = rhi + plane;
  uint16_t* xh = F32IN ? rlo + plane : nullptr;
  uint16_t* xl = F32IN ? xh + plane : nullptr;
  float* gpart = reinterpret_cast<float*>(scratch + plane * (F32IN ? 4 : 2));
  for (long c0 = 0; c0 < n; c0 += ch) {
    const long rows = (n - c0) < ch ? (n - c0) : ch;
    const int nrb = int((rows + WT - 1) / WT);
    const dim3 grid(unsigned((nrb + NXCD - 1) / NXCD * NXCD * nct));
    const void* xs = F32IN ? static_cast<const void*>(static_cast<const float*>(x) + size_t(c0) * xpitch)
                           : static_cast<const void*>(static_cast<const uint16_t*>(x) + size_t(c0) * xpitch);
    hipLaunchKernelGGL((qsplit_kernel<F32IN>), dim3(unsigned((rows + 3) / 4)), dim3(256), 0, s, xs,
                       rows, d, xpitch, xh, xl, c0, nu);
    const uint16_t* a1 = F32IN ? xh : static_cast<const uint16_t*>(xs);
    const long ap = F32IN ? long(d) : xpitch;
    if (u)
      hipLaunchKernelGGL((qgemm_kernel<1, BITS, F32IN, true>), grid, dim3(WAVES * 64), 0, s, params, a1, xl,
                         rows, pih, pil, d, ap, c0, nrb, codes, nu, gamma, rhi, rlo, gpart, u);
    else
      hipLaunchKernelGGL((qgemm_kernel<1, BITS, F32IN>), grid, dim3(WAVES * 64), 0, s, params, a1, xl,
                         rows, pih, pil, d, ap, c0, nrb, codes, nu, gamma, rhi, rlo, gpart, nullptr);
    hipLaunchKernelGGL((qgemm_kernel<2, BITS, true>), grid, dim3(WAVES * 64), 0, s, params, rhi, rlo,
                       rows, sph, spl, d, long(d), c0, nrb, codes, nu, gamma, nullptr, nullptr, gpart,
                       nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) break;
  }
  const hipError_t f = hipFreeAsync(scratch, s);
  return e != hipSuccess ? e : f;
}

// The MSE quantizer alone: per chunk the split pass (nu, x hi/lo) and phase 1 without the
// residual.
template <int BITS, bool F32IN>
hipError_t run_mse(const unsigned char* params, const Layout& lay, const void* x, long xpitch,
                   int64_t n, uint32_t* codes, float* nu, hipStream_t s) {
  const int d = lay.d;
  const uint16_t* pih = reinterpret_cast<const uint16_t*>(params + lay.off_gmat);
  const uint16_t* pil = pih + size_t(d) * d;
  const long ch = chunk_rows(n, d, xpitch, 2);
  const int nct = (d + WT - 1) / WT;
  const size_t plane = size_t(ch) * d;
  uint16_t* scratch = nullptr;
  hipError_t e = hipSuccess;
  if (F32IN) {
    e = hipMallocAsync(reinterpret_cast<void**>(&scratch), plane * 2 * 2, s);
    if (e != hipSuccess) return e;
  }
  uint16_t* xh = F32IN ? scratch : nullptr;
  uint16_t* xl = F32IN ? scratch + plane : nullptr;
  for (long c0 = 0; c0 < n; c0 += ch) {
    const long rows = (n - c0) < ch ? (n - c0) : ch;
    const int nrb = int((rows + WT - 1) / WT);
    const dim3 grid(unsigned((nrb + NXCD - 1) / NXCD * NXCD * nct));
    const void* xs = F32IN ? static_cast<const void*>(static_cast<const float*>(x) + size_t(c0) * xpitch)
                           : static_cast<const void*>(static_cast<const uint16_t*>(x) + size_t(c0) * xpitch);
    hipLaunchKernelGGL((qsplit_kernel<F32IN>), dim3(unsigned((rows + 3) / 4)), dim3(256), 0, s, xs,
                       rows, d, xpitch, xh, xl, c0, nu);
    const uint16_t* a1 = F32IN ? xh : static_cast<const uint16_t*>(xs);
    const long ap = F32IN ? long(d) : xpitch;
    hipLaunchKernelGGL((qgemm_kernel<3, BITS, F32IN>), grid, dim3(WAVES * 64), 0, s, params, a1, xl,
                       rows, pih, pil, d, ap, c0, nrb, codes, nu, nullptr, nullptr, nullptr, nullptr,
                       nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) break;
  }
  if (F32IN) {
    const hipError_t f = hipFreeAsync(scratch, s);
    if (e == hipSuccess) e = f;
  }
  return e;
}

}  // namespace

hipError_t launch_quantize_gemm(const void* params_v, int d, int b, const void* x, int x_dtype,
                                int64_t n, uint32_t* codes, float* nu, float* gamma,
                                hipStream_t s, int64_t xpitch, float* u) {
  const unsigned char* params = static_cast<const unsigned char*>(params_v);
  const Layout lay(d, b);
  const bool f32 = x_dtype == 0;
  const long xp = xpitch > 0 ? long(xpitch) : long(d);
  switch (b) {
    case 2: return f32 ? run<2, true>(params, lay, x, xp, n, codes, nu, gamma, s, u)
                       : run<2, false>(params, lay, x, xp, n, codes, nu, gamma, s, u);
    case 3: return f32 ? run<3, true>(params, lay, x, xp, n, codes, nu, gamma, s, u)
                       : run<3, false>(params, lay, x, xp, n, codes, nu, gamma, s, u);
    case 4: return f32 ? run<4, true>(params, lay, x, xp, n, codes, nu, gamma, s, u)
                       : run<4, false>(params, lay, x, xp, n, codes, nu, gamma, s, u);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq

namespace tq {

hipError_t launch_quantize_mse(const void* params_v, int d, int b, const void* x, int x_dtype,
                               int64_t n, uint32_t* codes, float* nu, hipStream_t s,
                               int64_t xpitch) {
  const unsigned char* params = static_cast<const unsigned char*>(params_v);
  const Layout lay(d, b);
  const bool f32 = x_dtype == 0;
  const long xp = xpitch > 0 ? long(xpitch) : long(d);
  switch (b) {
    case 2: return f32 ? run_mse<2, true>(params, lay, x, xp, n, codes, nu, s)
                       : run_mse<2, false>(params, lay, x, xp, n, codes, nu, s);
    case 3: return f32 ? run_mse<3, true>(params, lay, x, xp, n, codes, nu, s)
                       : run_mse<3, false>(params, lay, x, xp, n, codes, nu, s);
    case 4: return f32 ? run_mse<4, true>(params, lay, x, xp, n, codes, nu, s)
                       : run_mse<4, false>(params, lay, x, xp, n, codes, nu, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tq
