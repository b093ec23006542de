// Flat-scan top-k search over TurboQuant codes ([news, vector-search paragraph]: the index
// is the codes themselves, so there is nothing to build).
//
// Score of query a against key j ([review, problem statement]; [explainer, step 2]):
//   l_aj = nu_j (<Pi q_a, chat_j> + alpha gamma_j <S q_a, 2 z_j - 1>)
//        = < [Pi q_a | S q_a], [nu_j chat_j | nu_j alpha gamma_j (2 z_j - 1)] >,
// a dense contraction over K = 2d once the per-key scalars are folded into the key side.
// Many queries share every key, so the keys are dequantized once per chunk into fp16 rows
// K~ = [nu chat | nu alpha gamma (2z - 1)] and scored on v_mfma_f32_32x32x16_f16 against
// Q~ = [Pi q | S q] (fp16; float32 accumulation).  The epilogue of every 128 x 128 score
// tile updates per-query running top-k lists held in LDS, so the nq x n score matrix is
// never written; a last kernel merges the lists of all key ranges.
// Order: decreasing score, equal scores by increasing key index.
#include "tq_internal.h"

#include <cfloat>

namespace tq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;            // queries per tile
constexpr int BN = 128;            // keys per tile
constexpr int BK = 32;             // K step
constexpr int KMAX = 32;           // largest k held in the per-tile lists
constexpr int TILES_PER_WG = 16;   // key tiles per workgroup (2048 keys)
constexpr int KEYS_PER_WG = BN * TILES_PER_WG;
constexpr long CHUNK = 65536;      // keys dequantized per pass
constexpr int LDA = BK + 8;        // padded LDS row (halves) of the A / B staging tiles
constexpr int LDS_ROW = BN + 1;    // padded score-tile row (floats)

struct Plan {
  long nq, n, chunk, chunks, splits_total, qtiles;
  size_t off_q, off_k, off_cand, total;
};

Plan plan(int d, int64_t nq, int64_t n, int k) {
  Plan p;
  p.nq = nq;
  p.n = n;
  p.chunk = n < CHUNK ? n : CHUNK;
  p.chunks = (n + p.chunk - 1) / p.chunk;
  p.splits_total = 0;
  for (long c = 0; c < p.chunks; ++c) {
    const long len = (c + 1) * p.chunk <= n ? p.chunk : n - c * p.chunk;
    p.splits_total += (len + KEYS_PER_WG - 1) / KEYS_PER_WG;
  }
  p.qtiles = (nq + BM - 1) / BM;
  p.off_q = 0;
  p.off_k = align256(size_t(nq) * 2 * d * 2);
  p.off_cand = p.off_k + align256(size_t(p.chunk) * 2 * d * 2);
  p.total = p.off_cand + align256(size_t(nq) * p.splits_total * k * 8);
  (void)k;
  return p;
}

// ------------------------------------------------------------------ query operands
// Q~[a] = [Pi q_a | S q_a] in fp16; QPW queries per workgroup share each row of Pi and S
// (QPW = 8, or 4 when 8 query rows would not fit in 64 KiB of LDS).
template <int QPW>
__global__ __launch_bounds__(256) void topk_qprep_kernel(const unsigned char* __restrict__ params,
                                                          size_t off_pi, size_t off_s, int d,
                                                          const void* __restrict__ q, int q_f32,
                                                          long nq, _Float16* __restrict__ qt) {
  extern __shared__ float qs[];     // [QPW][d]
  const long a0 = long(blockIdx.x) * QPW;
  for (int i = threadIdx.x; i < QPW * d; i += blockDim.x) {
    const long a = a0 + i / d;
    float v = 0.f;
    if (a < nq) {
      const long off = a * d + i % d;
      v = q_f32 ? static_cast<const float*>(q)[off]
                : __uint_as_float(uint32_t(static_cast<const uint16_t*>(q)[off]) << 16);
    }
    qs[i] = v;
  }
  __syncthreads();
  for (int row = threadIdx.x; row < 2 * d; row += blockDim.x) {
    const float* m = reinterpret_cast<const float*>(params + (row < d ? off_pi : off_s)) +
                     size_t(row % d) * d;
    float acc[QPW];
#pragma unroll
    for (int j = 0; j < QPW; ++j) acc[j] = 0.f;
    for (int t = 0; t < d; t += 4) {
      const float4 w = *reinterpret_cast<const float4*>(m + t);
#pragma unroll
      for (int j = 0; j < QPW; ++j) {
        const float* qq = qs + j * d + t;
        acc[j] = fmaf(w.x, qq[0], fmaf(w.y, qq[1], fmaf(w.z, qq[2], fmaf(w.w, qq[3], acc[j]))));
      }
    }
#pragma unroll
    for (int j = 0; j < QPW; ++j)
      if (a0 + j < nq) qt[(a0 + j) * 2 * d + row] = (_Float16)acc[j];
  }
}

// ---------------------------------------------------------------- key operands (chunk)
// K~[j] = [nu chat | nu alpha gamma (2z - 1)] (the second half is 0 for the MSE estimate).
__global__ __launch_bounds__(256) void topk_keys_kernel(const unsigned char* __restrict__ params,
                                                         int d, int b,
                                                         const uint32_t* __restrict__ codes,
                                                         const float* __restrict__ nu,
                                                         const float* __restrict__ gamma, long j0,
                                                         long len, int prod,
                                                         _Float16* __restrict__ kt) {
  const Header* hdr = reinterpret_cast<const Header*>(params);
  const int groups = d / 32;
  const long item = long(blockIdx.x) * blockDim.x + threadIdx.x;   // (key, group of 32)
  if (item >= len * groups) return;
  const long jl = item / groups;
  const int w = int(item % groups);
  const long j = j0 + jl;
  const uint32_t* cw = codes + (size_t(j) * groups + w) * b;
  uint32_t pl[4] = {0, 0, 0, 0};
  for (int p = 0; p < b; ++p) pl[p] = cw[p];
  const float nv = nu[j];
  const float sq = prod ? nv * hdr->alpha * gamma[j] : 0.f;
  _Float16* row = kt + size_t(jl) * 2 * d;
  for (int e = 0; e < 32; e += 8) {
    f16x8 cv, sv;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int bit = e + i;
      int idx = 0;
      for (int p = 0; p < b - 1; ++p) idx |= int((pl[p] >> bit) & 1u) << p;
      cv[i] = (_Float16)(nv * hdr->cen[idx]);
      sv[i] = (_Float16)(((pl[b - 1] >> bit) & 1u) ? sq : -sq);
    }
    *reinterpret_cast<f16x8*>(row + 32 * w + e) = cv;
    *reinterpret_cast<f16x8*>(row + d + 32 * w + e) = sv;
  }
}

// --------------------------------------------------------- scores + running top-k
// Workgroup (query tile, key range of TILES_PER_WG tiles): 4 waves, each a 64 x 64 block of
// 2 x 2 32x32 MFMA tiles; A (queries) and B (keys) staged through LDS in BK-wide steps.
__global__ __launch_bounds__(256) void topk_gemm_select_kernel(
    const _Float16* __restrict__ qt, const _Float16* __restrict__ kt, int K2, long nq, long j0,
    long len, int k, long split0, long splits_total, int* __restrict__ cand_idx,
    float* __restrict__ cand_score) {
  __shared__ _Float16 As[BM * LDA];
  __shared__ _Float16 Bs[BN * LDA];
  __shared__ float St[BM * LDS_ROW];
  __shared__ float Ls[BM * KMAX];
  __shared__ int Li[BM * KMAX];
  __shared__ int Lc[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const long qbase = long(blockIdx.x) * BM;
  const long kbeg = long(blockIdx.y) * KEYS_PER_WG;
  const long kend = kbeg + KEYS_PER_WG < len ? kbeg + KEYS_PER_WG : len;
  for (int i = tid; i < BM; i += 256) Lc[i] = 0;

  for (long kt0 = kbeg; kt0 < kend; kt0 += BN) {
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) acc[i][jj] = f32x16{};
    for (int kk = 0; kk < K2; kk += BK) {
      // stage: thread -> (row = tid / 2, 16 halves at column 16 * (tid % 2))
      {
        const int r = tid >> 1, c = (tid & 1) * 16;
        const long qa = qbase + r;
        uint4 va0 = {0, 0, 0, 0}, va1 = {0, 0, 0, 0};
        if (qa < nq) {
          const uint4* src = reinterpret_cast<const uint4*>(qt + size_t(qa) * K2 + kk + c);
          va0 = src[0];
          va1 = src[1];
        }
        const long kj = kt0 + r;
        uint4 vb0 = {0, 0, 0, 0}, vb1 = {0, 0, 0, 0};
        if (kj < kend) {
          const uint4* src = reinterpret_cast<const uint4*>(kt + size_t(kj) * K2 + kk + c);
          vb0 = src[0];
          vb1 = src[1];
        }
        __syncthreads();   // previous step's fragments are consumed
        *reinterpret_cast<uint4*>(&As[r * LDA + c]) = va0;
        *reinterpret_cast<uint4*>(&As[r * LDA + c + 8]) = va1;
        *reinterpret_cast<uint4*>(&Bs[r * LDA + c]) = vb0;
        *reinterpret_cast<uint4*>(&Bs[r * LDA + c + 8]) = vb1;
        __syncthreads();
      }
#pragma unroll
      for (int ks = 0; ks < BK; ks += 16) {
        f16x8 af[2], bf[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          af[i] = *reinterpret_cast<const f16x8*>(&As[(wm + 32 * i + (lane & 31)) * LDA + ks + 8 * (lane >> 5)]);
          bf[i] = *reinterpret_cast<const f16x8*>(&Bs[(wn + 32 * i + (lane & 31)) * LDA + ks + 8 * (lane >> 5)]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
            acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[jj], acc[i][jj], 0, 0, 0);
      }
    }
    // scores to LDS: accumulator register r of lane l holds row 8(r/4) + 4(l/32) + r%4,
    // column l % 32 of its 32x32 tile
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm + 32 * i + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
          const int col = wn + 32 * jj + (lane & 31);
          St[row * LDS_ROW + col] = acc[i][jj][r];
        }
    __syncthreads();
    // running top-k of each query over this tile, keys in increasing index order
    if (tid < BM && qbase + tid < nq) {
      float* ls = Ls + tid * KMAX;
      int* li = Li + tid * KMAX;
      int cnt = Lc[tid];
      const int nk = int(kend - kt0 < BN ? kend - kt0 : BN);
      for (int c = 0; c < nk; ++c) {
        const float s = St[tid * LDS_ROW + c];
        if (cnt == k && !(s > ls[k - 1])) continue;
        int pos = cnt < k ? cnt : k - 1;
        while (pos > 0 && ls[pos - 1] < s) {
          ls[pos] = ls[pos - 1];
          li[pos] = li[pos - 1];
          --pos;
        }
        ls[pos] = s;
        li[pos] = int(j0 + kt0 + c);
        if (cnt < k) ++cnt;
      }
      Lc[tid] = cnt;
    }
    __syncthreads();
  }
  if (tid < BM && qbase + tid < nq) {
    const long split = split0 + blockIdx.y;
    const size_t base = (size_t(qbase + tid) * splits_total + split) * k;
    const int cnt = Lc[tid];
    for (int e = 0; e < k; ++e) {
      cand_score[base + e] = e < cnt ? Ls[tid * KMAX + e] : -FLT_MAX;
      cand_idx[base + e] = e < cnt ? Li[tid * KMAX + e] : -1;
    }
  }
}

// ------------------------------------------------------------------ final merge
// One workgroup per query: k rounds of a block-wide arg-max over the candidate lists
// (larger score first, then smaller index; empty slots carry index -1 and lose).
__device__ __forceinline__ bool better(float s1, int i1, float s2, int i2) {
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
      if (better(s, i, bs, bi)) {
        bs = s;
        bi = i;
        bp = p;
      }
    }
    rs[threadIdx.x] = bs;
    ri[threadIdx.x] = bi;
    rp[threadIdx.x] = bp;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
      if (threadIdx.x < h && better(rs[threadIdx.x + h], ri[threadIdx.x + h], rs[threadIdx.x], ri[threadIdx.x])) {
        rs[threadIdx.x] = rs[threadIdx.x + h];
        ri[threadIdx.x] = ri[threadIdx.x + h];
        rp[threadIdx.x] = rp[threadIdx.x + h];
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

}  // namespace

size_t topk_ws_bytes(int d, int b, int64_t nq, int64_t n, int k) {
  (void)b;
  return plan(d, nq, n, k).total;
}

hipError_t launch_topk(const void* params_v, int d, int b, const void* q, int q_dtype, int64_t nq,
                       const uint32_t* codes, const float* nu, const float* gamma, int64_t n,
                       int k, int mode, int32_t* idx, float* score, void* ws, hipStream_t s) {
  if (k > KMAX || (2 * d) % BK != 0) return hipErrorNotSupported;
  const unsigned char* params = static_cast<const unsigned char*>(params_v);
  const Layout lay(d, b);
  const Plan p = plan(d, nq, n, k);
  unsigned char* w = static_cast<unsigned char*>(ws);
  _Float16* qt = reinterpret_cast<_Float16*>(w + p.off_q);
  _Float16* kt = reinterpret_cast<_Float16*>(w + p.off_k);
  int* cand_idx = reinterpret_cast<int*>(w + p.off_cand);
  float* cand_score = reinterpret_cast<float*>(w + p.off_cand + size_t(nq) * p.splits_total * k * 4);
  const int K2 = 2 * d;

  if (size_t(8) * d * 4 <= 65536)
    hipLaunchKernelGGL((topk_qprep_kernel<8>), dim3(unsigned((nq + 7) / 8)), dim3(256),
                       size_t(8) * d * 4, s, params, lay.off_pi, lay.off_s, d, q,
                       q_dtype == 0 ? 1 : 0, long(nq), qt);
  else
    hipLaunchKernelGGL((topk_qprep_kernel<4>), dim3(unsigned((nq + 3) / 4)), dim3(256),
                       size_t(4) * d * 4, s, params, lay.off_pi, lay.off_s, d, q,
                       q_dtype == 0 ? 1 : 0, long(nq), qt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  long split0 = 0;
  for (long c = 0; c < p.chunks; ++c) {
    const long j0 = c * p.chunk;
    const long len = j0 + p.chunk <= n ? p.chunk : n - j0;
    const long items = len * (d / 32);
    hipLaunchKernelGGL(topk_keys_kernel, dim3(unsigned((items + 255) / 256)), dim3(256), 0, s,
                       params, d, b, codes, nu, gamma, j0, len, mode == 0 ? 1 : 0, kt);
    const long splits = (len + KEYS_PER_WG - 1) / KEYS_PER_WG;
    hipLaunchKernelGGL(topk_gemm_select_kernel, dim3(unsigned(p.qtiles), unsigned(splits)), dim3(256),
                       0, s, qt, kt, K2, long(nq), j0, len, k, split0, p.splits_total, cand_idx,
                       cand_score);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    split0 += splits;
  }
  hipLaunchKernelGGL(topk_merge_kernel, dim3(unsigned(nq)), dim3(256), 0, s, cand_idx, cand_score,
                     long(p.splits_total) * k, k, idx, score);
  return hipGetLastError();
}

}  // namespace tq
