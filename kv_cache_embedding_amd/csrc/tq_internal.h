// Internal definitions shared by the host ABI code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tq {

constexpr uint32_t kMagic = 0x51545152u;   // "RQTQ"
constexpr int kMaxLevels = 16;             // up to 4 Lloyd-Max bits in the parameter block

// Header at offset 0 of the device parameter block (256 bytes, read by the kernels).
struct Header {
  uint32_t magic;
  int32_t d, b, L;            // dimension, total bits, Lloyd-Max levels = 2^(b-1)
  float thr[kMaxLevels];      // thresholds[L-1] in units of the rotated unit vector
  float cen[kMaxLevels];      // centroids[L]
  float tpos[kMaxLevels / 2]; // positive thresholds thr[L/2 .. L-2] (thr[L/2-1] == 0)
  float mpos[kMaxLevels / 2]; // positive centroids cen[L/2 .. L-1]
  // Walsh expansion of the codebook on the index bits (odd terms only):
  //   cen[idx] = sum_P e[P] * prod_{p in P} (2 bit_p(idx) - 1)
  // ordered as the scoring kernel walks its bit planes: {b0}, {b1}, {b2}, {b0 b1 b2}.
  float e[4];
  int32_t ne;                 // number of Walsh terms used (1, 2 or 4)
  float esum;                 // sum of e[]
  float emax;                 // max |e|
  float alpha;                // QJL scale: sqrt(pi/2) / m (Gaussian S), 1 / (m E|w_1|) (orthonormal rows)
  float pad[4];
};
static_assert(sizeof(Header) <= 256, "header must fit in 256 bytes");

// Byte layout of the device parameter block for (d, b).
struct Layout {
  int d = 0, b = 0;
  size_t off_hdr = 0;
  size_t off_pi = 0;      // Pi  [d][d] fp32 row-major
  size_t off_s = 0;       // S   [d][d] fp32 row-major
  size_t off_qfrag = 0;   // d == 128: quantize MFMA fragments (2 x 64 KiB), else 0 bytes
  size_t qfrag_bytes = 0;
  size_t off_gmat = 0;    // bf16 Pi_hi, Pi_lo, S'_hi, S'_lo [d][d] (tiled encoders, every d)
  size_t gmat_bytes = 0;
  size_t off_tr = 0;      // d == 128: Pi^T and S^T fp32 [2][d][d] (column k of Pi at k * d)
  size_t tr_bytes = 0;
  size_t total = 0;
  Layout(int d_, int b_);
};

constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline Layout::Layout(int d_, int b_) : d(d_), b(b_) {
  off_hdr = 0;
  off_pi = 256;
  off_s = align256(off_pi + size_t(d) * d * 4);
  off_qfrag = align256(off_s + size_t(d) * d * 4);
  qfrag_bytes = (d == 128) ? size_t(2) * 64 * 1024 : 0;
  off_gmat = align256(off_qfrag + qfrag_bytes);
  gmat_bytes = size_t(4) * d * d * 2;
  off_tr = align256(off_gmat + gmat_bytes);
  tr_bytes = (d == 128) ? size_t(2) * d * d * 4 : 0;
  total = align256(off_tr + tr_bytes);
}

// Plane words per key that the scoring kernel feeds to the MFMA: the b-1 index planes,
// the derived xor plane for 3 index bits, and the QJL sign plane.
constexpr int score_words(int b) { return b == 4 ? 5 : b; }

// Score workspace: per group, the MFMA query operands and 4 floats per query.
constexpr size_t score_ws_per_group(int b) {
  return size_t(2 * score_words(b)) * 64 * 16 + 4 * 4 * 4;
}

// Split scoring workspace (a key split 64 + 64 of d = 128) per quad of query heads: group 0's
// NW0 MFMA operand registers (64 lanes x 16 bytes each), group 1's NW1, then float4 constants
// [group][head] (l_g = nu_g (x s_mse - y + gamma_g (z s_qjl - w))).
constexpr size_t score_split_ws_per_group(int b0, int b1) {
  return size_t(score_words(b0) + score_words(b1)) * 64 * 16 + size_t(2) * 4 * 16;
}

// Sets the calling thread's tq_last_error() text and returns status (host.cpp).
int report_error(int status, const char* message);

// ---- kernel launchers (defined in the .hip files), return hipError_t
hipError_t launch_quantize_d128(const void* params, int b, const void* x, int x_dtype, int64_t n,
                                uint32_t* codes, float* nu, float* gamma, hipStream_t s);
// The same encoder, also writing u = Pi x / nu ([n][128] float32) from its accumulators.
hipError_t launch_quantize_d128_u(const void* params, int b, const void* x, int x_dtype, int64_t n,
                                  uint32_t* codes, float* nu, float* gamma, float* u, hipStream_t s);
// Fused d = 128 encoder on two 64-channel groups (each its own d = 64 parameter block);
// mse: the MSE quantizer alone (b - 1 index planes per group, no gamma).
hipError_t launch_quantize_d128_split(const void* params0, const void* params1, int b0, int b1,
                                      const void* x, int x_dtype, int64_t n, uint32_t* codes0,
                                      float* nu0, float* gamma0, uint32_t* codes1, float* nu1,
                                      float* gamma1, hipStream_t s, bool mse = false);
// Tiled encoder, any valid d.  xpitch: elements between input rows (0: d), so that a
// channel group of wider rows is read in place.  u (optional): also write u = Pi x / nu
// ([n][d] float32) from phase 1's accumulators.
hipError_t launch_quantize_gemm(const void* params, int d, int b, const void* x, int x_dtype,
                                int64_t n, uint32_t* codes, float* nu, float* gamma,
                                hipStream_t s, int64_t xpitch = 0, float* u = nullptr);
// Scoring in two phases: kScorePrep writes the query operands into ws (needs q), kScoreScan
// scores the keys from them (needs codes, nu, gamma, logits); tq_score_ip runs both.
constexpr int kScorePrep = 1, kScoreScan = 2, kScoreBoth = 3;
hipError_t launch_score_d128(const void* params, int b, const void* q, int q_dtype,
                             const uint32_t* codes, const float* nu, const float* gamma,
                             int64_t groups, int64_t G, int64_t T, int mode, float* logits,
                             void* ws, hipStream_t s, int phases = kScoreBoth);
// Scoring for shapes the d = 128 kernel does not take (any d, any G): fp32 query prep into
// ws ([groups * G][2][d] floats: Pi q, S q), then one lane per key.  qpitch:
// elements between query rows (0: d).
hipError_t launch_score_generic(const void* params, int d, int b, const void* q, int q_dtype,
                                const uint32_t* codes, const float* nu, const float* gamma,
                                int64_t groups, int64_t G, int64_t T, int mode, float* logits,
                                void* ws, hipStream_t s, int64_t qpitch = 0,
                                int phases = kScoreBoth);
size_t score_generic_ws_bytes(int d, int64_t groups, int64_t G);
// Two channel groups (coordinates 0..d0-1 and d0..d0+d1-1 of the query rows, each group its
// own parameter block and codes): one query prep launch for both (group 1's operands at
// align256 of group 0's in ws), one scoring pass that sums the groups' estimates per key.
hipError_t launch_score_generic_split(const void* params0, const void* params1, int d0, int d1, int b0,
                                      int b1, const void* q, int q_dtype, const uint32_t* codes0,
                                      const float* nu0, const float* gamma0, const uint32_t* codes1,
                                      const float* nu1, const float* gamma1, int64_t groups, int64_t G,
                                      int64_t T, int mode, float* logits, void* ws, hipStream_t s,
                                      int phases = kScoreBoth);
size_t score_generic_split_ws_bytes(int d0, int d1, int64_t groups, int64_t G);
// The 64 + 64 split of d = 128 with G a multiple of 4 on the d = 128 integer scorer: one query
// prep launch writing both groups' operands, one scan summing the groups' estimates per key.
// applies: the shape (d = 128, d0 = 64, G a multiple of 4, both b in 2..4) and T (buffer
// offsets within 2^31); shape alone: what the query prep alone can decide.
bool score_split_d128_shape(int d, int d0, int b0, int b1, int64_t G);
bool score_split_d128_applies(int d, int d0, int b0, int b1, int64_t G, int64_t T);
size_t score_split_d128_ws_bytes(int b0, int b1, int64_t groups, int64_t G);
hipError_t launch_score_split_d128(const void* params0, const void* params1, int b0, int b1, const void* q,
                                   int q_dtype, const uint32_t* codes0, const float* nu0, const float* gamma0,
                                   const uint32_t* codes1, const float* nu1, const float* gamma1,
                                   int64_t groups, int64_t G, int64_t T, int mode, float* logits, void* ws,
                                   hipStream_t s, int phases = kScoreBoth);
bool score_generic_grid_fits(int64_t groups, int64_t G, int64_t T);
// The MSE stage alone (b-1 index planes and nu): d = 128 on the fused encoder without its
// GEMM2, every other d on the tiled encoder's phase 1.
hipError_t launch_quantize_d128_mse(const void* params, int b, const void* x, int x_dtype,
                                    int64_t n, uint32_t* codes, float* nu, hipStream_t s);
hipError_t launch_quantize_mse(const void* params, int d, int b, const void* x, int x_dtype,
                               int64_t n, uint32_t* codes, float* nu, hipStream_t s,
                               int64_t xpitch = 0);
// Decode attention after the logits: block partials of the softmax-weighted value sum, then
// their merge and the inverse rotation.
size_t attention_part_bytes(int d, int64_t groups, int64_t G, int64_t T);
bool attention_grid_fits(int64_t groups, int64_t G, int64_t T);
hipError_t launch_attention_values(const void* params_v, int d, int b_v, const float* logits,
                                   const uint32_t* vcodes, const float* vnu, int64_t groups,
                                   int64_t G, int64_t T, float scale, float* out, void* part,
                                   hipStream_t s, int64_t opitch = 0);
// d = 128 keys and values with G a multiple of 4: the block partials with each block's logits
// computed in the block kernel from the query operands that the d = 128 scorer's query prep
// wrote to qws (no logits in memory), then the merge.
hipError_t launch_attention_fused(const void* params_v, int b_k, bool prod, const uint32_t* codes_k,
                                  const float* nu_k, const float* gamma_k, const void* qws, int b_v,
                                  const uint32_t* vcodes, const float* vnu, int64_t groups, int64_t G,
                                  int64_t T, float scale, float* out, void* part, hipStream_t s);
// Two value channel groups (output columns 0..d0-1 and d0..d0+d1-1): the block partials of
// each group (group 1's at align256(attention_part_bytes(d0, ...)) in part), then one merge
// launch for both.
hipError_t launch_attention_values_split(const void* params_v0, const void* params_v1, int d0, int d1,
                                         int bv0, int bv1, const float* logits,
                                         const uint32_t* vcodes0, const float* vnu0,
                                         const uint32_t* vcodes1, const float* vnu1, int64_t groups,
                                         int64_t G, int64_t T, float scale, float* out, void* part,
                                         hipStream_t s);
// A 64 + 64 split of d = 128 keys (inner-product estimate) and values with G a multiple of 4:
// the block partials with each block's logits computed in the block kernel from the query
// operands that the split scorer's query prep wrote to qws (no logits in memory), then one
// merge of both value groups (partials of group 1 at align256(attention_part_bytes(64, ...))).
// applies: the bit pairs with a kernel (each group 0 count equal to group 1's or one above).
bool attention_fused_split_applies(int bk0, int bk1, int bv0, int bv1);
hipError_t launch_attention_fused_split(const void* params_v0, const void* params_v1, int bk0, int bk1,
                                        const uint32_t* codes_k0, const float* nu_k0, const float* gamma_k0,
                                        const uint32_t* codes_k1, const float* nu_k1, const float* gamma_k1,
                                        const void* qws, int bv0, int bv1, const uint32_t* vcodes0,
                                        const float* vnu0, const uint32_t* vcodes1, const float* vnu1,
                                        int64_t groups, int64_t G, int64_t T, float scale, float* out, void* part,
                                        hipStream_t s);
// Cache append: copies vector g's words, nu and gamma (gamma may be NULL) of a contiguous
// batch to slot (g, pos) of [groups][cap] caches.
hipError_t launch_scatter_slot(const uint32_t* src_codes, const float* src_nu,
                               const float* src_gamma, int words, int64_t groups, int64_t cap,
                               int64_t pos, uint32_t* codes, float* nu, float* gamma,
                               hipStream_t s);
hipError_t launch_dequantize(const void* params, int d, int b, const uint32_t* codes,
                             const float* nu, const float* gamma, int64_t n, int mode,
                             float* xhat, hipStream_t s);
hipError_t launch_topk(const void* params, int d, int b, const void* q, int q_dtype, int64_t nq,
                       const uint32_t* codes, const float* nu, const float* gamma, int64_t n,
                       int k, int mode, int32_t* idx, float* score, void* ws, hipStream_t s);
size_t topk_ws_bytes(int d, int b, int64_t nq, int64_t n, int k);
// k beyond the fused scan's lists: batches of queries scored by the general path, then
// one selection workgroup per query
hipError_t launch_topk_large(const void* params, int d, int b, const void* q, int q_dtype,
                             int64_t nq, const uint32_t* codes, const float* nu, const float* gamma,
                             int64_t n, int k, int mode, int32_t* idx, float* score, void* ws,
                             hipStream_t s);
size_t topk_large_ws_bytes(int d, int64_t nq, int64_t n);

// Compute units of the current device (looked up once per process; 256 if the query fails).
inline int device_cu_count() {
  static int cached = 0;
  if (!cached) {
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      c = 256;
    cached = c;
  }
  return cached;
}

// vmcnt-only s_waitcnt immediate for gfx9 (expcnt and lgkmcnt left unconstrained).  Direct
// global -> LDS loads count in vmcnt, and the compiler does not order later LDS reads after
// them: kernels that use them wait explicitly.
constexpr int vmcnt_only(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 3) << 14); }

}  // namespace tq
