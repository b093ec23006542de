// Host-side driver of libtq's C ABI for the sanitizer build (AddressSanitizer +
// UndefinedBehaviorSanitizer on the host code; no kernel runs).  Exercises the float64
// codebooks, the parameter-block construction of tq_prepare (operand splits, MFMA fragment
// layouts, S' = S Pi^T, Gram checks) and the argument validation of every entry point.  With
// no GPU present the parameter copy fails with TQ_EHIP after the host work is done; with a GPU
// the block goes to real device memory.  Prints "ok" and exits 0 when every expectation holds.
#include "tq.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);   \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

// A random signed permutation: orthogonal exactly in float32.
static std::vector<float> signed_permutation(int d, std::mt19937& g) {
  std::vector<int> p(d);
  for (int i = 0; i < d; ++i) p[i] = i;
  std::shuffle(p.begin(), p.end(), g);
  std::vector<float> m(size_t(d) * d, 0.f);
  for (int i = 0; i < d; ++i) m[size_t(i) * d + p[i]] = (g() & 1) ? 1.f : -1.f;
  return m;
}

int main() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) ndev = 0;

  // codebooks: every bit count at several d, ascending, odd-symmetric, midpoint thresholds
  for (int bits = 1; bits <= 8; ++bits)
    for (int d : {1, 2, 3, 64, 128, 1536, 4096}) {
      const int L = 1 << bits;
      std::vector<double> c(L), t(L - 1 > 0 ? L - 1 : 1);
      EXPECT(tq_codebook_build(bits, d, c.data(), t.data()) == TQ_OK);
      for (int i = 0; i + 1 < L; ++i) {
        EXPECT(c[i] < c[i + 1]);
        EXPECT(std::fabs(t[i] - 0.5 * (c[i] + c[i + 1])) < 1e-15);
      }
      for (int i = 0; i < L; ++i) EXPECT(std::fabs(c[i] + c[L - 1 - i]) < 1e-14);
    }
  for (int bits = 1; bits <= 6; ++bits)
    for (int d : {2, 3, 16, 128, 1536}) {
      const int L = 1 << bits;
      std::vector<double> c(L), t(L > 1 ? L - 1 : 1);
      EXPECT(tq_codebook_build_sphere(bits, d, c.data(), t.data()) == TQ_OK);
      for (int i = 0; i + 1 < L; ++i) EXPECT(c[i] < c[i + 1]);
    }
  {
    double c[4], t[3];
    EXPECT(tq_codebook_build(0, 128, c, t) == TQ_EINVAL);
    EXPECT(tq_codebook_build(9, 128, c, t) == TQ_EINVAL);
    EXPECT(tq_codebook_build(2, 0, c, t) == TQ_EINVAL);
    EXPECT(tq_codebook_build(2, 128, nullptr, t) == TQ_EINVAL);
    EXPECT(tq_codebook_build_sphere(2, 1, c, t) == TQ_EINVAL);
  }

  // sizes of every valid shape, and invalid ones
  for (int d = 64; d <= 4096; d += 64)
    for (int b = 2; b <= 4; ++b) {
      EXPECT(tq_params_bytes(d, b) >= size_t(d) * d * 8);
      EXPECT(tq_score_ws_bytes(d, b, 3, 5, 100) > 0);
      EXPECT(tq_topk_ws_bytes(d, b, 7, 1000, 10) > 0);
      EXPECT(tq_append_ws_bytes(d, b, 9) > 0);
      EXPECT(tq_attention_ws_bytes(d, b, 2, 4, 77) > 0);
    }
  EXPECT(tq_params_bytes(100, 4) == 0);
  EXPECT(tq_params_bytes(128, 5) == 0);
  EXPECT(tq_params_bytes(4160, 4) == 0);

  // parameter blocks: the whole host construction for d = 64, 128 (fused-encoder fragments,
  // transposed copies), 192 and 1536 (tiled-encoder splits), Gaussian and orthogonal S
  std::mt19937 g(12345);
  for (int d : {64, 128, 192, 1536})
    for (int b = 2; b <= 4; ++b) {
      const int L = 1 << (b - 1);
      std::vector<double> c(L), t(L - 1);
      EXPECT(tq_codebook_build(b - 1, d, c.data(), t.data()) == TQ_OK);
      std::vector<float> Pi = signed_permutation(d, g), So = signed_permutation(d, g);
      std::normal_distribution<float> nd;
      std::vector<float> S(size_t(d) * d);
      for (auto& v : S) v = nd(g);
      void* params = reinterpret_cast<void*>(uintptr_t(1) << 40);   // never dereferenced on the host
      if (ndev > 0 && hipMalloc(&params, tq_params_bytes(d, b)) != hipSuccess) params = nullptr;
      const int want = ndev > 0 ? TQ_OK : TQ_EHIP;
      EXPECT(tq_prepare(d, b, Pi.data(), S.data(), c.data(), t.data(), params, nullptr) == want);
      EXPECT(tq_prepare_orthogonal_qjl(d, b, Pi.data(), So.data(), c.data(), t.data(), params, nullptr) == want);
      // Gaussian S is not orthonormal; a non-orthogonal Pi and bad codebooks are refused
      EXPECT(tq_prepare_orthogonal_qjl(d, b, Pi.data(), S.data(), c.data(), t.data(), params, nullptr) == TQ_EINVAL);
      EXPECT(tq_prepare(d, b, S.data(), S.data(), c.data(), t.data(), params, nullptr) == TQ_EINVAL);
      std::vector<double> bad = c;
      bad[0] *= 1.5;
      EXPECT(tq_prepare(d, b, Pi.data(), S.data(), bad.data(), t.data(), params, nullptr) == TQ_EINVAL);
      EXPECT(tq_prepare(d, b, Pi.data(), S.data(), c.data(), t.data(),
                        static_cast<char*>(params) + 16, nullptr) == TQ_EINVAL);
      if (ndev > 0) (void)hipFree(params);
    }

  // validation of the device entry points: every case fails before any device access
  void* f = reinterpret_cast<void*>(uintptr_t(1) << 40);
  void* odd = reinterpret_cast<void*>((uintptr_t(1) << 40) + 4);
  uint32_t* fc = static_cast<uint32_t*>(f);
  float* ff = static_cast<float*>(f);
  EXPECT(tq_quantize(f, 100, 4, f, TQ_BF16, 10, fc, ff, ff, nullptr) == TQ_EINVAL);
  EXPECT(tq_quantize(f, 128, 4, f, 7, 10, fc, ff, ff, nullptr) == TQ_EINVAL);
  EXPECT(tq_quantize(f, 128, 4, odd, TQ_BF16, 10, fc, ff, ff, nullptr) == TQ_EINVAL);
  EXPECT(tq_quantize(nullptr, 128, 4, nullptr, TQ_BF16, 0, nullptr, nullptr, nullptr, nullptr) == TQ_OK);
  EXPECT(tq_quantize_with_rotation(f, 128, 4, f, TQ_BF16, 10, fc, ff, ff, static_cast<float*>(odd), nullptr) ==
         TQ_EINVAL);
  EXPECT(tq_quantize_mse(f, 128, 4, f, TQ_BF16, 10, static_cast<uint32_t*>(odd), ff, nullptr) == TQ_EINVAL);
  EXPECT(tq_dequantize(f, 128, 4, fc, ff, ff, 10, 5, ff, nullptr) == TQ_EINVAL);
  EXPECT(tq_score_ip(f, 128, 4, f, TQ_BF16, fc, ff, ff, 8, 4, 1024, 9, ff, f, 1 << 30, nullptr) == TQ_EINVAL);
  EXPECT(tq_score_ip(f, 128, 4, f, TQ_BF16, fc, ff, ff, 8, 4, 1024, 0, ff, f, 16, nullptr) == TQ_EWORKSPACE);
  EXPECT(tq_score_ip(f, 128, 4, f, TQ_BF16, fc, ff, ff, -1, 4, 1024, 0, ff, f, 16, nullptr) == TQ_EINVAL);
  EXPECT(tq_score_ip_noalloc(f, 128, 4, f, TQ_BF16, fc, ff, ff, 1 << 20, 4, 1024, 0, ff, nullptr) ==
         TQ_EUNSUPPORTED);
  EXPECT(tq_score_noalloc_max_ws_bytes() == (size_t(8) << 20));
  EXPECT(tq_score_prepare(f, 128, 4, f, 7, 8, 4, f, 1 << 30, nullptr) == TQ_EINVAL);
  EXPECT(tq_score_prepare(f, 128, 4, f, TQ_BF16, 8, 4, f, 16, nullptr) == TQ_EWORKSPACE);
  EXPECT(tq_score_prepare(f, 128, 4, f, TQ_BF16, 0, 4, nullptr, 0, nullptr) == TQ_OK);
  EXPECT(tq_score_ip_prepared(f, 128, 4, fc, ff, ff, 8, 4, 1024, 9, ff, f, 1 << 30, nullptr) == TQ_EINVAL);
  EXPECT(tq_score_ip_prepared(f, 128, 4, fc, ff, ff, 8, 4, 1024, 0, ff, f, 16, nullptr) == TQ_EWORKSPACE);
  EXPECT(tq_score_ip_prepared(f, 128, 4, static_cast<uint32_t*>(odd), ff, ff, 8, 4, 1024, 0, ff, f, 1 << 30,
                              nullptr) == TQ_EINVAL);
  EXPECT(tq_score_split_ws_bytes(128, 64, 3, 3, 8, 4, 100) > 0);
  EXPECT(tq_attention_split_ws_bytes(128, 64, 3, 3, 8, 4, 100) > 0);
  EXPECT(tq_topk(f, 128, 4, f, TQ_F32, 10, fc, ff, ff, 100, 0, 0, static_cast<int32_t*>(f), ff, f, 1 << 30,
                 nullptr) == TQ_EINVAL);
  EXPECT(tq_topk(f, 128, 4, f, TQ_F32, 10, fc, ff, ff, 5, 10, 0, static_cast<int32_t*>(f), ff, f, 1 << 30,
                 nullptr) == TQ_EINVAL);
  EXPECT(tq_append(f, 128, 4, TQ_EST_PROD, f, TQ_BF16, 8, 100, 100, fc, ff, ff, f, 1 << 20, nullptr) ==
         TQ_EINVAL);
  EXPECT(tq_attention(f, f, 128, 4, 4, f, TQ_BF16, fc, ff, ff, fc, ff, 8, 4, 0, 0.1f, 0, ff, f, 1 << 30,
                      nullptr) == TQ_EINVAL);
  EXPECT(tq_attention(f, f, 128, 4, 4, f, TQ_BF16, fc, ff, ff, fc, ff, 8, 4, 16, NAN, 0, ff, f, 1 << 30,
                      nullptr) == TQ_EINVAL);
  EXPECT(tq_quantize_split(f, f, 128, 32, 3, 3, f, TQ_BF16, 10, fc, ff, ff, fc, ff, ff, nullptr) == TQ_EINVAL);
  EXPECT(tq_score_ip_split(f, f, 128, 64, 5, 3, f, TQ_BF16, fc, ff, ff, fc, ff, ff, 8, 4, 100, 0, ff, f, 1 << 30,
                           nullptr) == TQ_EINVAL);
  EXPECT(tq_score_ip_split(f, f, 128, 64, 3, 3, f, TQ_BF16, fc, ff, ff, fc, ff, ff, 8, 4, 100, 0, ff, f, 16,
                           nullptr) == TQ_EWORKSPACE);
  EXPECT(tq_score_split_prepare(f, f, 128, 64, 3, 3, f, 7, 8, 4, f, 1 << 30, nullptr) == TQ_EINVAL);
  EXPECT(tq_score_split_prepare(f, f, 128, 64, 3, 3, f, TQ_BF16, 8, 4, f, 16, nullptr) == TQ_EWORKSPACE);
  EXPECT(tq_score_split_prepare(f, f, 192, 64, 3, 3, f, TQ_BF16, 8, 5, f, 16, nullptr) == TQ_EWORKSPACE);
  EXPECT(tq_score_split_prepare(f, f, 128, 64, 3, 3, f, TQ_BF16, 0, 4, nullptr, 0, nullptr) == TQ_OK);
  EXPECT(tq_score_ip_split_prepared(f, f, 128, 64, 3, 3, fc, ff, ff, fc, ff, ff, 8, 4, 100, 9, ff, f, 1 << 30,
                                    nullptr) == TQ_EINVAL);
  EXPECT(tq_score_ip_split_prepared(f, f, 128, 64, 3, 3, fc, ff, ff, fc, ff, ff, 8, 4, 100, 0, ff, f, 16,
                                    nullptr) == TQ_EWORKSPACE);
  EXPECT(tq_score_ip_split_prepared(f, f, 128, 64, 3, 3, fc, ff, ff, fc, ff, ff, 1, 4, int64_t(1) << 26, 0, ff, f,
                                    1 << 30, nullptr) == TQ_EUNSUPPORTED);
  EXPECT(tq_quantize_mse_split(f, f, 128, 64, 3, 3, f, TQ_BF16, 10, static_cast<uint32_t*>(odd), ff, fc, ff,
                               nullptr) == TQ_EINVAL);
  EXPECT(tq_attention_split(f, f, f, f, 128, 64, 4, 3, 4, 4, f, TQ_BF16, fc, ff, ff, fc, ff, ff, fc, ff, fc, ff,
                            8, 4, 0, 0.1f, 0, ff, f, 1 << 30, nullptr) == TQ_EINVAL);
  EXPECT(tq_last_error()[0] != '\0');

  if (failures) {
    std::fprintf(stderr, "%d expectations failed\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
