// Host side of the C ABI: argument validation, the float64 Lloyd-Max codebook, the
// parameter block (operand splits and MFMA fragment layouts), and kernel dispatch.
#include "tq.h"
#include "tq_internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() { return TQ_OK; }

int hip_fail(hipError_t e, const char* what) {
  return fail(TQ_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool valid_shape(int d, int b) {
  return d >= 64 && d <= 4096 && d % 64 == 0 && b >= 2 && b <= 4;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ------------------------------------------------------------------ Lloyd-Max (float64)
// [review, MSE paragraph]: optimal grid by the Max-Lloyd algorithm; [tldr, step 1]: 1-D
// k-means for the known bell-shaped law, solved once.  The quantizer of a symmetric law
// is odd-symmetric, so only the positive half is iterated here: positive centroids
// c_1 < ... < c_H (H = L/2) over cells [t_0 = 0, t_1), ..., [t_{H-1}, end), where
// t_i = (c_i + c_{i+1}) / 2 and c_i is the mean of the law over its cell.  Cell masses and
// first moments are integrated by 8-point Gauss-Legendre on panels no wider than a quarter
// of the law's scale (no differences of nearly equal tail values, so the fixed point is
// resolved to 1e-14 of the scale even with 128 cells a side).

const double kGL8x[4] = {0.1834346424956498, 0.5255324099163290, 0.7966664774136267, 0.9602898564975363};
const double kGL8w[4] = {0.3626837833783620, 0.3137066458778873, 0.2223810344533745, 0.1012285362903763};

// mass += int_a^b w(x) dx, moment += int_a^b w(x) m(x) dx, where dens(x) returns w(x) and
// sets m(x).
template <class Dens>
void gl_cell(double a, double b, double width, Dens dens, double& mass, double& moment) {
  mass = moment = 0.0;
  if (!(b > a)) return;
  const int np = std::max(1, int(std::ceil((b - a) / width)));
  const double h = (b - a) / np;
  for (int p = 0; p < np; ++p) {
    const double mid = a + (p + 0.5) * h;
    for (int k = 0; k < 4; ++k)
      for (int sgn = -1; sgn <= 1; sgn += 2) {
        double m;
        const double w = 0.5 * h * kGL8w[k] * dens(mid + sgn * 0.5 * h * kGL8x[k], m);
        mass += w;
        moment += w * m;
      }
  }
}

// Fixed-point iteration of the positive half: cell(lo, hi, mass, moment) integrates over
// the cell between two thresholds; edge(t) maps a threshold to the integration variable.
template <class Cell, class Edge>
bool lloyd_iterate(std::vector<double>& c, double top, double tol, Cell cell, Edge edge) {
  const int H = int(c.size());
  std::vector<double> t(H + 1);
  for (int it = 0; it < 1000000; ++it) {
    t[0] = edge(0.0);
    for (int i = 1; i < H; ++i) t[i] = edge(0.5 * (c[i - 1] + c[i]));
    t[H] = top;
    double delta = 0.0;
    for (int i = 0; i < H; ++i) {
      double m0, m1;
      cell(t[i], t[i + 1], m0, m1);
      if (!(m0 > 0.0)) return false;
      const double nc = m1 / m0;
      delta = std::fmax(delta, std::fabs(nc - c[i]));
      c[i] = nc;
    }
    if (delta < tol) return true;
  }
  return false;
}

double std_pdf(double t) { return std::exp(-0.5 * t * t) / std::sqrt(2.0 * M_PI); }
double std_upper_tail(double t) { return 0.5 * std::erfc(t / std::sqrt(2.0)); }

// Inverse of std_upper_tail on (0, 1/2], by bisection.
double std_upper_tail_inv(double p) {
  double lo = 0.0, hi = 40.0;
  for (int it = 0; it < 200; ++it) {
    const double mid = 0.5 * (lo + hi);
    (std_upper_tail(mid) > p ? lo : hi) = mid;
  }
  return 0.5 * (lo + hi);
}

// N(0, 1).  Starts from the high-resolution optimum (level density proportional to
// pdf^(1/3): the quantiles of N(0, 3)); the last cell is cut 12 sigma past its threshold,
// where the density has fallen by more than e^-72.  L = 2 has the closed form
// c_1 = sqrt(2/pi).
bool lloyd_max_positive_half(int H, std::vector<double>& c) {
  const int L = 2 * H;
  c.assign(H, 0.0);
  for (int i = 0; i < H; ++i) c[i] = std::sqrt(3.0) * std_upper_tail_inv((H - i - 0.5) / L);
  auto dens = [](double x, double& m) { m = x; return std_pdf(x); };
  auto cell = [&](double lo, double hi, double& m0, double& m1) {
    gl_cell(lo, std::isinf(hi) ? lo + 12.0 : hi, 0.25, dens, m0, m1);
  };
  return lloyd_iterate(c, INFINITY, 1e-14, cell, [](double t) { return t; });
}

// Exact law of a rotated coordinate u of a unit vector in R^d: density proportional to
// (1 - u^2)^((d-3)/2) on (-1, 1) ([explainer, per-component reduction]: its large-d limit is
// N(0, 1/d)).  Integrated in theta = asin(u), where the density becomes cos^(d-2)(theta) and
// the moment weight sin(theta); the normalizer cancels in the centroid.  Past
// theta = sqrt(1600 / (d - 2)) the integrand is below e^-800 and is dropped.
bool lloyd_max_sphere_positive_half(int H, int d, std::vector<double>& c) {
  std::vector<double> g;
  if (!lloyd_max_positive_half(H, g)) return false;
  const double sigma = 1.0 / std::sqrt(double(d));
  c.assign(H, 0.0);
  if (g[H - 1] * sigma < 0.9) {
    for (int i = 0; i < H; ++i) c[i] = g[i] * sigma;   // start at the Gaussian limit
  } else {
    for (int i = 0; i < H; ++i) c[i] = (i + 0.5) / H;  // broad law: start uniform
  }
  const double tmax = d > 2 ? std::fmin(M_PI / 2, std::sqrt(1600.0 / (d - 2))) : M_PI / 2;
  const double width = std::fmin(M_PI / 64, 0.25 * sigma);
  auto dens = [d](double th, double& m) {
    m = std::sin(th);
    return d == 2 ? 1.0 : std::exp((d - 2) * std::log(std::cos(th)));
  };
  auto cell = [&](double lo, double hi, double& m0, double& m1) {
    gl_cell(lo, std::fmin(hi, tmax), width, dens, m0, m1);
  };
  return lloyd_iterate(c, M_PI / 2, 1e-14 * sigma, cell, [](double u) { return std::asin(u); });
}

// ------------------------------------------------------------------ bf16 helpers (host)
uint16_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}
float bf16_to_f32(uint16_t h) {
  uint32_t u = uint32_t(h) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
void split_bf16(double v, uint16_t& hi, uint16_t& lo) {
  hi = bf16_rne(float(v));
  lo = bf16_rne(float(v - double(bf16_to_f32(hi))));
}

double dot(const double* a, const double* b, int n) {
  double s0 = 0, s1 = 0, s2 = 0, s3 = 0;
  int i = 0;
  for (; i + 4 <= n; i += 4) {
    s0 += a[i] * b[i];
    s1 += a[i + 1] * b[i + 1];
    s2 += a[i + 2] * b[i + 2];
    s3 += a[i + 3] * b[i + 3];
  }
  for (; i < n; ++i) s0 += a[i] * b[i];
  return (s0 + s1) + (s2 + s3);
}

// Run f(i) for i in [0, n) on the host cores (used for the d^3 host products at large d).
template <class F>
void parallel_for(int n, F f) {
  const unsigned hw = std::thread::hardware_concurrency();
  const int nt = int(hw == 0 ? 1 : (hw > 16 ? 16 : hw));
  if (n < 64 || nt == 1) {
    for (int i = 0; i < n; ++i) f(i);
    return;
  }
  std::vector<std::thread> th;
  for (int t = 0; t < nt; ++t)
    th.emplace_back([&, t] {
      for (int i = t; i < n; i += nt) f(i);
    });
  for (auto& x : th) x.join();
}

// Output-row permutation of a 32-row MFMA tile: row rho holds canonical coordinate
// 16*((rho>>2)&1) + 4*(rho>>3) + (rho&3) of the tile, so that in the 32x32 accumulator
// layout (row = 8*(r/4) + 4*(lane/32) + r%4) lane half h, register r holds coordinate
// 16h + r.
int row_coord(int rho) { return 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3); }

// Fragments for the fused d = 128 quantize kernel (see quantize.hip for the data flow).
//   Pi fragment [s][mt][pass][lane][e]: Pi[32mt + row_coord(lane%32)][64*(lane/32) + 8s + e]
//   S' fragment [mt][s][pass][lane][e]: S'[32mt + row_coord(lane%32)]
//                                          [32*(s>>1) + 16*(lane/32) + 8*(s&1) + e]
// pass 0 = bf16 high part, pass 1 = bf16 low part (value - high, rounded).
void build_quantize_fragments(const std::vector<double>& Pi, const std::vector<double>& Sp,
                              uint16_t* out) {
  const int D = 128;
  uint16_t* pif = out;
  uint16_t* spf = out + 64 * 1024 / 2;
  for (int s = 0; s < 8; ++s)
    for (int mt = 0; mt < 4; ++mt)
      for (int lane = 0; lane < 64; ++lane)
        for (int e = 0; e < 8; ++e) {
          int row = 32 * mt + row_coord(lane % 32);
          int col = 64 * (lane / 32) + 8 * s + e;
          uint16_t hi, lo;
          split_bf16(Pi[size_t(row) * D + col], hi, lo);
          size_t base = (size_t(s * 4 + mt) * 2) * 64 * 8;
          pif[base + size_t(lane) * 8 + e] = hi;
          pif[base + 64 * 8 + size_t(lane) * 8 + e] = lo;
        }
  for (int mt = 0; mt < 4; ++mt)
    for (int s = 0; s < 8; ++s)
      for (int lane = 0; lane < 64; ++lane)
        for (int e = 0; e < 8; ++e) {
          int row = 32 * mt + row_coord(lane % 32);
          int col = 32 * (s >> 1) + 16 * (lane / 32) + 8 * (s & 1) + e;
          uint16_t hi, lo;
          split_bf16(Sp[size_t(row) * D + col], hi, lo);
          size_t base = (size_t(mt * 8 + s) * 2) * 64 * 8;
          spf[base + size_t(lane) * 8 + e] = hi;
          spf[base + 64 * 8 + size_t(lane) * 8 + e] = lo;
        }
}

}  // namespace

extern "C" {

const char* tq_last_error(void) { return g_last_error.c_str(); }

int tq_codebook_build(int bits_mse, int d, double* centroids, double* thresholds) {
  if (bits_mse < 1 || bits_mse > 8) return fail(TQ_EINVAL, "bits_mse=%d outside 1..8", bits_mse);
  if (d <= 0) return fail(TQ_EINVAL, "d=%d must be positive", d);
  if (!centroids || !thresholds) return fail(TQ_EINVAL, "NULL output pointer");
  const int L = 1 << bits_mse, H = L / 2;
  std::vector<double> c;
  if (!lloyd_max_positive_half(H, c)) return fail(TQ_EINVAL, "Lloyd-Max did not converge");
  const double sigma = 1.0 / std::sqrt(double(d));
  for (int i = 0; i < H; ++i) {
    centroids[H + i] = c[i] * sigma;
    centroids[H - 1 - i] = -c[i] * sigma;
  }
  for (int i = 0; i < L - 1; ++i) thresholds[i] = 0.5 * (centroids[i] + centroids[i + 1]);
  thresholds[H - 1] = 0.0;
  return ok();
}

int tq_codebook_build_sphere(int bits_mse, int d, double* centroids, double* thresholds) {
  if (bits_mse < 1 || bits_mse > 8) return fail(TQ_EINVAL, "bits_mse=%d outside 1..8", bits_mse);
  if (d < 2) return fail(TQ_EINVAL, "d=%d must be at least 2", d);
  if (!centroids || !thresholds) return fail(TQ_EINVAL, "NULL output pointer");
  const int L = 1 << bits_mse, H = L / 2;
  std::vector<double> c;
  if (!lloyd_max_sphere_positive_half(H, d, c)) return fail(TQ_EINVAL, "Lloyd-Max (sphere) did not converge");
  for (int i = 0; i < H; ++i) {
    centroids[H + i] = c[i];
    centroids[H - 1 - i] = -c[i];
  }
  for (int i = 0; i < L - 1; ++i) thresholds[i] = 0.5 * (centroids[i] + centroids[i + 1]);
  thresholds[H - 1] = 0.0;
  return ok();
}

size_t tq_params_bytes(int d, int b) {
  if (!valid_shape(d, b)) return 0;
  return tq::Layout(d, b).total;
}

}  // extern "C"

namespace {

// Largest |M M^T - I| over the rows of a d x d matrix (float64 copy).
double gram_defect(const std::vector<double>& M, int d) {
  std::vector<double> row_worst(d, 0.0);
  parallel_for(d, [&](int i) {
    double w = 0.0;
    for (int j = i; j < d; ++j) {
      double g = dot(&M[size_t(i) * d], &M[size_t(j) * d], d) - (i == j ? 1.0 : 0.0);
      w = std::fmax(w, std::fabs(g));
    }
    row_worst[i] = w;
  });
  double worst = 0.0;
  for (double w : row_worst) worst = std::fmax(worst, w);
  return worst;
}

// s_orthonormal: S has orthonormal rows, else Gaussian entries; sets the QJL scale.
int prepare_params(int d, int b, const float* Pi, const float* S, const double* centroids,
                   const double* thresholds, bool s_orthonormal, void* params, void* stream) {
  if (!valid_shape(d, b)) return fail(TQ_EINVAL, "unsupported shape d=%d b=%d", d, b);
  if (!Pi || !S || !centroids || !thresholds || !params) return fail(TQ_EINVAL, "NULL pointer");
  if (!aligned(params, 256)) return fail(TQ_EINVAL, "params must be 256-byte aligned");
  const int L = 1 << (b - 1);
  double cmax = 0.0;
  for (int i = 0; i < L; ++i) {
    if (!std::isfinite(centroids[i])) return fail(TQ_EINVAL, "non-finite centroid");
    cmax = std::fmax(cmax, std::fabs(centroids[i]));
  }
  for (int i = 0; i < L; ++i)
    if (std::fabs(centroids[i] + centroids[L - 1 - i]) > 1e-12 * cmax)
      return fail(TQ_EINVAL, "codebook is not odd-symmetric (centroid %d)", i);
  for (int i = 0; i + 1 < L; ++i) {
    if (!(centroids[i] < thresholds[i] && thresholds[i] < centroids[i + 1]))
      return fail(TQ_EINVAL, "thresholds must interleave ascending centroids (index %d)", i);
    if (std::fabs(thresholds[i] + thresholds[L - 2 - i]) > 1e-12 * cmax)
      return fail(TQ_EINVAL, "thresholds are not odd-symmetric (index %d)", i);
  }
  const tq::Layout lay(d, b);
  std::vector<unsigned char> blob(lay.total, 0);

  // header
  tq::Header h;
  std::memset(&h, 0, sizeof(h));
  h.magic = tq::kMagic;
  h.d = d;
  h.b = b;
  h.L = L;
  for (int i = 0; i < L - 1; ++i) h.thr[i] = float(thresholds[i]);
  h.thr[L / 2 - 1] = 0.0f;
  for (int i = 0; i < L; ++i) h.cen[i] = float(centroids[i]);
  for (int k = 0; k + L / 2 < L - 1; ++k) h.tpos[k] = float(thresholds[L / 2 + k]);
  for (int k = 0; k < L / 2; ++k) h.mpos[k] = float(centroids[L / 2 + k]);
  // Walsh coefficients over the index bits: e_P = (1/L) sum_idx c_idx prod_{p in P} sigma_p.
  const int B = b - 1;
  auto walsh = [&](unsigned mask) {
    double s = 0.0;
    for (int idx = 0; idx < L; ++idx) {
      double prod = 1.0;
      for (int p = 0; p < B; ++p)
        if (mask & (1u << p)) prod *= ((idx >> p) & 1) ? 1.0 : -1.0;
      s += centroids[idx] * prod;
    }
    return s / L;
  };
  for (unsigned mask = 0; mask < (1u << B); ++mask) {
    int deg = __builtin_popcount(mask);
    if (deg % 2 == 0 && std::fabs(walsh(mask)) > 1e-12 * cmax)
      return fail(TQ_EINVAL, "codebook has an even Walsh term (not odd-symmetric)");
  }
  unsigned order[4] = {1u, 2u, 4u, 7u};
  h.ne = (B == 3) ? 4 : B;
  h.esum = 0.0f;
  h.emax = 0.0f;
  for (int i = 0; i < h.ne; ++i) {
    double e = walsh(order[i]);
    h.e[i] = float(e);
    h.esum += float(e);
    h.emax = std::fmax(h.emax, std::fabs(float(e)));
  }
  // QJL scale ([review, QJL paragraph]; m = d rows): a Gaussian row s has
  // E[sign<s, rho> <s, q>] = sqrt(2/pi) <q, rho>, a uniform unit row E|w_1| <q, rho> with
  // E|w_1| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)); the scale is the reciprocal over m.
  const double mean_abs = std::exp(std::lgamma(0.5 * d) - std::lgamma(0.5 * (d + 1))) / std::sqrt(M_PI);
  h.alpha = s_orthonormal ? float(1.0 / (d * mean_abs)) : float(std::sqrt(M_PI / 2.0) / d);
  std::memcpy(blob.data() + lay.off_hdr, &h, sizeof(h));

  // Pi and S in float32 (row-major), and float64 copies for host products
  std::memcpy(blob.data() + lay.off_pi, Pi, size_t(d) * d * 4);
  std::memcpy(blob.data() + lay.off_s, S, size_t(d) * d * 4);
  if (lay.tr_bytes) {
    // transposed copies: the scoring query prep reads column k of both with one
    // contiguous load per wave
    float* tr = reinterpret_cast<float*>(blob.data() + lay.off_tr);
    for (int i = 0; i < d; ++i)
      for (int k = 0; k < d; ++k) {
        tr[size_t(k) * d + i] = Pi[size_t(i) * d + k];
        tr[size_t(d) * d + size_t(k) * d + i] = S[size_t(i) * d + k];
      }
  }
  std::vector<double> P64(size_t(d) * d), S64(size_t(d) * d);
  for (size_t i = 0; i < P64.size(); ++i) {
    P64[i] = Pi[i];
    S64[i] = S[i];
    if (!std::isfinite(P64[i]) || !std::isfinite(S64[i]))
      return fail(TQ_EINVAL, "non-finite entry in Pi or S");
  }
  // Pi must be orthogonal: the kernels form the residual in the rotated space.
  const double worst = gram_defect(P64, d);
  if (worst > 1e-4) return fail(TQ_EINVAL, "Pi is not orthogonal (max |Pi Pi^T - I| = %g)", worst);
  if (s_orthonormal) {
    const double sw = gram_defect(S64, d);
    if (sw > 1e-4) return fail(TQ_EINVAL, "S rows are not orthonormal (max |S S^T - I| = %g)", sw);
  }

  if (lay.qfrag_bytes || lay.gmat_bytes) {
    // S' = S Pi^T, so that S r = S' (Pi r) for the residual r (rotated-space residual)
    std::vector<double> Sp(size_t(d) * d);
    parallel_for(d, [&](int i) {
      for (int k = 0; k < d; ++k) Sp[size_t(i) * d + k] = dot(&S64[size_t(i) * d], &P64[size_t(k) * d], d);
    });
    if (lay.qfrag_bytes)
      build_quantize_fragments(P64, Sp, reinterpret_cast<uint16_t*>(blob.data() + lay.off_qfrag));
    if (lay.gmat_bytes) {
      // row-major bf16 hi/lo of Pi and S' for the tiled encoder
      uint16_t* g = reinterpret_cast<uint16_t*>(blob.data() + lay.off_gmat);
      const size_t dd = size_t(d) * d;
      for (size_t i = 0; i < dd; ++i) {
        split_bf16(P64[i], g[i], g[dd + i]);
        split_bf16(Sp[i], g[2 * dd + i], g[3 * dd + i]);
      }
    }
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(params, blob.data(), lay.total, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "tq_prepare: copy");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "tq_prepare: synchronize");
  return ok();
}

}  // namespace

extern "C" {

int tq_prepare(int d, int b, const float* Pi, const float* S, const double* centroids,
               const double* thresholds, void* params, void* stream) {
  return prepare_params(d, b, Pi, S, centroids, thresholds, false, params, stream);
}

int tq_prepare_orthogonal_qjl(int d, int b, const float* Pi, const float* S, const double* centroids,
                              const double* thresholds, void* params, void* stream) {
  return prepare_params(d, b, Pi, S, centroids, thresholds, true, params, stream);
}

int tq_quantize(const void* params, int d, int b, const void* x, int x_dtype, int64_t n,
                uint32_t* codes, float* nu, float* gamma, void* stream) {
  if (!valid_shape(d, b)) return fail(TQ_EINVAL, "unsupported shape d=%d b=%d", d, b);
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return fail(TQ_EINVAL, "bad x_dtype %d", x_dtype);
  if (n < 0) return fail(TQ_EINVAL, "n=%lld < 0", (long long)n);
  if (n == 0) return ok();
  if (!params || !x || !codes || !nu || !gamma) return fail(TQ_EINVAL, "NULL pointer");
  if (!aligned(params, 256) || !aligned(x, 16) || !aligned(codes, 16) || !aligned(nu, 4) ||
      !aligned(gamma, 4))
    return fail(TQ_EINVAL, "misaligned pointer (params 256 B, x and codes 16 B)");
  hipError_t e = d == 128 ? tq::launch_quantize_d128(params, b, x, x_dtype, n, codes, nu, gamma,
                                                     static_cast<hipStream_t>(stream))
                          : tq::launch_quantize_gemm(params, d, b, x, x_dtype, n, codes, nu, gamma,
                                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tq_quantize launch");
  return ok();
}

int tq_quantize_with_rotation(const void* params, int d, int b, const void* x, int x_dtype, int64_t n,
                              uint32_t* codes, float* nu, float* gamma, float* u, void* stream) {
  if (!valid_shape(d, b)) return fail(TQ_EINVAL, "unsupported shape d=%d b=%d", d, b);
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return fail(TQ_EINVAL, "bad x_dtype %d", x_dtype);
  if (n < 0) return fail(TQ_EINVAL, "n=%lld < 0", (long long)n);
  if (n == 0) return ok();
  if (!params || !x || !codes || !nu || !gamma || !u) return fail(TQ_EINVAL, "NULL pointer");
  if (!aligned(params, 256) || !aligned(x, 16) || !aligned(codes, 16) || !aligned(nu, 4) ||
      !aligned(gamma, 4) || !aligned(u, 16))
    return fail(TQ_EINVAL, "misaligned pointer (params 256 B, x, codes and u 16 B)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = d == 128 ? tq::launch_quantize_d128_u(params, b, x, x_dtype, n, codes, nu, gamma, u, s)
                          : tq::launch_quantize_gemm(params, d, b, x, x_dtype, n, codes, nu, gamma, s, 0, u);
  if (e != hipSuccess) return hip_fail(e, "tq_quantize_with_rotation launch");
  return ok();
}

int tq_quantize_mse(const void* params, int d, int b, const void* x, int x_dtype, int64_t n,
                    uint32_t* codes, float* nu, void* stream) {
  if (!valid_shape(d, b)) return fail(TQ_EINVAL, "unsupported shape d=%d b=%d", d, b);
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return fail(TQ_EINVAL, "bad x_dtype %d", x_dtype);
  if (n < 0) return fail(TQ_EINVAL, "n=%lld < 0", (long long)n);
  if (n == 0) return ok();
  if (!params || !x || !codes || !nu) return fail(TQ_EINVAL, "NULL pointer");
  // the d = 128 encoder stores each lane's words with 8- or 16-byte stores
  if (!aligned(params, 256) || !aligned(x, 16) || !aligned(codes, d == 128 ? 16 : 4) || !aligned(nu, 4))
    return fail(TQ_EINVAL, "misaligned pointer (params 256 B, x 16 B, codes 16 B at d = 128)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = d == 128 ? tq::launch_quantize_d128_mse(params, b, x, x_dtype, n, codes, nu, s)
                          : tq::launch_quantize_mse(params, d, b, x, x_dtype, n, codes, nu, s);
  if (e != hipSuccess) return hip_fail(e, "tq_quantize_mse launch");
  return ok();
}

size_t tq_append_ws_bytes(int d, int b, int64_t groups) {
  if (!valid_shape(d, b) || groups < 0) return 0;
  return tq::align256(size_t(groups) * (d / 32) * b * 4) + 2 * tq::align256(size_t(groups) * 4);
}

int tq_append(const void* params, int d, int b, int mode, const void* x, int x_dtype,
              int64_t groups, int64_t cap, int64_t pos, uint32_t* codes, float* nu, float* gamma,
              void* ws, size_t ws_bytes, void* stream) {
  if (!valid_shape(d, b)) return fail(TQ_EINVAL, "unsupported shape d=%d b=%d", d, b);
  if (mode != TQ_EST_PROD && mode != TQ_EST_MSE) return fail(TQ_EINVAL, "bad mode %d", mode);
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return fail(TQ_EINVAL, "bad x_dtype %d", x_dtype);
  if (groups < 0 || cap < 0) return fail(TQ_EINVAL, "negative size");
  if (groups == 0) return ok();
  if (pos < 0 || pos >= cap) return fail(TQ_EINVAL, "pos=%lld outside [0, cap=%lld)", (long long)pos,
                                        (long long)cap);
  if (groups >= (int64_t(1) << 31)) return fail(TQ_EINVAL, "groups must be < 2^31");
  const bool prod = mode == TQ_EST_PROD;
  if (!params || !x || !codes || !nu || (prod && !gamma) || !ws) return fail(TQ_EINVAL, "NULL pointer");
  if (!aligned(params, 256) || !aligned(x, 16) || !aligned(ws, 256) || !aligned(codes, 4) ||
      !aligned(nu, 4) || (gamma && !aligned(gamma, 4)))
    return fail(TQ_EINVAL, "misaligned pointer (params, ws 256 B; x 16 B)");
  const size_t need = tq_append_ws_bytes(d, b, groups);
  if (ws_bytes < need) return fail(TQ_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  const int planes = prod ? b : b - 1;
  unsigned char* w = static_cast<unsigned char*>(ws);
  uint32_t* tc = reinterpret_cast<uint32_t*>(w);
  float* tn = reinterpret_cast<float*>(w + tq::align256(size_t(groups) * (d / 32) * b * 4));
  float* tg = tn + tq::align256(size_t(groups) * 4) / 4;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (prod)
    e = d == 128 ? tq::launch_quantize_d128(params, b, x, x_dtype, groups, tc, tn, tg, s)
                 : tq::launch_quantize_gemm(params, d, b, x, x_dtype, groups, tc, tn, tg, s);
  else
    e = d == 128 ? tq::launch_quantize_d128_mse(params, b, x, x_dtype, groups, tc, tn, s)
                 : tq::launch_quantize_mse(params, d, b, x, x_dtype, groups, tc, tn, s);
  if (e == hipSuccess)
    e = tq::launch_scatter_slot(tc, tn, prod ? tg : nullptr, (d / 32) * planes, groups, cap, pos, codes,
                                nu, prod ? gamma : nullptr, s);
  if (e != hipSuccess) return hip_fail(e, "tq_append launch");
  return ok();
}

int tq_dequantize(const void* params, int d, int b, const uint32_t* codes, const float* nu,
                  const float* gamma, int64_t n, int mode, float* xhat, void* stream) {
  if (!valid_shape(d, b)) return fail(TQ_EINVAL, "unsupported shape d=%d b=%d", d, b);
  if (mode != TQ_EST_PROD && mode != TQ_EST_MSE) return fail(TQ_EINVAL, "bad mode %d", mode);
  if (n < 0) return fail(TQ_EINVAL, "n=%lld < 0", (long long)n);
  if (n == 0) return ok();
  if (!params || !codes || !nu || !gamma || !xhat) return fail(TQ_EINVAL, "NULL pointer");
  if (!aligned(params, 256) || !aligned(codes, 4) || !aligned(xhat, 4))
    return fail(TQ_EINVAL, "misaligned pointer");
  hipError_t e = tq::launch_dequantize(params, d, b, codes, nu, gamma, n, mode, xhat,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tq_dequantize launch");
  return ok();
}

// The d = 128 kernel scores quads of query heads; every other shape takes the general path.
static bool score_uses_d128(int d, int64_t G) { return d == 128 && G % 4 == 0; }

static bool score_grid_fits(int d, int64_t groups, int64_t G, int64_t T) {
  return score_uses_d128(d, G) || tq::score_generic_grid_fits(groups, G, T);
}

static hipError_t launch_score_any(const void* params, int d, int b, const void* q, int q_dtype,
                                   const uint32_t* codes, const float* nu, const float* gamma,
                                   int64_t groups, int64_t G, int64_t T, int mode, float* logits,
                                   void* ws, hipStream_t s, int phases = tq::kScoreBoth) {
  return score_uses_d128(d, G)
             ? tq::launch_score_d128(params, b, q, q_dtype, codes, nu, gamma, groups, G, T, mode,
                                     logits, ws, s, phases)
             : tq::launch_score_generic(params, d, b, q, q_dtype, codes, nu, gamma, groups, G, T,
                                        mode, logits, ws, s, 0, phases);
}

size_t tq_score_ws_bytes(int d, int b, int64_t groups, int64_t G, int64_t T) {
  (void)T;
  if (!valid_shape(d, b) || groups < 0 || G < 0) return 0;
  if (score_uses_d128(d, G))   // one operand block per quad of query heads
    return tq::align256(size_t(groups) * size_t(G / 4) * tq::score_ws_per_group(b));
  return tq::align256(tq::score_generic_ws_bytes(d, groups, G));
}

int tq_score_ip(const void* params, int d, int b, const void* q, int q_dtype,
                const uint32_t* codes, const float* nu, const float* gamma, int64_t groups,
                int64_t G, int64_t T, int mode, float* logits, void* ws, size_t ws_bytes,
                void* stream) {
  if (!valid_shape(d, b)) return fail(TQ_EINVAL, "unsupported shape d=%d b=%d", d, b);
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return fail(TQ_EINVAL, "bad q_dtype %d", q_dtype);
  if (mode != TQ_EST_PROD && mode != TQ_EST_MSE) return fail(TQ_EINVAL, "bad mode %d", mode);
  if (groups < 0 || G < 0 || T < 0) return fail(TQ_EINVAL, "negative size");
  if (groups == 0 || G == 0 || T == 0) return ok();
  if (T >= (int64_t(1) << 31)) return fail(TQ_EINVAL, "T must be < 2^31");
  if (!params || !q || !codes || !nu || !gamma || !logits || !ws)
    return fail(TQ_EINVAL, "NULL pointer");
  if (!aligned(params, 256) || !aligned(ws, 256) || !aligned(codes, 16) || !aligned(q, 4) ||
      !aligned(logits, 4))
    return fail(TQ_EINVAL, "misaligned pointer (params, ws 256 B; codes 16 B)");
  if (!score_grid_fits(d, groups, G, T))
    return fail(TQ_EUNSUPPORTED, "tq_score_ip: groups * G * T too large for one launch");
  if (ws_bytes < tq_score_ws_bytes(d, b, groups, G, T))
    return fail(TQ_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes,
                tq_score_ws_bytes(d, b, groups, G, T));
  hipError_t e = launch_score_any(params, d, b, q, q_dtype, codes, nu, gamma, groups, G, T, mode,
                                  logits, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tq_score_ip launch");
  return ok();
}

int tq_score_prepare(const void* params, int d, int b, const void* q, int q_dtype, int64_t groups,
                     int64_t G, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_shape(d, b)) return fail(TQ_EINVAL, "unsupported shape d=%d b=%d", d, b);
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return fail(TQ_EINVAL, "bad q_dtype %d", q_dtype);
  if (groups < 0 || G < 0) return fail(TQ_EINVAL, "negative size");
  if (groups == 0 || G == 0) return ok();
  if (!params || !q || !ws) return fail(TQ_EINVAL, "NULL pointer");
  if (!aligned(params, 256) || !aligned(ws, 256) || !aligned(q, 4))
    return fail(TQ_EINVAL, "misaligned pointer (params, ws 256 B)");
  if (!score_grid_fits(d, groups, G, 1))
    return fail(TQ_EUNSUPPORTED, "tq_score_prepare: groups * G too large for one launch");
  const size_t need = tq_score_ws_bytes(d, b, groups, G, 1);
  if (ws_bytes < need) return fail(TQ_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  hipError_t e = launch_score_any(params, d, b, q, q_dtype, nullptr, nullptr, nullptr, groups, G, 1,
                                  TQ_EST_PROD, nullptr, ws, static_cast<hipStream_t>(stream), tq::kScorePrep);
  if (e != hipSuccess) return hip_fail(e, "tq_score_prepare launch");
  return ok();
}

int tq_score_ip_prepared(const void* params, int d, int b, const uint32_t* codes, const float* nu,
                         const float* gamma, int64_t groups, int64_t G, int64_t T, int mode, float* logits,
                         const void* ws, size_t ws_bytes, void* stream) {
  if (!valid_shape(d, b)) return fail(TQ_EINVAL, "unsupported shape d=%d b=%d", d, b);
  if (mode != TQ_EST_PROD && mode != TQ_EST_MSE) return fail(TQ_EINVAL, "bad mode %d", mode);
  if (groups < 0 || G < 0 || T < 0) return fail(TQ_EINVAL, "negative size");
  if (groups == 0 || G == 0 || T == 0) return ok();
  if (T >= (int64_t(1) << 31)) return fail(TQ_EINVAL, "T must be < 2^31");
  if (!params || !codes || !nu || !gamma || !logits || !ws) return fail(TQ_EINVAL, "NULL pointer");
  if (!aligned(params, 256) || !aligned(ws, 256) || !aligned(codes, 16) || !aligned(logits, 4))
    return fail(TQ_EINVAL, "misaligned pointer (params, ws 256 B; codes 16 B)");
  if (!score_grid_fits(d, groups, G, T))
    return fail(TQ_EUNSUPPORTED, "tq_score_ip_prepared: groups * G * T too large for one launch");
  const size_t need = tq_score_ws_bytes(d, b, groups, G, T);
  if (ws_bytes < need) return fail(TQ_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  hipError_t e = launch_score_any(params, d, b, nullptr, TQ_F32, codes, nu, gamma, groups, G, T, mode,
                                  logits, const_cast<void*>(ws), static_cast<hipStream_t>(stream),
                                  tq::kScoreScan);
  if (e != hipSuccess) return hip_fail(e, "tq_score_ip_prepared launch");
  return ok();
}

// ------------------------------------------------------------- fractional rates
// Two channel groups of each row: [0, d0) and [d0, d), each a TurboQuant instance of its own
// width and bit budget; the logits are the sum of the groups' estimates.

static bool valid_split(int d, int d0, int b0, int b1) {
  return d0 > 0 && d0 < d && valid_shape(d0, b0) && valid_shape(d - d0, b1);
}

int tq_quantize_split(const void* params0, const void* params1, int d, int d0, int b0, int b1,
                      const void* x, int x_dtype, int64_t n, uint32_t* codes0, float* nu0,
                      float* gamma0, uint32_t* codes1, float* nu1, float* gamma1, void* stream) {
  if (!valid_split(d, d0, b0, b1))
    return fail(TQ_EINVAL, "unsupported split d=%d d0=%d b0=%d b1=%d", d, d0, b0, b1);
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return fail(TQ_EINVAL, "bad x_dtype %d", x_dtype);
  if (n < 0) return fail(TQ_EINVAL, "n=%lld < 0", (long long)n);
  if (n == 0) return ok();
  if (!params0 || !params1 || !x || !codes0 || !nu0 || !gamma0 || !codes1 || !nu1 || !gamma1)
    return fail(TQ_EINVAL, "NULL pointer");
  if (!aligned(params0, 256) || !aligned(params1, 256) || !aligned(x, 16) || !aligned(codes0, 16) ||
      !aligned(codes1, 16) || !aligned(nu0, 4) || !aligned(gamma0, 4) || !aligned(nu1, 4) ||
      !aligned(gamma1, 4))
    return fail(TQ_EINVAL, "misaligned pointer (params 256 B, x and codes 16 B)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t esz = x_dtype == TQ_F32 ? 4 : 2;
  const void* x1 = static_cast<const unsigned char*>(x) + size_t(d0) * esz;
  hipError_t e;
  if (d == 128 && d0 == 64) {   // both groups in one pass of the fused encoder
    e = tq::launch_quantize_d128_split(params0, params1, b0, b1, x, x_dtype, n, codes0, nu0, gamma0,
                                       codes1, nu1, gamma1, s);
  } else {
    e = tq::launch_quantize_gemm(params0, d0, b0, x, x_dtype, n, codes0, nu0, gamma0, s, d);
    if (e == hipSuccess)
      e = tq::launch_quantize_gemm(params1, d - d0, b1, x1, x_dtype, n, codes1, nu1, gamma1, s, d);
  }
  if (e != hipSuccess) return hip_fail(e, "tq_quantize_split launch");
  return ok();
}

size_t tq_score_split_ws_bytes(int d, int d0, int b0, int b1, int64_t groups, int64_t G, int64_t T) {
  if (!valid_split(d, d0, b0, b1) || groups < 0 || G < 0) return 0;
  size_t need = tq::align256(tq::score_generic_split_ws_bytes(d0, d - d0, groups, G));
  // the larger of the two paths' needs, so that a size taken for one T also serves another
  if (d == 128 && d0 == 64 && G % 4 == 0) {
    const size_t n128 = tq::score_split_d128_ws_bytes(b0, b1, groups, G);
    if (n128 > need) need = n128;
  }
  (void)T;
  return need;
}

int tq_score_ip_split(const void* params0, const void* params1, int d, int d0, int b0, int b1,
                      const void* q, int q_dtype, const uint32_t* codes0, const float* nu0,
                      const float* gamma0, const uint32_t* codes1, const float* nu1,
                      const float* gamma1, int64_t groups, int64_t G, int64_t T, int mode,
                      float* logits, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_split(d, d0, b0, b1))
    return fail(TQ_EINVAL, "unsupported split d=%d d0=%d b0=%d b1=%d", d, d0, b0, b1);
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return fail(TQ_EINVAL, "bad q_dtype %d", q_dtype);
  if (mode != TQ_EST_PROD && mode != TQ_EST_MSE) return fail(TQ_EINVAL, "bad mode %d", mode);
  if (groups < 0 || G < 0 || T < 0) return fail(TQ_EINVAL, "negative size");
  if (groups == 0 || G == 0 || T == 0) return ok();
  if (T >= (int64_t(1) << 31)) return fail(TQ_EINVAL, "T must be < 2^31");
  if (!params0 || !params1 || !q || !codes0 || !nu0 || !gamma0 || !codes1 || !nu1 || !gamma1 ||
      !logits || !ws)
    return fail(TQ_EINVAL, "NULL pointer");
  if (!aligned(params0, 256) || !aligned(params1, 256) || !aligned(ws, 256) || !aligned(codes0, 16) ||
      !aligned(codes1, 16) || !aligned(q, 4) || !aligned(logits, 4))
    return fail(TQ_EINVAL, "misaligned pointer (params, ws 256 B; codes 16 B)");
  const bool d128 = tq::score_split_d128_applies(d, d0, b0, b1, G, T);
  if (!d128 && !tq::score_generic_grid_fits(groups, G, T))
    return fail(TQ_EUNSUPPORTED, "tq_score_ip_split: groups * G * T too large for one launch");
  const size_t need = tq_score_split_ws_bytes(d, d0, b0, b1, groups, G, T);
  if (ws_bytes < need) return fail(TQ_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // one query prep launch for both groups, one scoring pass summing their estimates
  const hipError_t e =
      d128 ? tq::launch_score_split_d128(params0, params1, b0, b1, q, q_dtype, codes0, nu0, gamma0, codes1,
                                         nu1, gamma1, groups, G, T, mode, logits, ws, s)
           : tq::launch_score_generic_split(params0, params1, d0, d - d0, b0, b1, q, q_dtype, codes0, nu0,
                                            gamma0, codes1, nu1, gamma1, groups, G, T, mode, logits, ws, s);
  if (e != hipSuccess) return hip_fail(e, "tq_score_ip_split launch");
  return ok();
}

int tq_score_split_prepare(const void* params0, const void* params1, int d, int d0, int b0, int b1,
                           const void* q, int q_dtype, int64_t groups, int64_t G, void* ws, size_t ws_bytes,
                           void* stream) {
  if (!valid_split(d, d0, b0, b1))
    return fail(TQ_EINVAL, "unsupported split d=%d d0=%d b0=%d b1=%d", d, d0, b0, b1);
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return fail(TQ_EINVAL, "bad q_dtype %d", q_dtype);
  if (groups < 0 || G < 0) return fail(TQ_EINVAL, "negative size");
  if (groups == 0 || G == 0) return ok();
  if (!params0 || !params1 || !q || !ws) return fail(TQ_EINVAL, "NULL pointer");
  if (!aligned(params0, 256) || !aligned(params1, 256) || !aligned(ws, 256) || !aligned(q, 4))
    return fail(TQ_EINVAL, "misaligned pointer (params, ws 256 B)");
  // the path is chosen from the shape alone, as tq_score_ip_split_prepared chooses it
  const bool d128 = tq::score_split_d128_shape(d, d0, b0, b1, G);
  if (!d128 && !tq::score_generic_grid_fits(groups, G, 1))
    return fail(TQ_EUNSUPPORTED, "tq_score_split_prepare: groups * G too large for one launch");
  const size_t need = tq_score_split_ws_bytes(d, d0, b0, b1, groups, G, 1);
  if (ws_bytes < need) return fail(TQ_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      d128 ? tq::launch_score_split_d128(params0, params1, b0, b1, q, q_dtype, nullptr, nullptr, nullptr, nullptr,
                                         nullptr, nullptr, groups, G, 1, TQ_EST_PROD, nullptr, ws, s,
                                         tq::kScorePrep)
           : tq::launch_score_generic_split(params0, params1, d0, d - d0, b0, b1, q, q_dtype, nullptr, nullptr,
                                            nullptr, nullptr, nullptr, nullptr, groups, G, 1, TQ_EST_PROD,
                                            nullptr, ws, s, tq::kScorePrep);
  if (e != hipSuccess) return hip_fail(e, "tq_score_split_prepare launch");
  return ok();
}

int tq_score_ip_split_prepared(const void* params0, const void* params1, int d, int d0, int b0, int b1,
                               const uint32_t* codes0, const float* nu0, const float* gamma0,
                               const uint32_t* codes1, const float* nu1, const float* gamma1, int64_t groups,
                               int64_t G, int64_t T, int mode, float* logits, const void* ws, size_t ws_bytes,
                               void* stream) {
  if (!valid_split(d, d0, b0, b1))
    return fail(TQ_EINVAL, "unsupported split d=%d d0=%d b0=%d b1=%d", d, d0, b0, b1);
  if (mode != TQ_EST_PROD && mode != TQ_EST_MSE) return fail(TQ_EINVAL, "bad mode %d", mode);
  if (groups < 0 || G < 0 || T < 0) return fail(TQ_EINVAL, "negative size");
  if (groups == 0 || G == 0 || T == 0) return ok();
  if (T >= (int64_t(1) << 31)) return fail(TQ_EINVAL, "T must be < 2^31");
  if (!params0 || !params1 || !codes0 || !nu0 || !gamma0 || !codes1 || !nu1 || !gamma1 || !logits || !ws)
    return fail(TQ_EINVAL, "NULL pointer");
  if (!aligned(params0, 256) || !aligned(params1, 256) || !aligned(ws, 256) || !aligned(codes0, 16) ||
      !aligned(codes1, 16) || !aligned(logits, 4))
    return fail(TQ_EINVAL, "misaligned pointer (params, ws 256 B; codes 16 B)");
  const bool d128 = tq::score_split_d128_shape(d, d0, b0, b1, G);
  if (d128 ? !tq::score_split_d128_applies(d, d0, b0, b1, G, T) : !tq::score_generic_grid_fits(groups, G, T))
    return fail(TQ_EUNSUPPORTED, "tq_score_ip_split_prepared: T too large for the prepared operands' scan");
  const size_t need = tq_score_split_ws_bytes(d, d0, b0, b1, groups, G, T);
  if (ws_bytes < need) return fail(TQ_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* w = const_cast<void*>(ws);
  const hipError_t e =
      d128 ? tq::launch_score_split_d128(params0, params1, b0, b1, nullptr, TQ_F32, codes0, nu0, gamma0, codes1,
                                         nu1, gamma1, groups, G, T, mode, logits, w, s, tq::kScoreScan)
           : tq::launch_score_generic_split(params0, params1, d0, d - d0, b0, b1, nullptr, TQ_F32, codes0, nu0,
                                            gamma0, codes1, nu1, gamma1, groups, G, T, mode, logits, w, s,
                                            tq::kScoreScan);
  if (e != hipSuccess) return hip_fail(e, "tq_score_ip_split_prepared launch");
  return ok();
}

int tq_quantize_mse_split(const void* params0, const void* params1, int d, int d0, int b0, int b1,
                          const void* x, int x_dtype, int64_t n, uint32_t* codes0, float* nu0,
                          uint32_t* codes1, float* nu1, void* stream) {
  if (!valid_split(d, d0, b0, b1))
    return fail(TQ_EINVAL, "unsupported split d=%d d0=%d b0=%d b1=%d", d, d0, b0, b1);
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return fail(TQ_EINVAL, "bad x_dtype %d", x_dtype);
  if (n < 0) return fail(TQ_EINVAL, "n=%lld < 0", (long long)n);
  if (n == 0) return ok();
  if (!params0 || !params1 || !x || !codes0 || !nu0 || !codes1 || !nu1)
    return fail(TQ_EINVAL, "NULL pointer");
  // the one-pass 64 + 64 split stores each lane's words with 8- or 16-byte stores
  const size_t ca = (d == 128 && d0 == 64) ? 16 : 4;
  if (!aligned(params0, 256) || !aligned(params1, 256) || !aligned(x, 16) || !aligned(codes0, ca) ||
      !aligned(codes1, ca) || !aligned(nu0, 4) || !aligned(nu1, 4))
    return fail(TQ_EINVAL, "misaligned pointer (params 256 B, x 16 B, codes 16 B for a 64 + 64 split)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t esz = x_dtype == TQ_F32 ? 4 : 2;
  const void* x1 = static_cast<const unsigned char*>(x) + size_t(d0) * esz;
  hipError_t e;
  if (d == 128 && d0 == 64) {   // both groups in one pass of the fused encoder
    e = tq::launch_quantize_d128_split(params0, params1, b0, b1, x, x_dtype, n, codes0, nu0, nullptr, codes1,
                                       nu1, nullptr, s, true);
  } else {
    e = tq::launch_quantize_mse(params0, d0, b0, x, x_dtype, n, codes0, nu0, s, d);
    if (e == hipSuccess) e = tq::launch_quantize_mse(params1, d - d0, b1, x1, x_dtype, n, codes1, nu1, s, d);
  }
  if (e != hipSuccess) return hip_fail(e, "tq_quantize_mse_split launch");
  return ok();
}

size_t tq_attention_split_ws_bytes(int d, int d0, int bk0, int bk1, int64_t groups, int64_t G, int64_t T) {
  if (!valid_split(d, d0, bk0, bk1) || groups < 0 || G < 0 || T < 0) return 0;
  return tq::align256(size_t(groups) * G * T * 4) + tq_score_split_ws_bytes(d, d0, bk0, bk1, groups, G, T) +
         tq::align256(tq::attention_part_bytes(d0, groups, G, T)) +
         tq::align256(tq::attention_part_bytes(d - d0, groups, G, T));
}

int tq_attention_split(const void* params_k0, const void* params_k1, const void* params_v0,
                       const void* params_v1, int d, int d0, int bk0, int bk1, int bv0, int bv1,
                       const void* q, int q_dtype, const uint32_t* codes_k0, const float* nu_k0,
                       const float* gamma_k0, const uint32_t* codes_k1, const float* nu_k1,
                       const float* gamma_k1, const uint32_t* codes_v0, const float* nu_v0,
                       const uint32_t* codes_v1, const float* nu_v1, int64_t groups, int64_t G,
                       int64_t T, float scale, int mode, float* out, void* ws, size_t ws_bytes,
                       void* stream) {
  if (!valid_split(d, d0, bk0, bk1) || !valid_split(d, d0, bv0, bv1))
    return fail(TQ_EINVAL, "unsupported split d=%d d0=%d keys b=%d,%d values b=%d,%d", d, d0, bk0, bk1,
                bv0, bv1);
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return fail(TQ_EINVAL, "bad q_dtype %d", q_dtype);
  if (mode != TQ_EST_PROD && mode != TQ_EST_MSE) return fail(TQ_EINVAL, "bad mode %d", mode);
  if (!std::isfinite(scale)) return fail(TQ_EINVAL, "scale must be finite");
  if (groups < 0 || G < 0 || T < 0) return fail(TQ_EINVAL, "negative size");
  if (groups == 0 || G == 0) return ok();
  if (T == 0) return fail(TQ_EINVAL, "T = 0: a softmax needs at least one key");
  if (T >= (int64_t(1) << 31)) return fail(TQ_EINVAL, "T must be < 2^31");
  if (!params_k0 || !params_k1 || !params_v0 || !params_v1 || !q || !codes_k0 || !nu_k0 || !gamma_k0 ||
      !codes_k1 || !nu_k1 || !gamma_k1 || !codes_v0 || !nu_v0 || !codes_v1 || !nu_v1 || !out || !ws)
    return fail(TQ_EINVAL, "NULL pointer");
  if (!aligned(params_k0, 256) || !aligned(params_k1, 256) || !aligned(params_v0, 256) ||
      !aligned(params_v1, 256) || !aligned(ws, 256) || !aligned(codes_k0, 16) || !aligned(codes_k1, 16) ||
      !aligned(codes_v0, 4) || !aligned(codes_v1, 4) || !aligned(q, 4) || !aligned(out, 16))
    return fail(TQ_EINVAL, "misaligned pointer (params, ws 256 B; key codes, out 16 B)");
  if ((!tq::score_split_d128_applies(d, d0, bk0, bk1, G, T) && !tq::score_generic_grid_fits(groups, G, T)) ||
      !tq::attention_grid_fits(groups, G, T))
    return fail(TQ_EUNSUPPORTED, "tq_attention_split: groups * G * T too large for one launch");
  const size_t need = tq_attention_split_ws_bytes(d, d0, bk0, bk1, groups, G, T);
  if (ws_bytes < need) return fail(TQ_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  unsigned char* w = static_cast<unsigned char*>(ws);
  float* logits = reinterpret_cast<float*>(w);
  const size_t sws_bytes = tq_score_split_ws_bytes(d, d0, bk0, bk1, groups, G, T);
  void* sws = w + tq::align256(size_t(groups) * G * T * 4);
  void* part = static_cast<unsigned char*>(sws) + sws_bytes;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (tq::score_split_d128_shape(d, d0, bk0, bk1, G) && mode == TQ_EST_PROD &&
      tq::attention_fused_split_applies(bk0, bk1, bv0, bv1)) {
    // the split scorer's query prep, then block kernels that score their own keys (the logits
    // region of the workspace stays unused) and one merge of both value groups
    hipError_t e = tq::launch_score_split_d128(params_k0, params_k1, bk0, bk1, q, q_dtype, nullptr, nullptr,
                                               nullptr, nullptr, nullptr, nullptr, groups, G, 1, TQ_EST_PROD,
                                               nullptr, sws, s, tq::kScorePrep);
    if (e == hipSuccess)
      e = tq::launch_attention_fused_split(params_v0, params_v1, bk0, bk1, codes_k0, nu_k0, gamma_k0, codes_k1,
                                           nu_k1, gamma_k1, sws, bv0, bv1, codes_v0, nu_v0, codes_v1, nu_v1,
                                           groups, G, T, scale, out, part, s);
    if (e != hipSuccess) return hip_fail(e, "tq_attention_split launch");
    return ok();
  }
  // logits of the split keys, then each value group's block partials and one merge of both
  // groups into their columns of out
  const int rc = tq_score_ip_split(params_k0, params_k1, d, d0, bk0, bk1, q, q_dtype, codes_k0, nu_k0,
                                   gamma_k0, codes_k1, nu_k1, gamma_k1, groups, G, T, mode, logits, sws,
                                   sws_bytes, stream);
  if (rc != TQ_OK) return rc;
  const hipError_t e = tq::launch_attention_values_split(params_v0, params_v1, d0, d - d0, bv0, bv1, logits,
                                                         codes_v0, nu_v0, codes_v1, nu_v1, groups, G, T,
                                                         scale, out, part, s);
  if (e != hipSuccess) return hip_fail(e, "tq_attention_split launch");
  return ok();
}

// Logits region of tq_attention's workspace: none where the block kernel scores its own keys.
static size_t attention_logit_bytes(int d, int64_t groups, int64_t G, int64_t T) {
  return score_uses_d128(d, G) ? 0 : tq::align256(size_t(groups) * G * T * 4);
}

size_t tq_attention_ws_bytes(int d, int b_k, int64_t groups, int64_t G, int64_t T) {
  if (!valid_shape(d, b_k) || groups < 0 || G < 0 || T < 0) return 0;
  return attention_logit_bytes(d, groups, G, T) + tq_score_ws_bytes(d, b_k, groups, G, T) +
         tq::align256(tq::attention_part_bytes(d, groups, G, T));
}

int tq_attention(const void* params_k, const void* params_v, int d, int b_k, int b_v,
                 const void* q, int q_dtype, const uint32_t* codes_k, const float* nu_k,
                 const float* gamma_k, const uint32_t* codes_v, const float* nu_v, int64_t groups,
                 int64_t G, int64_t T, float scale, int mode, float* out, void* ws,
                 size_t ws_bytes, void* stream) {
  if (!valid_shape(d, b_k) || !valid_shape(d, b_v))
    return fail(TQ_EINVAL, "unsupported shape d=%d b_k=%d b_v=%d", d, b_k, b_v);
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return fail(TQ_EINVAL, "bad q_dtype %d", q_dtype);
  if (mode != TQ_EST_PROD && mode != TQ_EST_MSE) return fail(TQ_EINVAL, "bad mode %d", mode);
  if (!std::isfinite(scale)) return fail(TQ_EINVAL, "scale must be finite");
  if (groups < 0 || G < 0 || T < 0) return fail(TQ_EINVAL, "negative size");
  if (groups == 0 || G == 0) return ok();
  if (T == 0) return fail(TQ_EINVAL, "T = 0: a softmax needs at least one key");
  if (T >= (int64_t(1) << 31)) return fail(TQ_EINVAL, "T must be < 2^31");
  if (!params_k || !params_v || !q || !codes_k || !nu_k || !gamma_k || !codes_v || !nu_v || !out ||
      !ws)
    return fail(TQ_EINVAL, "NULL pointer");
  if (!aligned(params_k, 256) || !aligned(params_v, 256) || !aligned(ws, 256) ||
      !aligned(codes_k, 16) || !aligned(codes_v, 4) || !aligned(q, 4) || !aligned(out, 16))
    return fail(TQ_EINVAL, "misaligned pointer (params, ws 256 B; key codes, out 16 B)");
  if (!score_grid_fits(d, groups, G, T) || !tq::attention_grid_fits(groups, G, T))
    return fail(TQ_EUNSUPPORTED, "tq_attention: groups * G * T too large for one launch");
  const size_t need = tq_attention_ws_bytes(d, b_k, groups, G, T);
  if (ws_bytes < need) return fail(TQ_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  unsigned char* w = static_cast<unsigned char*>(ws);
  float* logits = reinterpret_cast<float*>(w);   // unused (size 0) on the fused path
  void* sws = w + attention_logit_bytes(d, groups, G, T);
  void* part = static_cast<unsigned char*>(sws) + tq_score_ws_bytes(d, b_k, groups, G, T);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (score_uses_d128(d, G)) {
    // the query operands, then the block kernel scores its own keys (no logits in memory)
    e = launch_score_any(params_k, d, b_k, q, q_dtype, nullptr, nullptr, nullptr, groups, G, T, mode,
                         nullptr, sws, s, tq::kScorePrep);
    if (e == hipSuccess)
      e = tq::launch_attention_fused(params_v, b_k, mode == TQ_EST_PROD, codes_k, nu_k, gamma_k, sws, b_v,
                                     codes_v, nu_v, groups, G, T, scale, out, part, s);
  } else {
    e = launch_score_any(params_k, d, b_k, q, q_dtype, codes_k, nu_k, gamma_k, groups, G, T, mode, logits,
                         sws, s);
    if (e == hipSuccess)
      e = tq::launch_attention_values(params_v, d, b_v, logits, codes_v, nu_v, groups, G, T, scale, out,
                                      part, s);
  }
  if (e != hipSuccess) return hip_fail(e, "tq_attention launch");
  return ok();
}

size_t tq_topk_ws_bytes(int d, int b, int64_t nq, int64_t n, int k) {
  if (!valid_shape(d, b) || nq < 0 || n < 0 || k < 1 || k > 1024) return 0;
  return tq::align256(tq::topk_ws_bytes(d, b, nq, n, k));
}

int tq_topk(const void* params, int d, int b, const void* q, int q_dtype, int64_t nq,
            const uint32_t* codes, const float* nu, const float* gamma, int64_t n, int k,
            int mode, int32_t* idx, float* score, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_shape(d, b)) return fail(TQ_EINVAL, "unsupported shape d=%d b=%d", d, b);
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return fail(TQ_EINVAL, "bad q_dtype %d", q_dtype);
  if (mode != TQ_EST_PROD && mode != TQ_EST_MSE) return fail(TQ_EINVAL, "bad mode %d", mode);
  if (nq < 0 || n < 0) return fail(TQ_EINVAL, "negative size");
  if (k < 1 || k > 1024) return fail(TQ_EINVAL, "k=%d outside 1..1024", k);
  if (nq == 0) return ok();
  if (n < k) return fail(TQ_EINVAL, "k=%d > n=%lld", k, (long long)n);
  if (n >= (int64_t(1) << 31)) return fail(TQ_EINVAL, "n must be < 2^31");
  if (!params || !q || !codes || !nu || !gamma || !idx || !score || !ws)
    return fail(TQ_EINVAL, "NULL pointer");
  if (!aligned(params, 256) || !aligned(ws, 256) || !aligned(codes, 16) || !aligned(q, 4))
    return fail(TQ_EINVAL, "misaligned pointer");
  size_t need = tq_topk_ws_bytes(d, b, nq, n, k);
  if (ws_bytes < need) return fail(TQ_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  hipError_t e = tq::launch_topk(params, d, b, q, q_dtype, nq, codes, nu, gamma, n, k, mode, idx,
                                 score, ws, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported)
    return fail(TQ_EUNSUPPORTED, "tq_topk: not implemented for d=%d b=%d", d, b);
  if (e != hipSuccess) return hip_fail(e, "tq_topk launch");
  return ok();
}

}  // extern "C"

namespace tq {

// Sets the calling thread's tq_last_error() text (for entry points in other source files).
int report_error(int status, const char* message) { return fail(status, "%s", message); }

}  // namespace tq
