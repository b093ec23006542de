/*
 * tq.h — C ABI of the MI355X (gfx950) TurboQuant quantize / inner-product library.
 *
 * TurboQuant encodes a vector x of dimension d with a budget of b bits per coordinate:
 *   1. normalise and rotate by a random orthogonal matrix Pi:   u = Pi x / |x|
 *      ([review, MSE paragraph]; [explainer, caveats]; [tldr, step 1])
 *   2. quantize every coordinate of u on its own with a (b-1)-bit Lloyd-Max grid
 *      precomputed for the near-normal law N(0, 1/d)
 *      ([review, MSE paragraph]; [explainer, step 1]; [tldr, step 1])
 *   3. take the residual (original minus reconstruction), multiply it by a second random
 *      matrix S and keep one sign bit per row: the 1-bit QJL sketch
 *      ([review, inner-product and QJL paragraphs]; [tldr, step 2])
 *   4. estimate <q, x> for an unquantized query q without bias
 *      ([review, problem statement]; [explainer, step 2]; [news, bias paragraph]).
 * Page keys:
 *   [review]    TurboQuant paper review, quant_prune_distill channel (tgviewer.app, post 674)
 *   [news]      "Google ускоряет LLM в 8 раз" (comuna.ru, post 6696)
 *   [explainer] "TurboQuant: Redefining AI efficiency with extreme compression"
 *               (RecSysChannel, tgstat.ru, post 256)
 *   [tldr]      TurboQuant two-step TLDR, seeallochnaya channel (postsniper.ru, post 3476)
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers (memory owned by the caller) unless marked HOST.
 *     The library keeps no persistent allocation of its own.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default stream). Calls
 *     enqueue work and return; none synchronizes the stream unless its comment says so.
 *   - Return value: a tq_status. On any non-zero status except TQ_EHIP nothing was
 *     enqueued. tq_last_error() gives a message for the calling thread. No C++ exception
 *     crosses the ABI.
 *   - Supported shapes: d % 64 == 0, 64 <= d <= 4096; b in {2, 3, 4} total bits
 *     (b-1 bits of Lloyd-Max index + 1 QJL bit); m = d QJL rows. Individual calls may
 *     narrow this (TQ_EUNSUPPORTED). The fractional-rate (*_split) calls take rows of two
 *     channel groups, each a supported d with its own b.
 *   - n == 0 (or groups/T/nq == 0) is a no-op returning TQ_OK.
 *   - NaN / Inf inputs give unspecified codes and estimates but never a fault.
 *   - A zero vector gets nu = 0, its rotated coordinates are taken as 0, and every
 *     estimate against it is 0.
 *
 * Canonical code layout (the pages fix none): codes[n][d/32][b] uint32. For vector v and
 * coordinate group w (coordinates 32w .. 32w+31), word p < b-1 holds bit p of the
 * Lloyd-Max index of each coordinate, word b-1 holds the QJL sign bits (1 = projection
 * >= 0); coordinate 32w + j is bit j. nu[n] = |x|, gamma[n] = |residual of x/|x||, fp32.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_EINVAL = 1,        /* bad argument: shape, null pointer, codebook, enum value */
  TQ_EUNSUPPORTED = 2,  /* valid by the method but not implemented for this shape */
  TQ_EHIP = 3,          /* a HIP launch or copy failed; the stream may hold earlier work */
  TQ_EWORKSPACE = 4     /* workspace smaller than the matching *_ws_bytes() helper */
} tq_status;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1 } tq_dtype;

typedef enum {
  TQ_EST_PROD = 0,  /* MSE part + QJL correction: unbiased ([review, inner-product paragraph]) */
  TQ_EST_MSE = 1    /* MSE part alone: biased ([news, bias paragraph]) */
} tq_mode;

/*
 * tq_codebook_build — HOST only, float64. Lloyd-Max quantizer with L = 2^bits_mse levels for
 * a coordinate distributed N(0, 1/d) ([review, MSE paragraph]: Max-Lloyd grid for the target
 * bit width; [tldr, step 1]: 1-D k-means solved in advance, denser at the centre).
 * Alternates "threshold = midpoint of neighbouring centroids" and "centroid = mean of its
 * cell" to a fixed point (|change| < 1e-14 in sigma units), symmetrised exactly.
 *   bits_mse   1..8
 *   d          dimension (sets sigma = 1/sqrt(d)); > 0
 *   centroids  HOST out [L], ascending
 *   thresholds HOST out [L-1], ascending, thresholds[i] = (c[i] + c[i+1]) / 2, middle one 0
 * Errors: TQ_EINVAL for bits_mse or d out of range or NULL outputs.
 */
int tq_codebook_build(int bits_mse, int d, double* centroids, double* thresholds);

/*
 * tq_codebook_build_sphere — HOST only, float64. The same Lloyd-Max quantizer for the exact
 * law of a rotated coordinate of a unit vector in R^d, density proportional to
 * (1 - u^2)^((d-3)/2) on (-1, 1) ([explainer, per-component reduction]: N(0, 1/d) is its
 * large-d limit; at d = 3 the law is uniform).  Cell masses and first moments by quadrature;
 * fixed point to |change| < 1e-14 / sqrt(d).  The result differs from tq_codebook_build's by
 * O(1/d) in sigma units and can be passed to tq_prepare in its place.
 *   bits_mse   1..8
 *   d          dimension, >= 2
 *   centroids, thresholds  as for tq_codebook_build
 * Errors: TQ_EINVAL for bits_mse or d out of range, NULL outputs, or no convergence.
 */
int tq_codebook_build_sphere(int bits_mse, int d, double* centroids, double* thresholds);

/* Size in bytes of the device parameter block that tq_prepare fills for (d, b). 0 if invalid. */
size_t tq_params_bytes(int d, int b);

/*
 * tq_prepare — fills the device parameter block used by every other call.
 *   Pi          HOST in [d][d] float32, orthogonal ([review, MSE paragraph]: random orthogonal,
 *               not Hadamard); u = Pi x uses Pi's rows.
 *   S           HOST in [d][d] float32, the QJL matrix (m = d rows, [tldr, step 2]).
 *   centroids   HOST in [2^(b-1)] float64 ascending, odd-symmetric (c[i] = -c[L-1-i]),
 *               in the units of u (as returned by tq_codebook_build(b-1, d)).
 *   thresholds  HOST in [2^(b-1)-1] float64 ascending, interleaving the centroids.
 *   params      DEVICE out, tq_params_bytes(d, b) bytes, 256-byte aligned.
 * Works on the host in float64 (S' = S Pi^T, operand splits and layouts), then copies to
 * `params` on `stream` and WAITS for that copy (this call synchronizes `stream`).
 * Errors: TQ_EINVAL (shape, NULL, unsorted or asymmetric codebook, misaligned params),
 * TQ_EHIP (copy failed).
 */
int tq_prepare(int d, int b, const float* Pi, const float* S, const double* centroids,
               const double* thresholds, void* params, void* stream);

/*
 * tq_prepare_orthogonal_qjl — tq_prepare for a QJL matrix S with orthonormal rows
 * (S S^T = I, e.g. a second random rotation) in place of Gaussian entries ([review, QJL
 * paragraph]: the sign sketch works with orthogonalised rows).  Every row of such a random S
 * is a uniform unit vector, for which E[sign<s, rho> <s, q>] = E|w_1| <q, rho>,
 * E|w_1| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)), so the QJL term is scaled by 1/(d E|w_1|)
 * instead of sqrt(pi/2)/d; every other call is unchanged.  Arguments and behaviour as for
 * tq_prepare.
 * Errors: as tq_prepare, plus TQ_EINVAL when max |S S^T - I| > 1e-4.
 */
int tq_prepare_orthogonal_qjl(int d, int b, const float* Pi, const float* S, const double* centroids,
                              const double* thresholds, void* params, void* stream);

/*
 * tq_quantize — encodes n vectors ([review, inner-product paragraph]; [tldr, steps 1-2]).
 *   params   from tq_prepare(d, b, ...)
 *   x        [n][d] float32 (x_dtype TQ_F32) or bfloat16 (TQ_BF16), row-major, 16-byte aligned
 *   codes    out [n][d/32][b] uint32 (canonical layout above)
 *   nu       out [n] float32, |x|
 *   gamma    out [n] float32, norm of the residual of x/|x| after the Lloyd-Max stage
 * Integer decisions (index, sign) are taken in float32 against float32 thresholds; a
 * coordinate exactly on a threshold goes to the cell farther from zero (u = 0 to the positive
 * side), which keeps the quantizer odd-symmetric.
 * d = 128 runs one fused kernel; every other d runs a split pass and two tiled
 * kernels per chunk of c vectors and takes a stream-ordered scratch buffer of
 * c * d * 8 bytes for float32 input, c * d * 4 bytes for bfloat16, plus c * ceil(d / 256) * 4
 * bytes (hipMallocAsync / hipFreeAsync on `stream`, released when the call's work
 * completes).  c = min(n, max(32768, 384 MiB / (d * 8) for float32 or / (d * 4) for
 * bfloat16)): about 384 MiB of scratch whatever d is (more for float32 d > 1536).
 * Errors: TQ_EINVAL (shape, NULL, misalignment), TQ_EHIP (launch or scratch allocation failed).
 */
int tq_quantize(const void* params, int d, int b, const void* x, int x_dtype, int64_t n,
                uint32_t* codes, float* nu, float* gamma, void* stream);

/*
 * tq_quantize_with_rotation — tq_quantize that also returns the rotated unit coordinates
 * u = Pi x / |x| of step 1 ([review, MSE paragraph]: random orthogonal rotation of the
 * normalised vector), as the encoder computed them, for checking the rotation itself.
 *   u      out [n][d] float32, 16-byte aligned (u = 0 for a zero vector)
 *   other arguments, results and errors as tq_quantize; codes, nu and gamma are identical to
 *   tq_quantize's (the same kernels with one extra store).
 */
int tq_quantize_with_rotation(const void* params, int d, int b, const void* x, int x_dtype, int64_t n,
                              uint32_t* codes, float* nu, float* gamma, float* u, void* stream);

/*
 * tq_quantize_mse — the MSE quantizer alone ([review, problem statement]: MSE-optimal
 * TurboQuant is the random rotation followed by Lloyd-Max at the target bit width), for
 * vectors that are reconstructed rather than inner-producted (attention values).
 *   params   from tq_prepare(d, b, ...): its codebook has 2^(b-1) levels, so the codes carry
 *            b-1 index bits per coordinate (values at v bits take a block prepared for v + 1)
 *   x        [n][d] float32 or bfloat16, row-major, 16-byte aligned
 *   codes    out [n][d/32][b-1] uint32: plane p holds bit p of each coordinate's index,
 *            coordinate t in word t/32, bit t%32; 16-byte aligned at d = 128, else 4-byte
 *   nu       out [n] float32, |x|
 * The decisions are those of tq_quantize's index planes. It runs the split pass and the
 * first tiled GEMM of the tiled encoder for d != 128 (float32 input takes a stream-ordered
 * scratch of c * d * 4 bytes, c = min(n, max(32768, 384 MiB / (d * 4)))) and the fused
 * encoder without its QJL GEMM at d = 128.
 * Errors: TQ_EINVAL (shape, NULL, misalignment), TQ_EHIP.
 */
int tq_quantize_mse(const void* params, int d, int b, const void* x, int x_dtype, int64_t n,
                    uint32_t* codes, float* nu, void* stream);

/* Workspace bytes needed by tq_append for these sizes. */
size_t tq_append_ws_bytes(int d, int b, int64_t groups);

/*
 * tq_append — quantize-on-write of one new token per group into existing caches ([explainer,
 * step 1]: the grid is fixed ahead of time, so a token is encoded on arrival without
 * calibration or other tokens): x[g] is encoded as tq_quantize (mode TQ_EST_PROD: keys, b
 * planes, nu and gamma) or tq_quantize_mse (mode TQ_EST_MSE: values, b-1 planes and nu) would
 * encode it, and written to slot (g, pos) of caches laid out [groups][cap]:
 *   codes[g][pos][d/32][planes], nu[g][pos], gamma[g][pos] (gamma unused and may be NULL for
 *   TQ_EST_MSE).  0 <= pos < cap; the other slots are not touched.
 *   x    [groups][d] float32 or bfloat16, 16-byte aligned
 *   ws   tq_append_ws_bytes(d, b, groups) bytes, 256-aligned, scratch
 * Errors: TQ_EINVAL (pos outside [0, cap), NULL, misalignment, ...), TQ_EWORKSPACE, TQ_EHIP.
 */
int tq_append(const void* params, int d, int b, int mode, const void* x, int x_dtype,
              int64_t groups, int64_t cap, int64_t pos, uint32_t* codes, float* nu, float* gamma,
              void* ws, size_t ws_bytes, void* stream);

/*
 * tq_dequantize — reconstruction ([review, QJL paragraph]: inverse rotation and
 * renormalisation).
 *   TQ_EST_PROD: xhat = nu (Pi^T chat + alpha * gamma * S^T (2z - 1)), alpha = sqrt(pi/2)/m
 *                (1/(m E|w_1|) for a block from tq_prepare_orthogonal_qjl)
 *   TQ_EST_MSE : xhat = nu Pi^T chat
 *   codes/nu/gamma as written by tq_quantize; xhat out [n][d] float32.
 * Errors: TQ_EINVAL, TQ_EHIP.
 */
int tq_dequantize(const void* params, int d, int b, const uint32_t* codes, const float* nu,
                  const float* gamma, int64_t n, int mode, float* xhat, void* stream);

/* Workspace bytes needed by tq_score_ip for these sizes. */
size_t tq_score_ws_bytes(int d, int b, int64_t groups, int64_t G, int64_t T);

/*
 * tq_score_ip — attention logits over a quantized key cache: for every group g (a KV head
 * of one sequence), each of its G query heads and each of its T keys
 *   logits[g][h][t] = nu_k (<Pi q, chat_k> + alpha * gamma_k * <S q, 2 z_k - 1>)
 * (alpha as for tq_dequantize)
 * (TQ_EST_MSE drops the second term). The raw inner product, no softmax scale
 * ([review, problem statement]: one side quantized, unbiased; [news, 8x logit paragraph]).
 *   q        [groups][G][d] float32 or bfloat16 (q_dtype), unquantized
 *   codes    [groups][T][d/32][b] uint32; nu, gamma [groups][T] float32
 *   logits   out [groups][G][T] float32
 *   ws       workspace of at least tq_score_ws_bytes(d, b, groups, G, T) bytes, 256-aligned;
 *            its contents are scratch (overwritten by this call)
 * d = 128 with G a multiple of 4 runs the tuned kernel (int8 MFMA over the key bit planes);
 * every other shape runs a general path (float32 query prep, one lane per key).
 * Precision: the general path sums in float32.  The tuned kernel rounds each query value it
 * uses (the codebook's Walsh coefficients e_w times Pi q, and S q) to an integer of at most
 * 16000 in magnitude at the row's own scale (16000 / max|row|), held as two int8 digits
 * 128 hi + lo; the sums over key bits are exact integers and the constant terms are float32
 * sums of the unrounded values.  A logit therefore differs from the float64 estimate of the
 * same codes by at most
 *   nu_k (2 * 96 ne e_max max_t|(Pi q)_t| + gamma_k * 2 * 96 alpha max_t|(S q)_t|) / 16000
 * (ne Walsh terms: 1, 2, 4 for b = 2, 3, 4; half the coordinates round to a half digit, the
 * other half, stored halved, to a whole one) plus float32 rounding, about 1e-3 |q| nu_k at
 * b = 4 for a typical query if every rounding fell the same way, 2e-5 |q| nu_k as a root mean
 * square: far below the estimator's own error.
 * Errors: TQ_EINVAL, TQ_EUNSUPPORTED (groups * G * T beyond one launch of the general path),
 *         TQ_EWORKSPACE, TQ_EHIP.
 */
int tq_score_ip(const void* params, int d, int b, const void* q, int q_dtype,
                const uint32_t* codes, const float* nu, const float* gamma, int64_t groups,
                int64_t G, int64_t T, int mode, float* logits, void* ws, size_t ws_bytes,
                void* stream);

/*
 * tq_score_prepare, tq_score_ip_prepared — tq_score_ip in its two phases, so that the query
 * preparation (which depends only on q) can be issued ahead of, or beside, other work:
 *   tq_score_prepare      writes the query operands of q [groups][G][d] (Pi q and S q in the
 *                         form the scoring kernels read) into ws;
 *   tq_score_ip_prepared  scores the keys (codes, nu, gamma as for tq_score_ip) against the
 *                         operands in ws and writes logits [groups][G][T].
 * tq_score_ip(..., ws) is tq_score_prepare followed by tq_score_ip_prepared on the same
 * stream, and gives the same logits.  The prepared ws must come from tq_score_prepare with
 * the same params, d, b, groups and G, must not be written in between, and can serve any
 * number of scoring calls (any T, mode, key caches).  ws_bytes >= tq_score_ws_bytes(d, b,
 * groups, G, T) (which does not depend on T).  Arguments and errors as for tq_score_ip.
 */
int tq_score_prepare(const void* params, int d, int b, const void* q, int q_dtype, int64_t groups,
                     int64_t G, void* ws, size_t ws_bytes, void* stream);
int tq_score_ip_prepared(const void* params, int d, int b, const uint32_t* codes, const float* nu,
                         const float* gamma, int64_t groups, int64_t G, int64_t T, int mode, float* logits,
                         const void* ws, size_t ws_bytes, void* stream);

/*
 * tq_score_ip_noalloc — tq_score_ip for callers that cannot allocate or hand in a
 * workspace (code under HIP graph capture, tight serving loops): the workspace is a fixed
 * device array of tq_score_noalloc_max_ws_bytes() bytes (8 MiB) inside the library, one per
 * GPU, held until the process ends; its address on a device is looked up on the first call
 * there.  Arguments, results and errors as tq_score_ip without ws / ws_bytes; sizes whose
 * tq_score_ws_bytes exceeds the fixed array return TQ_EUNSUPPORTED before any device call.
 * This call allocates nothing.  All calls on one GPU share its array: calls that overlap on
 * one GPU (e.g. on two streams) race and must be ordered by the caller.
 */
size_t tq_score_noalloc_max_ws_bytes(void);
int tq_score_ip_noalloc(const void* params, int d, int b, const void* q, int q_dtype,
                        const uint32_t* codes, const float* nu, const float* gamma, int64_t groups,
                        int64_t G, int64_t T, int mode, float* logits, void* stream);

/*
 * Fractional bit rates ([review, experiments paragraph] and [news, results paragraph]: KV
 * caches at 2.5 and 3.5 bits per channel; the pages give no mechanism).  Each row of d
 * channels is two channel groups, [0, d0) and [d0, d), each a TurboQuant instance of its
 * own: a parameter block from tq_prepare(d0, b0, ...) and one from tq_prepare(d - d0, b1, ...)
 * (own rotation, QJL matrix and codebook), its own codes, nu and gamma.  The estimate of
 * <q, x> is the sum of the two groups' estimates, each unbiased.  Half the channels at b + 1
 * and half at b give b + 1/2 bits per channel (d = 128: d0 = 64, b0 = b + 1, b1 = b).  Any
 * other assignment of channels to groups is a permutation applied to both queries and keys,
 * which leaves <q, x> unchanged, so the producer of q and x can apply it.
 * A 64 + 64 split of d = 128 encodes both groups in one pass of the fused d = 128 encoder
 * (the two rotations and QJL matrices as block-diagonal operands); other splits run the
 * tiled encoder once per group.  Scoring runs one query-prep launch for both groups and one
 * pass over the keys that adds the two groups' estimates in registers and stores each logit
 * once: for a 64 + 64 split of d = 128 with G a multiple of 4 the integer MFMA scan of the
 * d = 128 scorer (query values rounded to per-row digits, as tq_score_ip rounds them there),
 * otherwise the float32 general path; tq_score_split_ws_bytes covers both paths' query
 * operands.  Channels are read in place (rows d apart).
 *
 * tq_quantize_split — encode x [n][d] (x_dtype as for tq_quantize) into
 *   codes0 [n][d0/32][b0], nu0, gamma0 [n]     (channels 0 .. d0-1, params0)
 *   codes1 [n][(d-d0)/32][b1], nu1, gamma1 [n] (channels d0 .. d-1, params1)
 * Errors: TQ_EINVAL (d0 or d - d0 not a valid d, bits out of 2..4, NULL, misaligned), TQ_EHIP.
 */
int tq_quantize_split(const void* params0, const void* params1, int d, int d0, int b0, int b1,
                      const void* x, int x_dtype, int64_t n, uint32_t* codes0, float* nu0,
                      float* gamma0, uint32_t* codes1, float* nu1, float* gamma1, void* stream);

/* Workspace bytes needed by tq_score_ip_split for these sizes. */
size_t tq_score_split_ws_bytes(int d, int d0, int b0, int b1, int64_t groups, int64_t G, int64_t T);

/*
 * tq_score_ip_split — logits[g][h][t] = estimate over channels [0, d0) + estimate over
 * channels [d0, d), each as tq_score_ip computes it (same mode for both), for queries
 * q [groups][G][d] and the two groups' codes laid out [groups][T] as for tq_score_ip.
 *   ws  at least tq_score_split_ws_bytes(...) bytes, 256-aligned, scratch.
 * Errors: as tq_score_ip.
 */
int tq_score_ip_split(const void* params0, const void* params1, int d, int d0, int b0, int b1,
                      const void* q, int q_dtype, const uint32_t* codes0, const float* nu0,
                      const float* gamma0, const uint32_t* codes1, const float* nu1,
                      const float* gamma1, int64_t groups, int64_t G, int64_t T, int mode,
                      float* logits, void* ws, size_t ws_bytes, void* stream);

/*
 * tq_score_split_prepare, tq_score_ip_split_prepared — tq_score_ip_split in its two phases,
 * as tq_score_prepare and tq_score_ip_prepared split tq_score_ip: the query preparation of
 * both channel groups (which depends only on q) can be issued ahead of, or beside, the key
 * encoding.  tq_score_ip_split(..., ws) gives the same logits as tq_score_split_prepare
 * followed by tq_score_ip_split_prepared on the same stream, wherever tq_score_ip_split
 * takes the path that the shape selects (every T below 2^26 keys per group).  The prepared
 * ws must come from tq_score_split_prepare with the same params0, params1, d, d0, b0, b1,
 * groups and G, must not be written in between, and serves any number of scoring calls (any
 * T, mode and key caches).  ws_bytes >= tq_score_split_ws_bytes(d, d0, b0, b1, groups, G, T)
 * (which does not depend on T).
 * Errors: as tq_score_ip_split; TQ_EUNSUPPORTED also where T is too large for the scan that
 * the prepared operands belong to (64 + 64 splits of d = 128 with G a multiple of 4: T below
 * 2^26; tq_score_ip_split then takes the general path).
 */
int tq_score_split_prepare(const void* params0, const void* params1, int d, int d0, int b0, int b1,
                           const void* q, int q_dtype, int64_t groups, int64_t G, void* ws, size_t ws_bytes,
                           void* stream);
int tq_score_ip_split_prepared(const void* params0, const void* params1, int d, int d0, int b0, int b1,
                               const uint32_t* codes0, const float* nu0, const float* gamma0,
                               const uint32_t* codes1, const float* nu1, const float* gamma1, int64_t groups,
                               int64_t G, int64_t T, int mode, float* logits, const void* ws, size_t ws_bytes,
                               void* stream);

/*
 * tq_quantize_mse_split — the MSE quantizer alone (as tq_quantize_mse) on the two channel
 * groups of x [n][d]: channels [0, d0) with params0 (b0 - 1 index bits) into codes0
 * [n][d0/32][b0-1], nu0 [n]; channels [d0, d) with params1 into codes1, nu1.  Values of a
 * fractional-rate KV cache.  A 64 + 64 split of d = 128 runs one pass of the fused
 * encoder (no QJL stage; codes0 and codes1 then 16-byte aligned); other splits run the tiled
 * encoder's first pass once per group, reading the channels in place.
 * Errors: as tq_quantize_split.
 */
int tq_quantize_mse_split(const void* params0, const void* params1, int d, int d0, int b0, int b1,
                          const void* x, int x_dtype, int64_t n, uint32_t* codes0, float* nu0,
                          uint32_t* codes1, float* nu1, void* stream);

/* Workspace bytes needed by tq_attention_split for these sizes. */
size_t tq_attention_split_ws_bytes(int d, int d0, int bk0, int bk1, int64_t groups, int64_t G, int64_t T);

/*
 * tq_attention_split — tq_attention over a fractional-rate KV cache: the logits are
 * tq_score_ip_split's (key groups [0, d0) and [d0, d) at bk0, bk1 bits), and each value group
 * g (params_v0 / params_v1 from tq_prepare(d_g, bv_g, ...), codes from tq_quantize_mse_split)
 * yields its channels of the output under the same softmax weights:
 *   out[g][h][channels of group v] = Pi_v^T sum_t p_t nu_v,t chat_v,t / sum_t p_t.
 *   out  [groups][G][d] float32, 16-byte aligned
 *   ws   at least tq_attention_split_ws_bytes(...) bytes, 256-aligned, scratch.
 * Errors: as tq_attention.
 */
int tq_attention_split(const void* params_k0, const void* params_k1, const void* params_v0,
                       const void* params_v1, int d, int d0, int bk0, int bk1, int bv0, int bv1,
                       const void* q, int q_dtype, const uint32_t* codes_k0, const float* nu_k0,
                       const float* gamma_k0, const uint32_t* codes_k1, const float* nu_k1,
                       const float* gamma_k1, const uint32_t* codes_v0, const float* nu_v0,
                       const uint32_t* codes_v1, const float* nu_v1, int64_t groups, int64_t G,
                       int64_t T, float scale, int mode, float* out, void* ws, size_t ws_bytes,
                       void* stream);

/* Workspace bytes needed by tq_attention for these sizes. */
size_t tq_attention_ws_bytes(int d, int b_k, int64_t groups, int64_t G, int64_t T);

/*
 * tq_attention — one decode step of attention over a TurboQuant KV cache ([review, problem
 * statement]: keys take the unbiased inner-product quantizer, values the MSE one; [news,
 * KV-cache paragraph]):
 *   out[g][h] = sum_t softmax_t(scale * l[g][h][t]) * nu_v[g][t] Pi_v^T chat_v[g][t]
 * with l the keys' logit estimate of tq_score_ip (mode TQ_EST_PROD or TQ_EST_MSE).
 *   params_k, b_k  keys' parameter block and bits; codes_k [groups][T][d/32][b_k], nu_k and
 *                  gamma_k [groups][T] from tq_quantize
 *   params_v, b_v  values' parameter block and its b; codes_v [groups][T][d/32][b_v - 1] and
 *                  nu_v [groups][T] from tq_quantize_mse
 *   q     [groups][G][d] float32 or bfloat16; scale: multiplies the logits (e.g. 1/sqrt(d))
 *   out   [groups][G][d] float32, 16-byte aligned
 *   ws    tq_attention_ws_bytes(d, b_k, groups, G, T) bytes, 256-aligned, scratch (the
 *         scoring workspace, per-256-key-block partial sums and, for the shapes below that
 *         score into memory, the logits)
 * With d = 128 and G a multiple of 4 the block kernel computes each 256-key block's logits
 * itself from the query operands (the same integer arithmetic as tq_score_ip, so the same
 * logits) and no logits pass through memory or the workspace; other shapes score into ws
 * first.
 * Errors: TQ_EINVAL (T = 0 with groups * G > 0, non-finite scale, ...), TQ_EUNSUPPORTED,
 *         TQ_EWORKSPACE, TQ_EHIP.
 */
int tq_attention(const void* params_k, const void* params_v, int d, int b_k, int b_v,
                 const void* q, int q_dtype, const uint32_t* codes_k, const float* nu_k,
                 const float* gamma_k, const uint32_t* codes_v, const float* nu_v, int64_t groups,
                 int64_t G, int64_t T, float scale, int mode, float* out, void* ws,
                 size_t ws_bytes, void* stream);

/* Workspace bytes needed by tq_topk for these sizes. */
size_t tq_topk_ws_bytes(int d, int b, int64_t nq, int64_t n, int k);

/*
 * tq_topk — flat-scan vector search ([news, vector-search paragraph]: no index to build):
 * for each of nq queries, the k keys with the largest estimated inner product (same
 * estimator as tq_score_ip, mode TQ_EST_PROD or TQ_EST_MSE), sorted by decreasing score,
 * equal scores by increasing key index.
 *   q       [nq][d] float32 or bfloat16; codes [n][d/32][b]; nu, gamma [n]
 *   idx     out [nq][k] int32 key indices;  score out [nq][k] float32
 *   1 <= k <= 1024, k <= n; n < 2^31.
 * k <= 26 runs the fused scan: fp16 MFMA scores keep the best 16 (k <= 10) or 32 candidates
 * per query, whose float32 estimates (the general scoring path's formula) then give the k
 * returned, so scores and order are float32's; larger k score batches of queries against
 * every key on the general scoring path (float32) and select each query's k best by radix
 * select, so their workspace holds up to 256 MiB of scores.
 * Errors: TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EWORKSPACE, TQ_EHIP.
 */
int tq_topk(const void* params, int d, int b, const void* q, int q_dtype, int64_t nq,
            const uint32_t* codes, const float* nu, const float* gamma, int64_t n, int k,
            int mode, int32_t* idx, float* score, void* ws, size_t ws_bytes, void* stream);

/* Message describing the last non-OK status returned on the calling thread ("" if none). */
const char* tq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H_ */
