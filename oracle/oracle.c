/*
 * oracle.c -- plain, slow CPU oracle of the low-bit quantized MoE expert FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code, header, table or constant with the HIP library; it computes the plain
 * definitions the pages give, in double precision, with scalar loops:
 *
 *   dequantize   w = s * q            (symmetric INT4 / INT2 and ternary)
 *                w = s * q + b        (affine; ternary stored as affine has b = -s)
 *   route        top-k experts per token by logit, weights = softmax over the
 *                selected logits (sums to one)
 *   expert FFN   a = W1 x;  h_i = silu(a[2i]) * a[2i+1];  o = W2 h
 *   combine      y[t] = sum_j w[t][j] * o_(t,j), then one round to nearest
 *                even into the activation dtype.
 *
 * Sources on the pages:
 *   - onnxruntime pull request 33005, "[CUDA] Enable SM80+ FP16/BF16 mixed
 *     INT2/INT4 QMoE prefill by default", sections Description and Current
 *     Scope: symmetric codes without zero points, blocks of 64 along K, gate
 *     and up rows interleaved for a fused SwiGLU, and the stage order routing,
 *     rows grouped by expert, FC1, SwiGLU, FC2, top-k weighted finalize.
 *   - MLX issue 3852, "2-bit quantized_matmul loses its size advantage over
 *     4-bit at M >= 3", the repro and the closing remarks: affine groups of
 *     128 with one scale and one bias per group, W stored as [N][K]
 *     (transpose=True), and ternary checkpoints that are affine with values
 *     {-s, 0, +s} and bias equal to minus the scale.
 *   - "The QMoE sub-1-bit expert kernel is a GEMV ..." (inference-research
 *     gotcha page): an inner loop over the tokens that share an expert
 *     computes the same products as one GEMV per token.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   canonical storage = fields LSB-first along K within each byte; symmetric
 *   b-bit code q = u - 2^(b-1); ternary q = u - 1 with u = 3 invalid; even
 *   FC1 row 2i is gate_i and odd row 2i+1 is up_i; SwiGLU is silu(g) * u with
 *   silu(g) = g / (1 + exp(-g)); top-k ties go to the lower expert index and
 *   the ids are ordered by descending logit; the routing weights are the
 *   softmax of the k selected logits; every routed slot is computed.
 *
 * Base-3 ternary (the denser ternary storage of about 1.6 bits per weight in
 * MLX issue 3852's closing remarks; the ternary sketch blocks of about 30
 * bytes per 128 weights in the channel-selection explainer): each block of
 * B weights takes ceil(B/5) bytes; weight i of the block is base-3 digit
 * i mod 5 (least significant first) of byte i / 5, q = digit - 1, and a byte
 * whose value needs more digits than it holds (>= 243, or >= 3^(B mod 5)
 * for a block's last partial byte) is invalid.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_SYM_INT4 = 0, ORC_SYM_INT2 = 1, ORC_TERNARY = 2, ORC_AFFINE_INT2 = 3, ORC_AFFINE_INT4 = 4,
       ORC_TERNARY_B3 = 5 };
enum { ORC_BF16 = 0, ORC_F16 = 1, ORC_F32 = 2 };

/* ---------- 16-bit floating point, from the IEEE 754 definitions ---------- */

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits.
 * binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static void orc_format(int dtype, int *mant, int *ebits, int *bias) {
  if (dtype == ORC_BF16) { *mant = 7; *ebits = 8; *bias = 127; }
  else { *mant = 10; *ebits = 5; *bias = 15; }
}

double orc_half_to_double(uint16_t h, int dtype) {
  int mant, ebits, bias;
  orc_format(dtype, &mant, &ebits, &bias);
  int sign = (h >> 15) & 1;
  int e = (h >> mant) & ((1 << ebits) - 1);
  int m = h & ((1 << mant) - 1);
  double v;
  if (e == 0) {
    v = ldexp((double)m, 1 - bias - mant);               /* subnormal or zero */
  } else if (e == (1 << ebits) - 1) {
    v = (m == 0) ? INFINITY : NAN;
  } else {
    v = ldexp((double)((1 << mant) + m), e - bias - mant); /* (1 + m/2^mant) 2^(e-bias) */
  }
  return sign ? -v : v;
}

/* Round a double to the nearest value of the 16-bit format, ties to even. */
uint16_t orc_double_to_half(double v, int dtype) {
  int mant, ebits, bias;
  orc_format(dtype, &mant, &ebits, &bias);
  const int emin = 1 - bias, emax = bias;
  const uint16_t sign = signbit(v) ? (uint16_t)0x8000 : 0;
  const uint16_t inf_bits = (uint16_t)(((1 << ebits) - 1) << mant);
  if (isnan(v)) return (uint16_t)(inf_bits | (1 << (mant - 1)));
  double a = fabs(v);
  if (isinf(a)) return sign | inf_bits;
  if (a == 0.0) return sign;
  int ex;
  frexp(a, &ex);              /* a = f 2^ex, f in [0.5, 1)  ->  binade exponent ex-1 */
  int E = ex - 1;
  if (E < emin) E = emin;     /* subnormal range: fixed spacing */
  if (E > emax) return sign | inf_bits;
  double ulp = ldexp(1.0, E - mant);
  double r = nearbyint(a / ulp); /* default rounding mode: nearest, ties to even */
  double rv = r * ulp;
  if (rv == 0.0) return sign;
  frexp(rv, &ex);
  int E2 = ex - 1;
  if (E2 > emax) return sign | inf_bits;
  if (E2 < emin) { /* subnormal result */
    uint16_t m = (uint16_t)(rv / ldexp(1.0, emin - mant));
    return sign | m;
  }
  uint16_t ebits_v = (uint16_t)(E2 + bias);
  uint16_t m = (uint16_t)(rv / ldexp(1.0, E2 - mant) - (double)(1 << mant));
  return (uint16_t)(sign | (ebits_v << mant) | m);
}

void orc_halves_to_double(const uint16_t *h, int64_t n, int dtype, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_half_to_double(h[i], dtype);
}

void orc_doubles_to_half(const double *v, int64_t n, int dtype, uint16_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_double_to_half(v[i], dtype);
}

/* ---------------------------- codec & dequant ---------------------------- */

int orc_bits(int fmt) {
  return (fmt == ORC_SYM_INT4 || fmt == ORC_AFFINE_INT4) ? 4 : 2;
}

/* Bytes of one packed row of K weights in blocks of `block`. */
int64_t orc_row_bytes(int fmt, int block, int64_t K) {
  if (fmt == ORC_TERNARY_B3) return (K / block) * ((block + 4) / 5);
  return K * orc_bits(fmt) / 8;
}

/* Stored field u of weight k in a packed row: fields run LSB-first along K. */
static int orc_field(const uint8_t *row, int bits, int64_t k) {
  int64_t bit = k * bits;
  return (row[bit >> 3] >> (bit & 7)) & ((1 << bits) - 1);
}

/* Field value -> integer code.  *bad is set for the unused ternary value 3. */
static int orc_code(int fmt, int u, int *bad) {
  switch (fmt) {
    case ORC_SYM_INT4: return u - 8;  /* [-8, 7] */
    case ORC_SYM_INT2: return u - 2;  /* [-2, 1] */
    case ORC_TERNARY:
      if (u == 3) { *bad = 1; return 0; }
      return u - 1;                   /* {-1, 0, 1} */
    default: return u;                /* affine: unsigned [0, 2^b - 1] */
  }
}

static int orc_is_affine(int fmt) { return fmt == ORC_AFFINE_INT2 || fmt == ORC_AFFINE_INT4; }

/* Base-3 digit d (0 = least significant) of byte v, by repeated division. */
static int orc_b3_digit(int v, int d) {
  for (int i = 0; i < d; ++i) v /= 3;
  return v % 3;
}

/* Integer code of weight k of a packed row (any format).  *bad is set for an
 * invalid field or byte. */
static int orc_code_at(int fmt, int block, const uint8_t *row, int64_t k, int *bad) {
  if (fmt == ORC_TERNARY_B3) {
    const int64_t per = (block + 4) / 5;          /* bytes per block */
    const int64_t b = k / block, i = k % block;   /* block, position in block */
    const int j = (int)(i / 5);                   /* byte within the block */
    const int held = (j == per - 1 && block % 5) ? block % 5 : 5;
    int limit = 1;
    for (int h = 0; h < held; ++h) limit *= 3;
    const int v = row[b * per + j];
    if (v >= limit) { *bad = 1; return 0; }
    return orc_b3_digit(v, (int)(i % 5)) - 1;
  }
  return orc_code(fmt, orc_field(row, orc_bits(fmt), k), bad);
}

/* Integer codes of a [rows][K] matrix with blocks of `block` (the block only
 * matters for base-3 rows); returns the number of invalid fields (or, for
 * base-3, of weights in invalid bytes). */
int64_t orc_unpack_codes_b(int fmt, int block, const uint8_t *packed, int64_t rows, int64_t K, int8_t *out) {
  const int64_t row_bytes = orc_row_bytes(fmt, block, K);
  int64_t nbad = 0;
  for (int64_t n = 0; n < rows; ++n) {
    for (int64_t k = 0; k < K; ++k) {
      int bad = 0;
      out[n * K + k] = (int8_t)orc_code_at(fmt, block, packed + n * row_bytes, k, &bad);
      nbad += bad;
    }
  }
  return nbad;
}

/* Integer codes of a [rows][K] matrix; returns the number of invalid fields. */
int64_t orc_unpack_codes(int fmt, const uint8_t *packed, int64_t rows, int64_t K, int8_t *out) {
  return orc_unpack_codes_b(fmt, 128, packed, rows, K, out);
}

/* One dequantized row: w[k] = s*q (+ b for affine), s and b of block k/B. */
static void orc_dequant_row(int fmt, int block, int sdtype, const uint8_t *codes_row,
                            const uint16_t *scales_row, const uint16_t *biases_row,
                            int64_t K, double *w, int *bad) {
  for (int64_t k = 0; k < K; ++k) {
    int q = orc_code_at(fmt, block, codes_row, k, bad);
    double s = orc_half_to_double(scales_row[k / block], sdtype);
    double v = s * (double)q;
    if (orc_is_affine(fmt)) v += orc_half_to_double(biases_row[k / block], sdtype);
    w[k] = v;
  }
}

void orc_dequant(int fmt, int block, int sdtype, const uint8_t *codes, const uint16_t *scales,
                 const uint16_t *biases, int64_t rows, int64_t K, double *W) {
  const int64_t row_bytes = orc_row_bytes(fmt, block, K), nb = K / block;
  int bad = 0;
  for (int64_t n = 0; n < rows; ++n)
    orc_dequant_row(fmt, block, sdtype, codes + n * row_bytes, scales + n * nb,
                    biases ? biases + n * nb : NULL, K, W + n * K, &bad);
}

/* -------------------------------- routing -------------------------------- */

/* Per token: the k largest logits (ties to the lower expert index), in
 * descending order.  Weights: with renorm, the softmax over the k selected
 * logits (they sum to 1); without, the softmax over all E logits, of which
 * the k selected probabilities are kept as they are (for k = 1 the Switch
 * router's top probability).  Then the expert map: counts, exclusive offsets
 * (E+1 entries) and the list of flat slots r = t*k + j grouped by expert,
 * ascending r within an expert. */
void orc_route(int T, int E, int k, int renorm, const float *logits, int32_t *ids, double *w,
               int32_t *counts, int32_t *offsets, int32_t *row_list) {
  char *taken = (char *)malloc((size_t)E);
  for (int t = 0; t < T; ++t) {
    const float *l = logits + (int64_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e;
      }
      taken[best] = 1;
      ids[(int64_t)t * k + j] = best;
    }
    double m = (double)l[ids[(int64_t)t * k]];
    double sum = 0.0;
    if (renorm)
      for (int j = 0; j < k; ++j) sum += exp((double)l[ids[(int64_t)t * k + j]] - m);
    else
      for (int e = 0; e < E; ++e) sum += exp((double)l[e] - m);
    for (int j = 0; j < k; ++j) w[(int64_t)t * k + j] = exp((double)l[ids[(int64_t)t * k + j]] - m) / sum;
  }
  free(taken);
  const int64_t S = (int64_t)T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t r = 0; r < S; ++r) counts[ids[r]] += 1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int64_t pos = 0;
  for (int e = 0; e < E; ++e)
    for (int64_t r = 0; r < S; ++r)
      if (ids[r] == e) row_list[pos++] = (int32_t)r;
}

/* ------------------------------ expert FFN ------------------------------- */

double orc_silu(double g) { return g / (1.0 + exp(-g)); }

/* Configurable SwiGLU (onnxruntime pull request 33005, Description: the
 * expert bias is followed by a configurable SwiGLU; the page gives no
 * parameters).  With limit > 0 the gate is clipped from above and the up
 * value to [-limit, limit]; then h = g * sigmoid(alpha * g) * (u + beta).
 * alpha = 1, beta = 0, limit = 0 (no clipping) is the plain silu(g) * u. */
double orc_swiglu(double g, double u, double alpha, double beta, double limit) {
  if (limit > 0.0) {
    if (g > limit) g = limit;
    if (u > limit) u = limit;
    if (u < -limit) u = -limit;
  }
  return g / (1.0 + exp(-alpha * g)) * (u + beta);
}

/* Activation-dtype element i of p: 16-bit patterns of bf16 / f16, or f32. */
static double orc_act(const void *p, int64_t i, int dtype) {
  if (dtype == ORC_F32) return (double)((const float *)p)[i];
  return orc_half_to_double(((const uint16_t *)p)[i], dtype);
}

typedef struct {
  int fmt, block, sdtype;
  const uint8_t *codes;
  const uint16_t *scales, *biases;
} orc_mat;

/* out[n] = sum_k W[e][n][k] * v[k] for n in [0, N). */
static void orc_matvec(const orc_mat *m, int64_t e, int64_t N, int64_t K, const double *v,
                       double *out, double *wrow, int *bad) {
  const int64_t row_bytes = orc_row_bytes(m->fmt, m->block, K), nb = K / m->block;
  for (int64_t n = 0; n < N; ++n) {
    const int64_t r = e * N + n;
    orc_dequant_row(m->fmt, m->block, m->sdtype, m->codes + r * row_bytes, m->scales + r * nb,
                    m->biases ? m->biases + r * nb : NULL, K, wrow, bad);
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) acc += wrow[k] * v[k];
    out[n] = acc;
  }
}

/*
 * Full MoE layer for T tokens.  x [T][H] and y_out [T][H] hold act_dtype
 * elements (16-bit patterns of bf16 / f16, or f32; y_out is y64 rounded once
 * to that dtype), logits [T][E] float32, y64 [T][H] the unrounded result.  Optional
 * per-slot diagnostics in slot order r = t*k + j: a_dbg [T*k][2I] (FC1),
 * h_dbg [T*k][I] (after SwiGLU), o_dbg [T*k][H] (FC2).  Optional expert
 * biases, act_dtype elements: fc1_ebias [E][2I], in FC1's interleaved row order, is
 * added to FC1's output before the SwiGLU, and fc2_ebias [E][H] to FC2's
 * output before the top-k weighting (onnxruntime pull request 33005,
 * Description: expert bias before the SwiGLU, FC2 bias in the finalize).
 * With relu, FC1 is a single [I][H] matrix and h = max(a, 0) (the Switch
 * Transformer FFN); a_dbg and fc1_ebias then have I entries per slot /
 * expert.  Returns 0, or -1 if a ternary row it used holds the invalid field
 * value 3 (read as 0).  renorm selects the routing weights as in orc_route.
 * sw_alpha, sw_beta, sw_limit configure the SwiGLU as in orc_swiglu (1, 0, 0:
 * the plain silu(g) * u).
 */
int orc_moe(int E, int H, int I, int k, int act_dtype,
            int fc1_fmt, int fc1_block, int fc1_sdtype,
            const uint8_t *fc1_codes, const uint16_t *fc1_scales, const uint16_t *fc1_biases,
            int fc2_fmt, int fc2_block, int fc2_sdtype,
            const uint8_t *fc2_codes, const uint16_t *fc2_scales, const uint16_t *fc2_biases,
            const void *fc1_ebias, const void *fc2_ebias, int renorm, int relu,
            double sw_alpha, double sw_beta, double sw_limit,
            const void *x, const float *logits, int T,
            double *y64, void *y_out, double *a_dbg, double *h_dbg, double *o_dbg) {
  orc_mat w1 = {fc1_fmt, fc1_block, fc1_sdtype, fc1_codes, fc1_scales, fc1_biases};
  orc_mat w2 = {fc2_fmt, fc2_block, fc2_sdtype, fc2_codes, fc2_scales, fc2_biases};
  const int64_t S = (int64_t)T * k;
  int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
  double *wts = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
  int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  int32_t *offsets = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t *rows = (int32_t *)malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
  double *xv = (double *)malloc(sizeof(double) * (size_t)H);
  const int64_t R1 = relu ? (int64_t)I : 2 * (int64_t)I;  /* FC1 rows */
  double *a = (double *)malloc(sizeof(double) * (size_t)R1);
  double *h = (double *)malloc(sizeof(double) * (size_t)I);
  double *o = (double *)malloc(sizeof(double) * (size_t)H);
  double *wrow = (double *)malloc(sizeof(double) * (size_t)(H > I ? H : I));
  int bad = 0;
  orc_route(T, E, k, renorm, logits, ids, wts, counts, offsets, rows);
  for (int t = 0; t < T; ++t) {
    for (int64_t n = 0; n < H; ++n) xv[n] = orc_act(x, (int64_t)t * H + n, act_dtype);
    double *yt = y64 + (int64_t)t * H;
    for (int64_t n = 0; n < H; ++n) yt[n] = 0.0;
    for (int j = 0; j < k; ++j) {
      const int64_t r = (int64_t)t * k + j;
      const int e = ids[r];
      orc_matvec(&w1, e, R1, H, xv, a, wrow, &bad);
      if (fc1_ebias)
        for (int64_t n = 0; n < R1; ++n) a[n] += orc_act(fc1_ebias, (int64_t)e * R1 + n, act_dtype);
      if (relu)
        for (int64_t i = 0; i < I; ++i) h[i] = a[i] > 0.0 ? a[i] : 0.0;
      else
        for (int64_t i = 0; i < I; ++i) h[i] = orc_swiglu(a[2 * i], a[2 * i + 1], sw_alpha, sw_beta, sw_limit);
      orc_matvec(&w2, e, H, I, h, o, wrow, &bad);
      if (fc2_ebias)
        for (int64_t n = 0; n < H; ++n) o[n] += orc_act(fc2_ebias, (int64_t)e * H + n, act_dtype);
      for (int64_t n = 0; n < H; ++n) yt[n] += wts[r] * o[n];
      if (a_dbg) memcpy(a_dbg + r * R1, a, sizeof(double) * (size_t)R1);
      if (h_dbg) memcpy(h_dbg + r * I, h, sizeof(double) * (size_t)I);
      if (o_dbg) memcpy(o_dbg + r * H, o, sizeof(double) * (size_t)H);
    }
    for (int64_t n = 0; n < H; ++n) {
      if (act_dtype == ORC_F32) ((float *)y_out)[(int64_t)t * H + n] = (float)yt[n];  /* one RNE */
      else ((uint16_t *)y_out)[(int64_t)t * H + n] = orc_double_to_half(yt[n], act_dtype);
    }
  }
  free(ids); free(wts); free(counts); free(offsets); free(rows);
  free(xv); free(a); free(h); free(o); free(wrow);
  return bad ? -1 : 0;
}

/*
 * The same layer with every sum in single precision: weights dequantized to
 * float (w = s*q is exact in float; affine s*q + b rounds once), each dot
 * product accumulated in float with k ascending, silu from the float expf,
 * the top-k weights in float, the combine in float with j ascending from 0,
 * and one round to nearest even from the float sum to the activation dtype.
 * This is the fp32-accumulation reading of the layer; it serves as a second
 * evaluation of the same definitions in another precision, which must agree
 * with orc_moe's double-precision sums to within fp32 rounding.  Writes the
 * float sums to y32 [T][H] and the rounded outputs to y_out.  No expert
 * biases, ReLU or diagnostics.  Returns 0, or -1 for an invalid ternary field.
 */
static void orc_dequant_row_f32(int fmt, int block, int sdtype, const uint8_t *codes_row,
                                const uint16_t *scales_row, const uint16_t *biases_row,
                                int64_t K, float *w, int *bad) {
  for (int64_t k = 0; k < K; ++k) {
    int q = orc_code_at(fmt, block, codes_row, k, bad);
    float s = (float)orc_half_to_double(scales_row[k / block], sdtype);
    float v = s * (float)q;
    if (orc_is_affine(fmt)) v = v + (float)orc_half_to_double(biases_row[k / block], sdtype);
    w[k] = v;
  }
}

static void orc_matvec_f32(const orc_mat *m, int64_t e, int64_t N, int64_t K, const float *v,
                           float *out, float *wrow, int *bad) {
  const int64_t row_bytes = orc_row_bytes(m->fmt, m->block, K), nb = K / m->block;
  for (int64_t n = 0; n < N; ++n) {
    const int64_t r = e * N + n;
    orc_dequant_row_f32(m->fmt, m->block, m->sdtype, m->codes + r * row_bytes, m->scales + r * nb,
                        m->biases ? m->biases + r * nb : NULL, K, wrow, bad);
    float acc = 0.0f;
    for (int64_t k = 0; k < K; ++k) acc = acc + wrow[k] * v[k];
    out[n] = acc;
  }
}

int orc_moe_f32acc(int E, int H, int I, int k, int act_dtype,
                   int fc1_fmt, int fc1_block, int fc1_sdtype,
                   const uint8_t *fc1_codes, const uint16_t *fc1_scales, const uint16_t *fc1_biases,
                   int fc2_fmt, int fc2_block, int fc2_sdtype,
                   const uint8_t *fc2_codes, const uint16_t *fc2_scales, const uint16_t *fc2_biases,
                   const void *x, const float *logits, int T, float *y32, void *y_out) {
  orc_mat w1 = {fc1_fmt, fc1_block, fc1_sdtype, fc1_codes, fc1_scales, fc1_biases};
  orc_mat w2 = {fc2_fmt, fc2_block, fc2_sdtype, fc2_codes, fc2_scales, fc2_biases};
  const int64_t S = (int64_t)T * k;
  int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
  double *wd = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
  int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  int32_t *offsets = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t *rows = (int32_t *)malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
  float *xv = (float *)malloc(sizeof(float) * (size_t)H);
  float *a = (float *)malloc(sizeof(float) * (size_t)(2 * (int64_t)I));
  float *h = (float *)malloc(sizeof(float) * (size_t)I);
  float *o = (float *)malloc(sizeof(float) * (size_t)H);
  float *wrow = (float *)malloc(sizeof(float) * (size_t)(H > I ? H : I));
  int bad = 0;
  /* the selection is the same; the weights are recomputed in float */
  orc_route(T, E, k, 1, logits, ids, wd, counts, offsets, rows);
  for (int t = 0; t < T; ++t) {
    const float *l = logits + (int64_t)t * E;
    const float m = l[ids[(int64_t)t * k]];
    float sum = 0.0f;
    for (int j = 0; j < k; ++j) sum = sum + expf(l[ids[(int64_t)t * k + j]] - m);
    for (int64_t n = 0; n < H; ++n) xv[n] = (float)orc_act(x, (int64_t)t * H + n, act_dtype);
    float *yt = y32 + (int64_t)t * H;
    for (int64_t n = 0; n < H; ++n) yt[n] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int64_t r = (int64_t)t * k + j;
      const int e = ids[r];
      const float wt = expf(l[ids[r]] - m) / sum;
      orc_matvec_f32(&w1, e, 2 * (int64_t)I, H, xv, a, wrow, &bad);
      for (int64_t i = 0; i < I; ++i) {
        const float g = a[2 * i];
        h[i] = g / (1.0f + expf(-g)) * a[2 * i + 1];
      }
      orc_matvec_f32(&w2, e, H, I, h, o, wrow, &bad);
      for (int64_t n = 0; n < H; ++n) yt[n] = yt[n] + wt * o[n];
    }
    for (int64_t n = 0; n < H; ++n) {
      if (act_dtype == ORC_F32) ((float *)y_out)[(int64_t)t * H + n] = yt[n];
      else ((uint16_t *)y_out)[(int64_t)t * H + n] = orc_double_to_half((double)yt[n], act_dtype);
    }
  }
  free(ids); free(wd); free(counts); free(offsets); free(rows);
  free(xv); free(a); free(h); free(o); free(wrow);
  return bad ? -1 : 0;
}

/*
 * Gathered channels (MoE channel selection explainer: top-k channel
 * selection reads the selected channels in full and computes them exactly).
 * For each routed slot (t, j) with expert e, channels ch[t][j][0..C-1]
 * (entries < 0 are unused) are the only ones computed:
 *   g = W1[e][2c] . x_t,  u = W1[e][2c+1] . x_t,  h_c = silu(g) * u,
 *   y_t = sum_j w[t][j] * sum_{listed c} h_c * D[e][c][:],
 * where D[e] = the down projection stored channel-major, [I][H], row c being
 * channel c's column of the down matrix (its own canonical codes and block
 * scales along H).  Summed in double in list order, y rounded once.  Routing
 * as orc_route with renormalised weights.  Returns 0, or -1 for an invalid
 * ternary field.
 */
int orc_moe_channels(int E, int H, int I, int k, int act_dtype,
                     int fc1_fmt, int fc1_block, int fc1_sdtype,
                     const uint8_t *fc1_codes, const uint16_t *fc1_scales,
                     int dn_fmt, int dn_block, int dn_sdtype,
                     const uint8_t *dn_codes, const uint16_t *dn_scales,
                     const void *x, const float *logits, int T, const int32_t *ch, int C,
                     double *y64, void *y_out, double *h_dbg) {
  orc_mat w1 = {fc1_fmt, fc1_block, fc1_sdtype, fc1_codes, fc1_scales, NULL};
  const int64_t S = (int64_t)T * k;
  int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
  double *wts = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
  int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  int32_t *offsets = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t *rows = (int32_t *)malloc(sizeof(int32_t) * (size_t)(S > 0 ? S : 1));
  double *xv = (double *)malloc(sizeof(double) * (size_t)H);
  double *wrow = (double *)malloc(sizeof(double) * (size_t)H);
  double *o = (double *)malloc(sizeof(double) * (size_t)H);
  const int64_t row1 = orc_row_bytes(fc1_fmt, fc1_block, H), nb1 = H / fc1_block;
  const int64_t rowd = orc_row_bytes(dn_fmt, dn_block, H), nbd = H / dn_block;
  int bad = 0;
  orc_route(T, E, k, 1, logits, ids, wts, counts, offsets, rows);
  for (int t = 0; t < T; ++t) {
    for (int64_t n = 0; n < H; ++n) xv[n] = orc_act(x, (int64_t)t * H + n, act_dtype);
    double *yt = y64 + (int64_t)t * H;
    for (int64_t n = 0; n < H; ++n) yt[n] = 0.0;
    for (int j = 0; j < k; ++j) {
      const int64_t r = (int64_t)t * k + j;
      const int64_t e = ids[r];
      for (int64_t n = 0; n < H; ++n) o[n] = 0.0;
      for (int c = 0; c < C; ++c) {
        const int32_t cc = ch[r * C + c];
        double h = 0.0;
        if (cc >= 0) {
          double a[2];
          for (int q = 0; q < 2; ++q) {
            const int64_t rr = e * 2 * (int64_t)I + 2 * (int64_t)cc + q;
            orc_dequant_row(w1.fmt, w1.block, w1.sdtype, w1.codes + rr * row1, w1.scales + rr * nb1, NULL, H, wrow,
                            &bad);
            double acc = 0.0;
            for (int64_t kk = 0; kk < H; ++kk) acc += wrow[kk] * xv[kk];
            a[q] = acc;
          }
          h = orc_silu(a[0]) * a[1];
          const int64_t dr = e * (int64_t)I + cc;
          orc_dequant_row(dn_fmt, dn_block, dn_sdtype, dn_codes + dr * rowd, dn_scales + dr * nbd, NULL, H, wrow,
                          &bad);
          for (int64_t n = 0; n < H; ++n) o[n] += h * wrow[n];
        }
        if (h_dbg) h_dbg[r * C + c] = h;
      }
      for (int64_t n = 0; n < H; ++n) yt[n] += wts[r] * o[n];
    }
    for (int64_t n = 0; n < H; ++n) {
      if (act_dtype == ORC_F32) ((float *)y_out)[(int64_t)t * H + n] = (float)yt[n];
      else ((uint16_t *)y_out)[(int64_t)t * H + n] = orc_double_to_half(yt[n], act_dtype);
    }
  }
  free(ids); free(wts); free(counts); free(offsets); free(rows);
  free(xv); free(wrow); free(o);
  return bad ? -1 : 0;
}

/*
 * Dense quantized matmul y = x W^T for output rows n in [n0, n1):
 * y64 [M][n1-n0] unrounded, y16 the same rounded to x's dtype.
 */
void orc_linear(int fmt, int block, int sdtype, const uint8_t *codes, const uint16_t *scales,
                const uint16_t *biases, int64_t N, int64_t K, const uint16_t *x, int x_dtype, int M,
                int64_t n0, int64_t n1, double *y64, uint16_t *y16) {
  (void)N;
  const int64_t row_bytes = orc_row_bytes(fmt, block, K), nb = K / block, W = n1 - n0;
  double *wrow = (double *)malloc(sizeof(double) * (size_t)K);
  double *xv = (double *)malloc(sizeof(double) * (size_t)K * (size_t)(M > 0 ? M : 1));
  for (int m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) xv[(int64_t)m * K + k] = orc_half_to_double(x[(int64_t)m * K + k], x_dtype);
  int bad = 0;
  for (int64_t n = n0; n < n1; ++n) {
    orc_dequant_row(fmt, block, sdtype, codes + n * row_bytes, scales + n * nb,
                    biases ? biases + n * nb : NULL, K, wrow, &bad);
    for (int m = 0; m < M; ++m) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += wrow[k] * xv[(int64_t)m * K + k];
      y64[(int64_t)m * W + (n - n0)] = acc;
      y16[(int64_t)m * W + (n - n0)] = orc_double_to_half(acc, x_dtype);
    }
  }
  free(wrow);
  free(xv);
}
