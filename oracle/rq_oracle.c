/*
 * rq_oracle.c -- plain fp64 CPU reference of the ResidualQuant KV codec and of
 * decode attention over it.  TEST INFRASTRUCTURE ONLY (tests, smoke check and
 * the benchmark's CPU-baseline leg); the GPU library never links or calls it.
 *
 * Every routine follows a definition written out directly: nearest-value
 * rounding for the number formats, the Sylvester construction for the
 * Hadamard matrix, min/max asymmetric group quantization, the least-squares
 * scale, and textbook softmax attention.  No blocking, fusion or reordering.
 * Sources are cited per function with the tags explained in rq_oracle.h.
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes):
 *   R1 FP8 means OCP E4M3 "fn" (bias 7, no infinities, max 448), round to
 *      nearest with ties to even, saturating at +-448, sign of zero kept.
 *   R2 Quantization is asymmetric per group of g consecutive head_dim values:
 *      scale = fp8((max-min)/Q), offset = fp8(min), code = clamp(rne((x-offset)
 *      /scale), 0, Q) against the STORED fp8 scale and offset; scale 0 -> all
 *      codes 0.  ([ai4s p2]: "FP8 scales and offsets".)
 *   R3 The residual of loop l is x_l minus the DEQUANTIZED anchor ([agihunt]:
 *      "subtracts the anchor", "reconstruct one loop first, then store the
 *      difference").
 *   R4 The rotation is H = B*diag(signs) with B the Sylvester Walsh-Hadamard
 *      matrix scaled to be orthogonal; for d that is not a power of two, B is
 *      block diagonal over the binary decomposition of d, largest block first
 *      (d=96 -> 64+32).  It rotates residuals only, never the anchor
 *      ([ai4s p1]: "rotations applied to the residuals rather than to the KV
 *      states").
 *   R5 One BF16 least-squares coefficient alpha per residual d-vector scales
 *      the dequantized residual: alpha = <y,yhat>/<yhat,yhat> ([abstract]:
 *      "least-square scaling"; [ai4s p2]: "BF16 least-squares coefficients
 *      stored for residuals"); 0 when yhat = 0.
 *   R11 The chained ("previous-loop") reference of the ablation ([ai4s p3]:
 *      chained reconstruction grows with the distance from the anchor): loop
 *      l < a of a group takes its residual against the reconstruction of loop
 *      l+1, the anchor ending the chain, so reconstructing loop j reads the
 *      anchor and the residuals of loops j..a-1.  Because H is linear, the
 *      rotated residual is H(x_l - deq(A)) minus the sum of alpha_i yhat_i
 *      over i = a-1 down to l+1, and it is computed in that form.
 */
#include "rq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Number formats                                                            */
/* ------------------------------------------------------------------------- */

/* OCP FP8 E4M3 "fn": 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; there is
 * no infinity.  Reading R1. */
double rqo_fp8_decode(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 7;
  double mag;
  if (e == 0xF && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Nearest finite E4M3fn value by exhaustive search over the 127 non-negative
 * finite codes; on an exact tie the code with the even mantissa bit wins;
 * magnitudes beyond 448 saturate to 448 (the nearest finite value).  The sign
 * of the input is kept, so negative values that round to zero give 0x80. */
uint8_t rqo_fp8_encode(double x) {
  if (isnan(x)) return 0x7F;
  double a = fabs(x);
  uint8_t best = 0;
  double bestd = a;
  for (int c = 1; c <= 0x7E; ++c) {
    double dist = fabs(a - rqo_fp8_decode((uint8_t)c));
    if (dist < bestd || (dist == bestd && (c & 1) == 0)) {
      best = (uint8_t)c;
      bestd = dist;
    }
  }
  return (uint8_t)((signbit(x) ? 0x80 : 0x00) | best);
}

/* BF16 is the upper half of an IEEE binary32 pattern. */
double rqo_bf16_decode(uint16_t code) {
  uint32_t bits = (uint32_t)code << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Nearest BF16 value of a double, ties to even, computed directly from the
 * double (no intermediate binary32 rounding): BF16 keeps 8 significant bits,
 * so within [2^E, 2^(E+1)) its spacing is 2^(E-7); below 2^-126 the spacing is
 * fixed at 2^-133 (subnormals).  Overflow rounds to infinity. */
uint16_t rqo_bf16_encode(double x) {
  if (isnan(x)) return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
  double a = fabs(x);
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);       /* a in [2^(e2-1), 2^e2) */
  int E = e2 - 1;
  if (E < -126) E = -126;
  double quantum = ldexp(1.0, E - 7);
  double k = nearbyint(a / quantum); /* power-of-two division is exact */
  double r = k * quantum;
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
  float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t bits;
  memcpy(&bits, &f, sizeof bits);
  return (uint16_t)(sign | (uint16_t)((bits >> 16) & 0x7FFF));
}

void rqo_fp8_decode_n(const uint8_t* in, long n, double* out) {
  for (long i = 0; i < n; ++i) out[i] = rqo_fp8_decode(in[i]);
}
void rqo_fp8_encode_n(const double* in, long n, uint8_t* out) {
  for (long i = 0; i < n; ++i) out[i] = rqo_fp8_encode(in[i]);
}
void rqo_bf16_decode_n(const uint16_t* in, long n, double* out) {
  for (long i = 0; i < n; ++i) out[i] = rqo_bf16_decode(in[i]);
}
void rqo_bf16_encode_n(const double* in, long n, uint16_t* out) {
  for (long i = 0; i < n; ++i) out[i] = rqo_bf16_encode(in[i]);
}

/* ------------------------------------------------------------------------- */
/* Rotation (reading R4)                                                     */
/* ------------------------------------------------------------------------- */

/* Sylvester construction: S_1 = [1], S_2k = [[S_k, S_k], [S_k, -S_k]]. */
static void sylvester(int n, double* S /* n*n */) {
  S[0] = 1.0;
  for (int k = 1; k < n; k *= 2) {
    for (int i = 0; i < k; ++i)
      for (int j = 0; j < k; ++j) {
        double v = S[i * n + j];
        S[i * n + (j + k)] = v;
        S[(i + k) * n + j] = v;
        S[(i + k) * n + (j + k)] = -v;
      }
  }
}

int rqo_rotation_matrix(int d, const int8_t* signs, double* H) {
  if (d <= 0) return -1;
  memset(H, 0, sizeof(double) * (size_t)d * (size_t)d);
  int off = 0;
  for (int bit = 30; bit >= 0; --bit) {
    int n = 1 << bit;
    if (!(d & n)) continue;
    double* S = (double*)malloc(sizeof(double) * (size_t)n * (size_t)n);
    if (!S) return -2;
    sylvester(n, S);
    double inv = 1.0 / sqrt((double)n);
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < n; ++j)
        H[(size_t)(off + i) * d + (off + j)] = S[(size_t)i * n + j] * inv;
    free(S);
    off += n;
  }
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) H[(size_t)i * d + j] *= (double)signs[j];
  return 0;
}

/* A rotation of dimension d as its definition factors it: per block of the
 * binary decomposition of d, the Sylvester matrix S_n (entries +-1) and the
 * scale 1/sqrt(n); the signs multiply the input.  Applying it as the +-1 sum
 * followed by one multiplication by 1/sqrt(n) keeps the sum exact, so an exact
 * zero stays an exact zero and a rounding tie downstream is decided on the
 * exact value. */
typedef struct {
  int d, nblk;
  int off[32], n[32];
  double inv[32];
  double* S[32];
  const int8_t* signs;
} rot_t;

static void rot_free(rot_t* R) {
  for (int b = 0; b < R->nblk; ++b) free(R->S[b]);
  R->nblk = 0;
}

static int rot_init(rot_t* R, int d, const int8_t* signs) {
  memset(R, 0, sizeof *R);
  R->d = d;
  R->signs = signs;
  int off = 0;
  for (int bit = 30; bit >= 0; --bit) {
    int n = 1 << bit;
    if (!(d & n)) continue;
    double* S = (double*)malloc(sizeof(double) * (size_t)n * (size_t)n);
    if (!S) {
      rot_free(R);
      return -2;
    }
    sylvester(n, S);
    R->off[R->nblk] = off;
    R->n[R->nblk] = n;
    R->inv[R->nblk] = 1.0 / sqrt((double)n);
    R->S[R->nblk] = S;
    R->nblk++;
    off += n;
  }
  return 0;
}

/* y = B diag(signs) r */
static void rot_apply(const rot_t* R, const double* r, double* y) {
  for (int b = 0; b < R->nblk; ++b) {
    const int n = R->n[b], o = R->off[b];
    for (int i = 0; i < n; ++i) {
      double acc = 0.0;
      for (int j = 0; j < n; ++j) acc += R->S[b][(size_t)i * n + j] * (R->signs[o + j] * r[o + j]);
      y[o + i] = acc * R->inv[b];
    }
  }
}

/* r = diag(signs) B^T y */
static void rot_apply_t(const rot_t* R, const double* y, double* r) {
  for (int b = 0; b < R->nblk; ++b) {
    const int n = R->n[b], o = R->off[b];
    for (int j = 0; j < n; ++j) {
      double acc = 0.0;
      for (int i = 0; i < n; ++i) acc += R->S[b][(size_t)i * n + j] * y[o + i];
      r[o + j] = R->signs[o + j] * (acc * R->inv[b]);
    }
  }
}

int rqo_rotate(int d, const int8_t* signs, const double* r, double* y) {
  rot_t R;
  if (d <= 0 || rot_init(&R, d, signs)) return -1;
  rot_apply(&R, r, y);
  rot_free(&R);
  return 0;
}

int rqo_rotate_t(int d, const int8_t* signs, const double* y, double* r) {
  rot_t R;
  if (d <= 0 || rot_init(&R, d, signs)) return -1;
  rot_apply_t(&R, y, r);
  rot_free(&R);
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Group quantizer (reading R2; [ai4s p1], [ai4s p2], [agihunt])             */
/* ------------------------------------------------------------------------- */

void rqo_quant_group(const double* x, int g, int bits, uint8_t* s8, uint8_t* z8,
                     uint8_t* codes) {
  int Q = (1 << bits) - 1;
  double mn = x[0], mx = x[0];
  for (int i = 1; i < g; ++i) {
    if (x[i] < mn) mn = x[i];
    if (x[i] > mx) mx = x[i];
  }
  *s8 = rqo_fp8_encode((mx - mn) / Q);
  *z8 = rqo_fp8_encode(mn);
  double s = rqo_fp8_decode(*s8);
  double z = rqo_fp8_decode(*z8);
  for (int i = 0; i < g; ++i) {
    int c = 0;
    if (s != 0.0) {
      double t = nearbyint((x[i] - z) / s);
      if (t < 0) t = 0;
      if (t > Q) t = Q;
      c = (int)t;
    }
    codes[i] = (uint8_t)c;
  }
}

void rqo_quant_vector(const double* x, int d, int g, int bits, uint8_t* codes,
                      uint8_t* s8, uint8_t* z8) {
  for (int j = 0; j < d / g; ++j)
    rqo_quant_group(x + j * g, g, bits, s8 + j, z8 + j, codes + j * g);
}

void rqo_dequant_vector(const uint8_t* codes, const uint8_t* s8, const uint8_t* z8,
                        int d, int g, double* out) {
  for (int i = 0; i < d; ++i) {
    double s = rqo_fp8_decode(s8[i / g]);
    double z = rqo_fp8_decode(z8[i / g]);
    out[i] = s * codes[i] + z;
  }
}

/* ------------------------------------------------------------------------- */
/* One loop group of one token vector                                        */
/* ------------------------------------------------------------------------- */

static int params_ok(const rqo_params* p) {
  if (!p || p->d <= 0 || p->g <= 0 || p->d % p->g || p->P <= 0 || p->d > 4096) return 0;
  if (p->anchor_bits < 1 || p->anchor_bits > 8) return 0;
  if (p->residual_bits < 1 || p->residual_bits > 8) return 0;
  if (p->mode != RQO_MODE_RESIDUAL && p->mode != RQO_MODE_DIRECT && p->mode != RQO_MODE_CHAINED)
    return 0;
  return 1;
}

static int uses_rotation(const rqo_params* p) {
  return p->mode != RQO_MODE_DIRECT && p->rotate;
}

/* Rotation of a parameter set: initialized only when residuals are rotated. */
static int rot_for(const rqo_params* p, const int8_t* signs, rot_t* R) {
  memset(R, 0, sizeof *R);
  if (!uses_rotation(p)) return 0;
  if (!signs) return -1;
  return rot_init(R, p->d, signs);
}

/* Anchor = last loop of the group ([abstract]: "uses the final-loop KV states
 * as a reference"; [ai4s p1]: "final-loop KV as a shared anchor").  Residual
 * mode: the anchor is stored at anchor_bits without rotation; every other
 * loop l stores y = H (x_l - deq(anchor)) at residual_bits plus alpha
 * (readings R3-R5; [ai4s p1]: "INT4 for the anchor and INT2 for residuals").
 * Direct mode: every loop is quantized on its own, the anchor-position loop at
 * anchor_bits and the others at residual_bits ([ai4s p2]: "direct
 * quantization"). */
static int encode_group_r(const rqo_params* p, const double* x, const rot_t* R,
                          uint8_t* codes, uint8_t* s8, uint8_t* z8, uint16_t* alpha) {
  const int d = p->d, g = p->g, P = p->P, ng = d / g, a = P - 1;
  double* A = (double*)malloc(sizeof(double) * d * 4);
  if (!A) return -2;
  double* r = A + d;
  double* y = A + 2 * d;
  double* yh = A + 3 * d;

  rqo_quant_vector(x + a * d, d, g, p->anchor_bits, codes + a * d, s8 + a * ng, z8 + a * ng);
  rqo_dequant_vector(codes + a * d, s8 + a * ng, z8 + a * ng, d, g, A);
  alpha[a] = 0;

  if (p->mode == RQO_MODE_CHAINED) {
    /* reading R11: from the loop next to the anchor outwards; corr holds
     * sum alpha_i yhat_i over the loops already stored, largest i first */
    double* corr = (double*)calloc((size_t)d, sizeof(double));
    if (!corr) {
      free(A);
      return -2;
    }
    for (int l = P - 2; l >= 0; --l) {
      for (int i = 0; i < d; ++i) r[i] = x[l * d + i] - A[i];
      if (p->rotate)
        rot_apply(R, r, y);
      else
        memcpy(y, r, sizeof(double) * d);
      for (int i = 0; i < d; ++i) y[i] -= corr[i];
      rqo_quant_vector(y, d, g, p->residual_bits, codes + l * d, s8 + l * ng, z8 + l * ng);
      rqo_dequant_vector(codes + l * d, s8 + l * ng, z8 + l * ng, d, g, yh);
      double num = 0.0, den = 0.0, yy = 0.0;
      for (int i = 0; i < d; ++i) {
        num += y[i] * yh[i];
        den += yh[i] * yh[i];
        yy += y[i] * y[i];
      }
      double al;
      if (p->alpha_mode == RQO_ALPHA_ONE)
        al = 1.0;
      else if (den <= 0.0)
        al = 0.0;
      else if (p->alpha_mode == RQO_ALPHA_NORM_RATIO)
        al = sqrt(yy) / sqrt(den);
      else
        al = num / den;
      alpha[l] = rqo_bf16_encode(al);
      const double ab = rqo_bf16_decode(alpha[l]);
      for (int i = 0; i < d; ++i) corr[i] += ab * yh[i];
    }
    free(corr);
    free(A);
    return 0;
  }

  for (int l = 0; l < P - 1; ++l) {
    if (p->mode == RQO_MODE_DIRECT) {
      rqo_quant_vector(x + l * d, d, g, p->residual_bits, codes + l * d, s8 + l * ng, z8 + l * ng);
      alpha[l] = 0;
      continue;
    }
    for (int i = 0; i < d; ++i) r[i] = x[l * d + i] - A[i];
    if (p->rotate)
      rot_apply(R, r, y);
    else
      memcpy(y, r, sizeof(double) * d);
    rqo_quant_vector(y, d, g, p->residual_bits, codes + l * d, s8 + l * ng, z8 + l * ng);
    rqo_dequant_vector(codes + l * d, s8 + l * ng, z8 + l * ng, d, g, yh);
    double num = 0.0, den = 0.0, yy = 0.0;
    for (int i = 0; i < d; ++i) {
      num += y[i] * yh[i];
      den += yh[i] * yh[i];
      yy += y[i] * y[i];
    }
    double al;
    if (p->alpha_mode == RQO_ALPHA_ONE)
      al = 1.0;
    else if (den <= 0.0)
      al = 0.0;
    else if (p->alpha_mode == RQO_ALPHA_NORM_RATIO)
      al = sqrt(yy) / sqrt(den);
    else
      al = num / den;
    alpha[l] = rqo_bf16_encode(al);
  }
  free(A);
  return 0;
}

int rqo_encode_group(const rqo_params* p, const double* x, const int8_t* signs,
                     uint8_t* codes, uint8_t* s8, uint8_t* z8, uint16_t* alpha) {
  if (!params_ok(p)) return -1;
  rot_t R;
  if (rot_for(p, signs, &R)) return -1;
  int rc = encode_group_r(p, x, &R, codes, s8, z8, alpha);
  rot_free(&R);
  return rc;
}

/* Shared-anchor reconstruction from exactly two stored pieces, the anchor and
 * the loop's own residual ([ai4s p3]: "shared-anchor reconstruction ... needs
 * only two KV cache reads"; [agihunt]: "reads back the anchor plus the
 * residuals"): xhat_l = deq(anchor) + alpha_l * H^T deq(residual_l). */
static int reconstruct_group_r(const rqo_params* p, const uint8_t* codes, const uint8_t* s8,
                               const uint8_t* z8, const uint16_t* alpha, const rot_t* R, int j,
                               double* out) {
  const int d = p->d, g = p->g, ng = d / g, a = p->P - 1;
  if (p->mode == RQO_MODE_DIRECT || j == a) {
    rqo_dequant_vector(codes + j * d, s8 + j * ng, z8 + j * ng, d, g, out);
    return 0;
  }
  double* A = (double*)malloc(sizeof(double) * d * 4);
  if (!A) return -2;
  double* yh = A + d;
  double* rh = A + 2 * d;
  rqo_dequant_vector(codes + a * d, s8 + a * ng, z8 + a * ng, d, g, A);
  if (p->mode == RQO_MODE_CHAINED) {
    /* reading R11: deq(anchor) + H^T sum_{i = a-1 .. j} alpha_i yhat_i, the
     * anchor and the residuals of loops j..a-1 (distance + 1 reads) */
    double* sum = A + 3 * d;
    memset(sum, 0, sizeof(double) * d);
    for (int i = a - 1; i >= j; --i) {
      rqo_dequant_vector(codes + i * d, s8 + i * ng, z8 + i * ng, d, g, yh);
      const double al = rqo_bf16_decode(alpha[i]);
      for (int e = 0; e < d; ++e) sum[e] += al * yh[e];
    }
    if (p->rotate)
      rot_apply_t(R, sum, rh);
    else
      memcpy(rh, sum, sizeof(double) * d);
    for (int e = 0; e < d; ++e) out[e] = A[e] + rh[e];
    free(A);
    return 0;
  }
  rqo_dequant_vector(codes + j * d, s8 + j * ng, z8 + j * ng, d, g, yh);
  if (p->rotate)
    rot_apply_t(R, yh, rh);
  else
    memcpy(rh, yh, sizeof(double) * d);
  double al = rqo_bf16_decode(alpha[j]);
  for (int i = 0; i < d; ++i) out[i] = A[i] + al * rh[i];
  free(A);
  return 0;
}

int rqo_reconstruct_group(const rqo_params* p, const uint8_t* codes, const uint8_t* s8,
                          const uint8_t* z8, const uint16_t* alpha, const int8_t* signs,
                          int j, double* out) {
  if (!params_ok(p) || j < 0 || j >= p->P) return -1;
  rot_t R;
  if (rot_for(p, signs, &R)) return -1;
  int rc = reconstruct_group_r(p, codes, s8, z8, alpha, &R, j, out);
  rot_free(&R);
  return rc;
}

/* ------------------------------------------------------------------------- */
/* Slices                                                                    */
/* ------------------------------------------------------------------------- */

int rqo_encode_slice(const rqo_params* p, int L, int N, const uint16_t* x, const int8_t* signs,
                     uint8_t* codes, uint8_t* s8, uint8_t* z8, uint16_t* alpha) {
  if (!params_ok(p) || L <= 0 || L % p->P || N < 0) return -1;
  const int d = p->d, P = p->P, ng = d / p->g;
  rot_t R;
  if (rot_for(p, signs, &R)) return -1;
  double* xg = (double*)malloc(sizeof(double) * P * d);
  uint8_t* cg = (uint8_t*)malloc((size_t)P * d);
  uint8_t* sg = (uint8_t*)malloc((size_t)P * ng);
  uint8_t* zg = (uint8_t*)malloc((size_t)P * ng);
  uint16_t* ag = (uint16_t*)malloc(sizeof(uint16_t) * P);
  int rc = (!xg || !cg || !sg || !zg || !ag) ? -2 : 0;
  for (int k = 0; k < L / P && rc == 0; ++k) {
    for (int t = 0; t < N && rc == 0; ++t) {
      for (int j = 0; j < P; ++j) {
        const uint16_t* src = x + ((size_t)(k * P + j) * N + t) * d;
        for (int i = 0; i < d; ++i) xg[j * d + i] = rqo_bf16_decode(src[i]);
      }
      rc = encode_group_r(p, xg, &R, cg, sg, zg, ag);
      for (int j = 0; j < P; ++j) {
        size_t v = (size_t)(k * P + j) * N + t;
        memcpy(codes + v * d, cg + j * d, (size_t)d);
        memcpy(s8 + v * ng, sg + j * ng, (size_t)ng);
        memcpy(z8 + v * ng, zg + j * ng, (size_t)ng);
        alpha[v] = ag[j];
      }
    }
  }
  free(xg); free(cg); free(sg); free(zg); free(ag);
  rot_free(&R);
  return rc;
}

/* Gathers the loop group of `loop` for token t into [P][..] scratch arrays. */
static void gather_group(const rqo_params* p, int N, int loop, int t, const uint8_t* codes,
                         const uint8_t* s8, const uint8_t* z8, const uint16_t* alpha,
                         uint8_t* cg, uint8_t* sg, uint8_t* zg, uint16_t* ag) {
  const int d = p->d, P = p->P, ng = d / p->g, k = loop / P;
  for (int j = 0; j < P; ++j) {
    size_t v = (size_t)(k * P + j) * N + t;
    memcpy(cg + j * d, codes + v * d, (size_t)d);
    memcpy(sg + j * ng, s8 + v * ng, (size_t)ng);
    memcpy(zg + j * ng, z8 + v * ng, (size_t)ng);
    ag[j] = alpha[v];
  }
}

static int reconstruct_slice_r(const rqo_params* p, int N, const uint8_t* codes,
                               const uint8_t* s8, const uint8_t* z8, const uint16_t* alpha,
                               const rot_t* R, int loop, int t0, int t1, double* out) {
  const int d = p->d, P = p->P, ng = d / p->g;
  uint8_t* cg = (uint8_t*)malloc((size_t)P * d);
  uint8_t* sg = (uint8_t*)malloc((size_t)P * ng);
  uint8_t* zg = (uint8_t*)malloc((size_t)P * ng);
  uint16_t* ag = (uint16_t*)malloc(sizeof(uint16_t) * P);
  int rc = (!cg || !sg || !zg || !ag) ? -2 : 0;
  for (int t = t0; t < t1 && rc == 0; ++t) {
    gather_group(p, N, loop, t, codes, s8, z8, alpha, cg, sg, zg, ag);
    rc = reconstruct_group_r(p, cg, sg, zg, ag, R, loop % P, out + (size_t)(t - t0) * d);
  }
  free(cg); free(sg); free(zg); free(ag);
  return rc;
}

int rqo_reconstruct_slice(const rqo_params* p, int L, int N, const uint8_t* codes,
                          const uint8_t* s8, const uint8_t* z8, const uint16_t* alpha,
                          const int8_t* signs, int loop, int t0, int t1, double* out) {
  if (!params_ok(p) || L <= 0 || L % p->P || loop < 0 || loop >= L || t0 < 0 || t1 > N ||
      t0 > t1)
    return -1;
  rot_t R;
  if (rot_for(p, signs, &R)) return -1;
  int rc = reconstruct_slice_r(p, N, codes, s8, z8, alpha, &R, loop, t0, t1, out);
  rot_free(&R);
  return rc;
}

/* ------------------------------------------------------------------------- */
/* Attention                                                                 */
/* ------------------------------------------------------------------------- */

/* Textbook single-query softmax attention: logit_t = scale * <q, K_t>,
 * out = sum_t softmax(logit)_t V_t, with the maximum subtracted before exp. */
int rqo_attention_dense(int n, int d, const double* q, const double* Khat, const double* Vhat,
                        double scale, double* out) {
  for (int i = 0; i < d; ++i) out[i] = 0.0;
  if (n <= 0) return 0;
  double* lg = (double*)malloc(sizeof(double) * (size_t)n);
  if (!lg) return -2;
  double m = -INFINITY;
  for (int t = 0; t < n; ++t) {
    double acc = 0.0;
    for (int i = 0; i < d; ++i) acc += q[i] * Khat[(size_t)t * d + i];
    lg[t] = scale * acc;
    if (lg[t] > m) m = lg[t];
  }
  double l = 0.0;
  for (int t = 0; t < n; ++t) {
    double w = exp(lg[t] - m);
    l += w;
    for (int i = 0; i < d; ++i) out[i] += w * Vhat[(size_t)t * d + i];
  }
  for (int i = 0; i < d; ++i) out[i] /= l;
  free(lg);
  return 0;
}

/* Attention of one BF16 query for loop `loop` over tokens [0, n) of a slice.
 * fused == 0: reconstruct K and V (two reads per token) and run the textbook
 * form.  fused == 1: the same quantity rearranged so nothing is
 * reconstructed: q.deq(A_t) + alpha_t (H q).deq(R_t) per group as
 * s*sum(q*c) + z*sum(q), and H^T applied once to sum_t p_t alpha_t deq(R_t).
 * Both must agree to rounding. */
int rqo_attention_slice(const rqo_params* p, int L, int N, int n, int loop,
                        const uint16_t* q_bf16, const int8_t* signs_k, const int8_t* signs_v,
                        const uint8_t* kc, const uint8_t* ks, const uint8_t* kz,
                        const uint16_t* ka, const uint8_t* vc, const uint8_t* vs,
                        const uint8_t* vz, const uint16_t* va, double scale, int fused,
                        double* out) {
  if (!params_ok(p) || L <= 0 || L % p->P || loop < 0 || loop >= L || n < 0 || n > N)
    return -1;
  const int d = p->d, g = p->g, ng = d / g, P = p->P;
  rot_t RK, RV;
  if (rot_for(p, signs_k, &RK)) return -1;
  if (rot_for(p, signs_v, &RV)) {
    rot_free(&RK);
    return -1;
  }
  double* q = (double*)malloc(sizeof(double) * d);
  double* Kh = NULL;
  double* Vh = NULL;
  double* u = (double*)malloc(sizeof(double) * d);
  double* lg = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double* accA = (double*)calloc((size_t)d, sizeof(double));
  double* accR = (double*)calloc((size_t)d, sizeof(double));
  double* tmp = (double*)malloc(sizeof(double) * d);
  int rc = (!q || !u || !lg || !accA || !accR || !tmp) ? -2 : 0;
  if (rc == 0)
    for (int i = 0; i < d; ++i) q[i] = rqo_bf16_decode(q_bf16[i]);

  if (rc == 0 && !fused) {
    Kh = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * d);
    Vh = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * d);
    rc = (!Kh || !Vh) ? -2 : 0;
    if (!rc) rc = reconstruct_slice_r(p, N, kc, ks, kz, ka, &RK, loop, 0, n, Kh);
    if (!rc) rc = reconstruct_slice_r(p, N, vc, vs, vz, va, &RV, loop, 0, n, Vh);
    if (!rc) rc = rqo_attention_dense(n, d, q, Kh, Vh, scale, out);
  } else if (rc == 0) {
    const int j = loop % P, a = P - 1;
    const int two = (p->mode != RQO_MODE_DIRECT && j != a);
    const int own = (p->mode == RQO_MODE_DIRECT) ? loop : (loop - j + a); /* first plane */
    /* residual planes read for this loop: its own (residual mode) or those of
     * loops j..a-1 of the group (chained mode, reading R11) */
    const int r_last = (p->mode == RQO_MODE_CHAINED) ? loop - j + a - 1 : loop;
    if (two && p->rotate)
      rot_apply(&RK, q, u);
    else
      memcpy(u, q, sizeof(double) * d);

    double m = -INFINITY;
    for (int t = 0; t < n; ++t) {
      size_t vA = (size_t)own * N + t;
      double la = 0.0;
      for (int gi = 0; gi < ng; ++gi) {
        double sq = 0.0, sqc = 0.0;
        for (int i = gi * g; i < (gi + 1) * g; ++i) {
          sq += q[i];
          sqc += q[i] * kc[vA * d + i];
        }
        la += rqo_fp8_decode(ks[vA * ng + gi]) * sqc + rqo_fp8_decode(kz[vA * ng + gi]) * sq;
      }
      double lr = 0.0;
      for (int rl = loop; two && rl <= r_last; ++rl) {
        size_t vR = (size_t)rl * N + t;
        double lp = 0.0;
        for (int gi = 0; gi < ng; ++gi) {
          double su = 0.0, suc = 0.0;
          for (int i = gi * g; i < (gi + 1) * g; ++i) {
            su += u[i];
            suc += u[i] * kc[vR * d + i];
          }
          lp += rqo_fp8_decode(ks[vR * ng + gi]) * suc + rqo_fp8_decode(kz[vR * ng + gi]) * su;
        }
        lr += rqo_bf16_decode(ka[vR]) * lp;
      }
      lg[t] = scale * (la + lr);
      if (lg[t] > m) m = lg[t];
    }
    double l = 0.0;
    for (int t = 0; t < n; ++t) {
      double w = exp(lg[t] - m);
      l += w;
      size_t vA = (size_t)own * N + t;
      for (int i = 0; i < d; ++i)
        accA[i] += w * (rqo_fp8_decode(vs[vA * ng + i / g]) * vc[vA * d + i] +
                        rqo_fp8_decode(vz[vA * ng + i / g]));
      for (int rl = loop; two && rl <= r_last; ++rl) {
        size_t vR = (size_t)rl * N + t;
        double al = rqo_bf16_decode(va[vR]);
        for (int i = 0; i < d; ++i)
          accR[i] += w * al *
                     (rqo_fp8_decode(vs[vR * ng + i / g]) * vc[vR * d + i] +
                      rqo_fp8_decode(vz[vR * ng + i / g]));
      }
    }
    if (two && p->rotate)
      rot_apply_t(&RV, accR, tmp);
    else
      memcpy(tmp, accR, sizeof(double) * d);
    for (int i = 0; i < d; ++i) out[i] = (n > 0) ? (accA[i] + tmp[i]) / l : 0.0;
  }
  free(q); free(u); free(lg); free(accA); free(accR); free(tmp); free(Kh); free(Vh);
  rot_free(&RK);
  rot_free(&RV);
  return rc;
}

/* ------------------------------------------------------------------------- */
/* Storage accounting ([abstract] and [ai4s p2]: effective bitwidth counts the */
/* codes, the FP8 scales and offsets, and the BF16 least-squares coefficients) */
/* ------------------------------------------------------------------------- */

/* Average stored bits per KV element over a loop group of P loops: the anchor
 * carries its codes plus one FP8 scale and one FP8 offset per group of g; each
 * of the other P-1 loops carries its codes, the same per-group pair, and (when
 * with_alpha) one BF16 coefficient per d-vector. */
double rqo_bits_per_element(int anchor_bits, int residual_bits, int g, int d, int P,
                            int with_alpha) {
  double per_group = 16.0 / g;
  double anchor = anchor_bits + per_group;
  double other = residual_bits + per_group + (with_alpha ? 16.0 / d : 0.0);
  return (anchor + (P - 1) * other) / P;
}
