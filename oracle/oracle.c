/*
 * oracle.c -- plain fp64 CPU reference for the grouped / mixed-input /
 * implicit-convolution GEMM library.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library links, loads or calls this
 * file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * do.  It shares no code, header or table with the HIP sources.
 *
 * Every routine reads the *stored* element bytes (fp16 / bf16 bit patterns,
 * uint4 nibbles), converts them exactly to double, and returns the unrounded
 * fp64 result of the plain mathematical definition.  Products of two fp16 or
 * bf16 values are exact in double; sums over K <= 2^16 terms carry a relative
 * error far below the fp16/bf16 output tolerance.  The only rounding routine,
 * ora_round, exists for bit-exact pins.
 *
 * Sources (the pages these definitions restate):
 *   [p1] sm90_gemm_array_tma_warpspecialized_cooperative.hpp -- grouped and
 *        pointer-array problem modes (Arguments, can_implement), per-problem
 *        shape (M,N,K) with strides [M,K,L] / [N,K,L] / [M,N,L], fp32
 *        accumulator fragment, epilogue store of the accumulators.
 *   [p2] machete_mainloop.cuh -- ConversionMode ConvertAndScaleWithZero,
 *        scale_k = ceil(K / group_size) (to_underlying_arguments), the scale
 *        column chosen per k-tile (load), convert / scale / zero in
 *        transform_A_kblock, round-to-nearest conversion (convert_tensor).
 *   [p3] sm100_implicit_gemm_umma_warpspecialized.hpp -- fprop over an
 *        activation addressed through im2col with lower/upper padding,
 *        traversal stride and dilation (get_tma_load_a_instance), linearised
 *        GEMM shape (get_problem_shape_MNKL), cross-correlation only and
 *        channel-innermost layouts (can_implement).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORA_F16 0
#define ORA_BF16 1
#define ORA_F8 2 /* OCP fp8 E4M3: A and B of the fp8 GEMM, one byte per element */

/* ------------------------------------------------------------------------
 * Element decoding: IEEE-754 binary16 and bfloat16 (the upper half of
 * binary32), written from the encodings' definitions.
 * ------------------------------------------------------------------------ */
double ora_f16_to_f64(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/2^10) * 2^(e-15) */
  return s ? -v : v;
}

double ora_bf16_to_f64(uint16_t b) {
  int s = b >> 15, e = (b >> 7) & 255, m = b & 127;
  double v;
  if (e == 0)
    v = ldexp((double)m, -133); /* subnormal: m * 2^-133 */
  else if (e == 255)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(128 + m), e - 134); /* (1 + m/2^7) * 2^(e-127) */
  return s ? -v : v;
}

/* OCP 8-bit floating point E4M3 ("fn": finite, no infinities): sign 1,
 * exponent 4 with bias 7, mantissa 3; exponent 0 holds the subnormals
 * m * 2^-9; S.1111.111 is NaN, so the largest finite value is 1.75 * 2^8. */
double ora_e4m3_to_f64(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9); /* subnormal: (m / 8) * 2^(1-7) */
  else
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

static double dec(uint16_t v, int dt) {
  if (dt == ORA_F8) return ora_e4m3_to_f64((uint8_t)(v & 0xFFu));
  return dt == ORA_BF16 ? ora_bf16_to_f64(v) : ora_f16_to_f64(v);
}

void ora_decode(const uint16_t* in, int64_t n, int32_t dt, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = dec(in[i], dt);
}

/* Round a double to the nearest representable value of a format with
 * `mbits` explicit mantissa bits, minimum normal exponent `emin` and maximum
 * exponent `emax`, ties to even (the default rounding mode of nearbyint).
 * Returns the bit pattern. */
static uint16_t round_fmt(double x, int mbits, int emin, int emax, int ebias) {
  uint16_t sign = signbit(x) ? 0x8000u : 0; /* both formats keep the sign in bit 15 */
  int ebits = 15 - mbits;
  uint16_t inf = (uint16_t)(((1u << ebits) - 1u) << mbits);
  double a = fabs(x);
  if (isnan(x)) return (uint16_t)(sign | inf | (1u << (mbits - 1)));
  if (a == 0.0) return sign;
  /* largest finite value is (2 - 2^-mbits) * 2^emax; the halfway point to
   * 2^(emax+1) rounds to the even neighbour 2^(emax+1), i.e. overflows */
  double halfway = ldexp(2.0 - ldexp(1.0, -(mbits + 1)), emax);
  if (a >= halfway) return sign | inf;
  int e2;
  frexp(a, &e2);
  int E = e2 - 1; /* a in [2^E, 2^(E+1)) */
  double quantum = (E < emin) ? ldexp(1.0, emin - mbits) : ldexp(1.0, E - mbits);
  double r = nearbyint(a / quantum) * quantum;
  if (r == 0.0) return sign;
  if (r < ldexp(1.0, emin)) /* subnormal */
    return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, emin - mbits)));
  frexp(r, &e2);
  E = e2 - 1;
  if (E > emax) return sign | inf;
  uint16_t mant = (uint16_t)((r / ldexp(1.0, E) - 1.0) * ldexp(1.0, mbits));
  return (uint16_t)(sign | ((uint16_t)(E + ebias) << mbits) | mant);
}

void ora_round(const double* in, int64_t n, int32_t dt, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = (dt == ORA_BF16) ? round_fmt(in[i], 7, -126, 127, 127) : round_fmt(in[i], 10, -14, 15, 15);
}

/* ------------------------------------------------------------------------
 * GEMM [p1]: one problem of a grouped or pointer-array list.
 *   out[m*ldo + n] = alpha * sum_{k<K} A[m][k] * B[k][n] + beta * C[m][n]
 * A and B elements arrive as uint16 codes: fp16 / bf16 bit patterns, or an
 * fp8 E4M3 byte zero-extended (dt_ab == ORA_F8); C is of type dt_c.
 * A row-major (A[m][k] at A[m*lda + k]); B column-major (B[k][n] at
 * B[n*ldb + k]); C row-major (C[m][n] at C[m*ldc + n]); the C term is
 * omitted when beta == 0 (C may then be NULL).
 * Returns 0, or -1 on an invalid argument.
 * ------------------------------------------------------------------------ */
int ora_gemm(int32_t M, int32_t N, int32_t K, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
             const uint16_t* C, int64_t ldc, int32_t dt_ab, int32_t dt_c, double alpha, double beta, double* out,
             int64_t ldo) {
  if (M < 0 || N < 0 || K < 0) return -1;
  if (M == 0 || N == 0) return 0;
  if (beta != 0.0 && !C) return -1;
  double* a = (double*)malloc(sizeof(double) * (size_t)M * (size_t)(K ? K : 1));
  double* b = (double*)malloc(sizeof(double) * (size_t)N * (size_t)(K ? K : 1));
  if (!a || !b) {
    free(a);
    free(b);
    return -1;
  }
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) a[m * K + k] = dec(A[m * lda + k], dt_ab);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) b[n * K + k] = dec(B[n * ldb + k], dt_ab);
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += a[m * K + k] * b[n * K + k];
      double v = alpha * acc;
      if (beta != 0.0) v += beta * dec(C[m * ldc + n], dt_c);
      out[m * ldo + n] = v;
    }
  }
  free(a);
  free(b);
  return 0;
}

/* ------------------------------------------------------------------------
 * Mixed-input weights [p2], conversion mode "convert, scale, with zero".
 *   W logically [N][K] uint4: w_u4[n*(K/2) + k/2], even k in the low nibble.
 *   scales [ceil(K/g)][N] fp16, n contiguous (MN-major).
 *   zeros  [ceil(K/g)][ceil(N/2)] uint4, even n in the low nibble.
 *   w[n][k] = (q[n][k] - z[k/g][n]) * s[k/g][n]     (exact in double)
 * ------------------------------------------------------------------------ */
static int nib(const uint8_t* p, int64_t idx) { return (p[idx >> 1] >> ((idx & 1) * 4)) & 15; }

int ora_dequant_w4(int32_t N, int32_t K, const uint8_t* w_u4, const uint16_t* scales, const uint8_t* zeros,
                   int32_t g, double* wout) {
  if (N < 0 || K < 0 || g <= 0 || (K & 1)) return -1;
  int64_t kh = K / 2, nz = (N + 1) / 2;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      int64_t grp = k / g;
      int q = nib(w_u4 + n * kh, k);
      int z = nib(zeros + grp * nz, n);
      double s = ora_f16_to_f64(scales[grp * N + n]);
      wout[n * K + k] = (double)(q - z) * s;
    }
  return 0;
}

/* Y = X W^T with the weights above; X [M][ldx] fp16 row-major, out [M][N]. */
int ora_w4a16(int32_t M, int32_t N, int32_t K, const uint16_t* X, int64_t ldx, const uint8_t* w_u4,
              const uint16_t* scales, const uint8_t* zeros, int32_t g, double* out) {
  if (M < 0 || N < 0 || K < 0 || g <= 0 || (K & 1)) return -1;
  int64_t kh = K / 2, nz = (N + 1) / 2;
  double* x = (double*)malloc(sizeof(double) * (size_t)M * (size_t)(K ? K : 1));
  if (!x) return -1;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) x[m * K + k] = ora_f16_to_f64(X[m * ldx + k]);
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    double* wrow = (double*)malloc(sizeof(double) * (size_t)(K ? K : 1));
    for (int64_t k = 0; k < K; ++k) {
      int64_t grp = k / g;
      int q = nib(w_u4 + n * kh, k);
      int z = nib(zeros + grp * nz, n);
      wrow[k] = (double)(q - z) * ora_f16_to_f64(scales[grp * N + n]);
    }
    for (int64_t m = 0; m < M; ++m) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += x[m * K + k] * wrow[k];
      out[m * N + n] = acc;
    }
    free(wrow);
  }
  free(x);
  return 0;
}

/* ------------------------------------------------------------------------
 * The three conversion modes of [p2] (ConversionMode, chosen by which of the
 * scale and zero types is void) over a 4-bit weight of either signedness:
 *   DirectConvert            (scales == NULL, zeros == NULL): w = v(q)
 *   ConvertAndScale          (zeros == NULL):                 w = v(q) s
 *   ConvertAndScaleWithZero  (both):                          w = (v(q) - v(z)) s
 * v() is the value of a nibble: itself for uint4, two's complement for int4
 * (nibbles 8..15 are -8..-1).  Scales are stored in `sdt` (fp16 or bf16),
 * [ceil(K/g)][N]; zeros have the weight's type, [ceil(K/g)][N/2] packed.
 * ------------------------------------------------------------------------ */
static int nib_value(int q, int is_signed) { return (is_signed && q >= 8) ? q - 16 : q; }

int ora_dequant_mixed(int32_t N, int32_t K, const uint8_t* w_u4, int32_t is_signed, const uint16_t* scales,
                      int32_t sdt, const uint8_t* zeros, int32_t g, double* wout) {
  if (N < 0 || K < 0 || g <= 0 || (K & 1) || (zeros && !scales)) return -1;
  if (scales && sdt != ORA_F16 && sdt != ORA_BF16) return -1;
  int64_t kh = K / 2, nz = (N + 1) / 2;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      int64_t grp = k / g;
      int v = nib_value(nib(w_u4 + n * kh, k), is_signed);
      if (zeros) v -= nib_value(nib(zeros + grp * nz, n), is_signed);
      double s = scales ? dec(scales[grp * N + n], sdt) : 1.0;
      wout[n * K + k] = (double)v * s;
    }
  return 0;
}

/* Y = X W^T with the weights of ora_dequant_mixed; X [M][ldx] and the scales
 * of type `xdt`, out [M][N] unrounded. */
int ora_mixed(int32_t M, int32_t N, int32_t K, const uint16_t* X, int64_t ldx, int32_t xdt, const uint8_t* w_u4,
              int32_t is_signed, const uint16_t* scales, const uint8_t* zeros, int32_t g, double* out) {
  if (M < 0 || N < 0 || K < 0 || g <= 0 || (K & 1) || (xdt != ORA_F16 && xdt != ORA_BF16)) return -1;
  double* w = (double*)malloc(sizeof(double) * (size_t)(N ? N : 1) * (size_t)(K ? K : 1));
  double* x = (double*)malloc(sizeof(double) * (size_t)(M ? M : 1) * (size_t)(K ? K : 1));
  if (!w || !x || ora_dequant_mixed(N, K, w_u4, is_signed, scales, xdt, zeros, g, w)) {
    free(w);
    free(x);
    return -1;
  }
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) x[m * K + k] = dec(X[m * ldx + k], xdt);
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t m = 0; m < M; ++m) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += x[m * K + k] * w[n * K + k];
      out[m * N + n] = acc;
    }
  free(w);
  free(x);
  return 0;
}

/* ------------------------------------------------------------------------
 * Convolution forward [p3], direct form (no im2col), cross-correlation:
 *   out[n][p][q][k] = alpha * sum_{r,s,c} x[n][p*sh - ph + r*dh][q*sw - pw + s*dw][c]
 *                                         * w[k][r][s][c]   + beta * C[n][p][q][k]
 * taps outside the image contribute 0.  x NHWC, w KRSC, C / out NPQK.
 *   P = floor((H + 2 ph - dh (R-1) - 1) / sh) + 1, likewise Q.
 * ------------------------------------------------------------------------ */
int ora_conv2d_fprop(int32_t N, int32_t H, int32_t W, int32_t C, int32_t K, int32_t R, int32_t S, int32_t ph,
                     int32_t pw, int32_t sh, int32_t sw, int32_t dh, int32_t dw, const uint16_t* x,
                     const uint16_t* w, const uint16_t* cin, int32_t dt, double alpha, double beta, double* out) {
  if (N < 0 || H <= 0 || W <= 0 || C <= 0 || K <= 0 || R <= 0 || S <= 0) return -1;
  if (ph < 0 || pw < 0 || sh <= 0 || sw <= 0 || dh <= 0 || dw <= 0) return -1;
  if (beta != 0.0 && !cin) return -1;
  int64_t P = (H + 2 * (int64_t)ph - (int64_t)dh * (R - 1) - 1) / sh + 1;
  int64_t Q = (W + 2 * (int64_t)pw - (int64_t)dw * (S - 1) - 1) / sw + 1;
  if (P <= 0 || Q <= 0) return -1;
  int64_t nx = (int64_t)N * H * W * C, nw = (int64_t)K * R * S * C;
  double* xd = (double*)malloc(sizeof(double) * (size_t)(nx ? nx : 1));
  double* wd = (double*)malloc(sizeof(double) * (size_t)nw);
  if (!xd || !wd) {
    free(xd);
    free(wd);
    return -1;
  }
  for (int64_t i = 0; i < nx; ++i) xd[i] = dec(x[i], dt);
  for (int64_t i = 0; i < nw; ++i) wd[i] = dec(w[i], dt);
#pragma omp parallel for schedule(static)
  for (int64_t np = 0; np < (int64_t)N * P; ++np) {
    int64_t n = np / P, p = np % P;
    for (int64_t q = 0; q < Q; ++q)
      for (int64_t k = 0; k < K; ++k) {
        double acc = 0.0;
        for (int64_t r = 0; r < R; ++r) {
          int64_t ih = p * sh - ph + r * dh;
          if (ih < 0 || ih >= H) continue;
          for (int64_t s = 0; s < S; ++s) {
            int64_t iw = q * sw - pw + s * dw;
            if (iw < 0 || iw >= W) continue;
            const double* xp = xd + ((n * H + ih) * W + iw) * C;
            const double* wp = wd + ((k * R + r) * S + s) * C;
            for (int64_t c = 0; c < C; ++c) acc += xp[c] * wp[c];
          }
        }
        int64_t o = ((n * P + p) * Q + q) * K + k;
        double v = alpha * acc;
        if (beta != 0.0) v += beta * dec(cin[o], dt);
        out[o] = v;
      }
  }
  free(xd);
  free(wd);
  return 0;
}

/* ------------------------------------------------------------------------
 * Convolution weight gradient [p3] (the wgrad operator): the adjoint of the
 * forward map in its filter argument.  Every product the forward pass forms,
 * x[n][ih][iw][c] * w[k][r][s][c] feeding y[n][p][q][k], sends
 * dy[n][p][q][k] * x[n][ih][iw][c] back to dw[k][r][s][c]:
 *   dw[k][r][s][c] = alpha * sum over (n, p, q) with ih = p*sh - ph + r*dh,
 *                    iw = q*sw - pw + s*dw inside the image
 *                    of dy[n][p][q][k] * x[n][ih][iw][c]   + beta * C[k][r][s][c]
 * x NHWC, dy NPQK, dw and C KRSC.
 * ------------------------------------------------------------------------ */
/* With channel groups (the grouped wgrad): output channel k belongs to group
 * g = k / (K/G) and sees only input channels g*(C/G) + c, c < C/G; dw and C
 * are [K][R][S][C/G].  G = 1 is the plain weight gradient. */
int ora_conv2d_wgrad_grouped(int32_t N, int32_t H, int32_t W, int32_t C, int32_t K, int32_t R, int32_t S, int32_t ph,
                             int32_t pw, int32_t sh, int32_t sw, int32_t dh, int32_t dw, int32_t G,
                             const uint16_t* x, const uint16_t* dy, const uint16_t* cin, int32_t dt, double alpha,
                             double beta, double* out);

int ora_conv2d_wgrad(int32_t N, int32_t H, int32_t W, int32_t C, int32_t K, int32_t R, int32_t S, int32_t ph,
                     int32_t pw, int32_t sh, int32_t sw, int32_t dh, int32_t dw, const uint16_t* x,
                     const uint16_t* dy, const uint16_t* cin, int32_t dt, double alpha, double beta, double* out) {
  return ora_conv2d_wgrad_grouped(N, H, W, C, K, R, S, ph, pw, sh, sw, dh, dw, 1, x, dy, cin, dt, alpha, beta, out);
}

int ora_conv2d_wgrad_grouped(int32_t N, int32_t H, int32_t W, int32_t C, int32_t K, int32_t R, int32_t S, int32_t ph,
                             int32_t pw, int32_t sh, int32_t sw, int32_t dh, int32_t dw, int32_t G,
                             const uint16_t* x, const uint16_t* dy, const uint16_t* cin, int32_t dt, double alpha,
                             double beta, double* out) {
  if (N < 0 || H <= 0 || W <= 0 || C <= 0 || K <= 0 || R <= 0 || S <= 0) return -1;
  if (G <= 0 || C % G || K % G) return -1;
  if (ph < 0 || pw < 0 || sh <= 0 || sw <= 0 || dh <= 0 || dw <= 0) return -1;
  if (beta != 0.0 && !cin) return -1;
  int64_t P = (H + 2 * (int64_t)ph - (int64_t)dh * (R - 1) - 1) / sh + 1;
  int64_t Q = (W + 2 * (int64_t)pw - (int64_t)dw * (S - 1) - 1) / sw + 1;
  if (P <= 0 || Q <= 0) return -1;
  int64_t nx = (int64_t)N * H * W * C, ny = (int64_t)N * P * Q * K;
  double* xd = (double*)malloc(sizeof(double) * (size_t)(nx ? nx : 1));
  double* gd = (double*)malloc(sizeof(double) * (size_t)(ny ? ny : 1));
  if (!xd || !gd) {
    free(xd);
    free(gd);
    return -1;
  }
  for (int64_t i = 0; i < nx; ++i) xd[i] = dec(x[i], dt);
  for (int64_t i = 0; i < ny; ++i) gd[i] = dec(dy[i], dt);
  const int64_t Cg = C / G, Kg = K / G;
  /* one filter tap (k, r, s) per iteration: a plain sum over images and output pixels */
#pragma omp parallel for schedule(static)
  for (int64_t krs = 0; krs < (int64_t)K * R * S; ++krs) {
    int64_t k = krs / (R * S), r = (krs / S) % R, s = krs % S;
    int64_t c0 = (k / Kg) * Cg; /* the group's first input channel */
    double* acc = out + krs * Cg;
    for (int64_t c = 0; c < Cg; ++c) acc[c] = 0.0;
    for (int64_t n = 0; n < N; ++n)
      for (int64_t p = 0; p < P; ++p) {
        int64_t ih = p * sh - ph + r * dh;
        if (ih < 0 || ih >= H) continue;
        for (int64_t q = 0; q < Q; ++q) {
          int64_t iw = q * sw - pw + s * dw;
          if (iw < 0 || iw >= W) continue;
          double g = gd[((n * P + p) * Q + q) * K + k];
          const double* xp = xd + ((n * H + ih) * W + iw) * C + c0;
          for (int64_t c = 0; c < Cg; ++c) acc[c] += g * xp[c];
        }
      }
    for (int64_t c = 0; c < Cg; ++c) {
      double v = alpha * acc[c];
      if (beta != 0.0) v += beta * dec(cin[krs * Cg + c], dt);
      acc[c] = v;
    }
  }
  free(xd);
  free(gd);
  return 0;
}

/* ------------------------------------------------------------------------
 * Convolution data gradient [p3] (the dgrad operator): the adjoint of the
 * forward map above in its first argument.  Every product the forward pass
 * forms, x[n][ih][iw][c] * w[k][r][s][c] feeding y[n][p][q][k], sends
 * dy[n][p][q][k] * w[k][r][s][c] back to dx[n][ih][iw][c]:
 *   dx[n][h][w][c] = alpha * sum over (p, q, k, r, s) with
 *                    p*sh - ph + r*dh = h and q*sw - pw + s*dw = w
 *                    of dy[n][p][q][k] * w[k][r][s][c]   + beta * C[n][h][w][c]
 * dy NPQK with P, Q as for the forward pass; dx, C NHWC.
 * ------------------------------------------------------------------------ */
int ora_conv2d_dgrad(int32_t N, int32_t H, int32_t W, int32_t C, int32_t K, int32_t R, int32_t S, int32_t ph,
                     int32_t pw, int32_t sh, int32_t sw, int32_t dh, int32_t dw, const uint16_t* dy,
                     const uint16_t* w, const uint16_t* cin, int32_t dt, double alpha, double beta, double* out) {
  if (N < 0 || H <= 0 || W <= 0 || C <= 0 || K <= 0 || R <= 0 || S <= 0) return -1;
  if (ph < 0 || pw < 0 || sh <= 0 || sw <= 0 || dh <= 0 || dw <= 0) return -1;
  if (beta != 0.0 && !cin) return -1;
  int64_t P = (H + 2 * (int64_t)ph - (int64_t)dh * (R - 1) - 1) / sh + 1;
  int64_t Q = (W + 2 * (int64_t)pw - (int64_t)dw * (S - 1) - 1) / sw + 1;
  if (P <= 0 || Q <= 0) return -1;
  int64_t nx = (int64_t)N * H * W * C, nw = (int64_t)K * R * S * C;
  double* wd = (double*)malloc(sizeof(double) * (size_t)nw);
  double* acc = (double*)calloc((size_t)(nx ? nx : 1), sizeof(double));
  if (!wd || !acc) {
    free(wd);
    free(acc);
    return -1;
  }
  for (int64_t i = 0; i < nw; ++i) wd[i] = dec(w[i], dt);
  /* one image per thread: the scatter of image n touches only dx of image n */
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t p = 0; p < P; ++p)
      for (int64_t q = 0; q < Q; ++q)
        for (int64_t k = 0; k < K; ++k) {
          double g = dec(dy[((n * P + p) * Q + q) * K + k], dt);
          if (g == 0.0) continue;
          for (int64_t r = 0; r < R; ++r) {
            int64_t ih = p * sh - ph + r * dh;
            if (ih < 0 || ih >= H) continue;
            for (int64_t s = 0; s < S; ++s) {
              int64_t iw = q * sw - pw + s * dw;
              if (iw < 0 || iw >= W) continue;
              double* xp = acc + ((n * H + ih) * W + iw) * C;
              const double* wp = wd + ((k * R + r) * S + s) * C;
              for (int64_t c = 0; c < C; ++c) xp[c] += g * wp[c];
            }
          }
        }
  for (int64_t i = 0; i < nx; ++i) {
    double v = alpha * acc[i];
    if (beta != 0.0) v += beta * dec(cin[i], dt);
    out[i] = v;
  }
  free(wd);
  free(acc);
  return 0;
}

/* ------------------------------------------------------------------------
 * Weight prepack [p2 design note: the narrow weight is reordered once so that
 * each lane's operand values for several consecutive matrix instructions sit
 * in one 128-bit word].  This library's permutation pi, over N x K uint4
 * values with N % 16 == 0 and K % 128 == 0:
 *
 *   block   b  = (n / 16) * (K / 128) + k / 128      (1024 bytes each)
 *   row     r  = n % 16,  kk = k % 128
 *   word    j  = kk / 32          (0..3)
 *   half    h  = (kk % 32) / 8    (0..3)
 *   element e  = kk % 8
 *   lane    L  = 16 h + r         (0..63)
 *   byte offset of the 32-bit little-endian word: 1024 b + 16 L + 4 j
 *   nibble slot inside the word: p = e / 2 + 4 (e % 2), bits [4p, 4p + 4)
 *
 * so a word holds 8 consecutive k of one row with the even elements in the
 * low nibble of each byte-quad and the odd elements in the high 16 bits.
 * ------------------------------------------------------------------------ */
static int pp_check(int32_t N, int32_t K) { return (N >= 0 && K >= 0 && N % 16 == 0 && K % 128 == 0) ? 0 : -1; }

int ora_prepack_w4(int32_t N, int32_t K, const uint8_t* w_u4, uint8_t* out) {
  if (pp_check(N, K)) return -1;
  int64_t kh = K / 2, kblocks = K / 128;
  memset(out, 0, (size_t)N * (size_t)kh);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      int q = nib(w_u4 + n * kh, k);
      int64_t b = (n / 16) * kblocks + k / 128;
      int64_t r = n % 16, kk = k % 128;
      int64_t j = kk / 32, h = (kk % 32) / 8, e = kk % 8;
      int64_t lane = 16 * h + r;
      int64_t word_byte = 1024 * b + 16 * lane + 4 * j;
      int p = (int)(e / 2 + 4 * (e % 2));
      out[word_byte + p / 2] |= (uint8_t)(q << (4 * (p % 2)));
    }
  return 0;
}

/* Inverse of pi, walking the prepacked bytes in storage order. */
int ora_unprepack_w4(int32_t N, int32_t K, const uint8_t* pp, uint8_t* w_u4) {
  if (pp_check(N, K)) return -1;
  int64_t kh = K / 2, kblocks = K / 128;
  int64_t total = (int64_t)N * kh;
  memset(w_u4, 0, (size_t)total);
  for (int64_t byte = 0; byte < total; ++byte)
    for (int hi = 0; hi < 2; ++hi) {
      int q = (pp[byte] >> (4 * hi)) & 15;
      int64_t b = byte / 1024, within = byte % 1024;
      int64_t lane = within / 16, j = (within % 16) / 4;
      int p = (int)(2 * (within % 4) + hi); /* nibble slot inside the word */
      int64_t e = (p < 4) ? 2 * p : 2 * (p - 4) + 1;
      int64_t h = lane / 16, r = lane % 16;
      int64_t n = (b / kblocks) * 16 + r;
      int64_t k = (b % kblocks) * 128 + 32 * j + 8 * h + e;
      w_u4[n * kh + k / 2] |= (uint8_t)(q << (4 * (k % 2)));
    }
  return 0;
}
