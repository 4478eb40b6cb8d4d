/*
 * CPU ORACLE for the NVFP4 block-scaled MoE grouped GEMM and its activation
 * quantiser.  TEST INFRASTRUCTURE ONLY: it is built and called by the tests,
 * by the smoke check and by the benchmark's CPU-baseline leg, and by nothing
 * on the product path.  It shares no code, header, table or helper with the
 * HIP library.
 *
 * What the pages fix (see the citations per function):
 *   - 4-bit values, two per byte ("Peering into the CUTLASS Kernel Cache",
 *     section "Knowledge Required"; "Peering into the CUTLASS SharedStorage",
 *     section "Input Knowledge", item 3);
 *   - one FP8 scale per 16 elements ("Peering into the CUTLASS SharedStorage",
 *     section "Input Knowledge", item 3; the "Vs16" schedule name in "Peering
 *     into the CUTLASS Kernel", section "Mistakes and Incorrect Assumptions");
 *   - grouped problem: every expert's weights meet only the tokens routed to
 *     that expert, so the group heights vary ("Peering into the CUTLASS Kernel
 *     Cache", section "Knowledge Required", the MoE grouped GEMM item);
 *   - FP32 accumulation, BF16 output staging ("Peering into the CUTLASS
 *     SharedStorage", section "Why This Message Was Written", the epilogue
 *     estimate).
 * Element format E2M1 and scale format E4M3 follow the OCP Microscaling (MX)
 * v1.0 and OCP 8-bit Floating Point (OFP8) v1.0 specifications.  The scale
 * recipe (amax / (6*448) tensor scale, RNE block scale, IEEE division) is a
 * reading the pages leave open; it is this library's definition.
 *
 * Style: plain C99, no intrinsics, fp64 / exact int64 where the arithmetic is
 * not fixed by the definition.  Compile with -ffp-contract=off so every float
 * expression is one IEEE single operation with round-to-nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define EXPORT __attribute__((visibility("default")))

/* Threads the OpenMP loops below run on (reported beside oracle timings). */
EXPORT int oracle_num_threads(void) { return omp_get_max_threads(); }

/* ---------------------------------------------------------------- E2M1 ---- */

/* E2M1 decode: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
 * Magnitudes of the 8 non-negative codes, written out from the format's
 * definition: e=0 is subnormal (m * 0.5), e>0 is 2^(e-1) * (1 + m/2). */
EXPORT double oracle_e2m1_decode(int code) {
  int e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return (code & 8) ? -mag : mag;
}

/* E2M1 encode with round-to-nearest-even and saturation to +-6.
 * The representable magnitudes are 0, .5, 1, 1.5, 2, 3, 4, 6; the midpoints
 * between neighbours are .25, .75, 1.25, 1.75, 2.5, 3.5, 5.  A value exactly
 * on a midpoint goes to the neighbour whose code is even (mantissa bit 0).
 * The sign bit is the sign bit of y (so -0 and small negatives give code 8). */
EXPORT int oracle_e2m1_encode(float y) {
  int sign = signbit(y) ? 8 : 0;
  float a = fabsf(y);
  int c;
  if (a <= 0.25f) c = 0;        /* tie .25 -> 0 (even) */
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;   /* ties .75 and 1.25 -> 2 (even) */
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;    /* ties 1.75 and 2.5 -> 4 (even) */
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;    /* ties 3.5 and 5 -> 6 (even) */
  else c = 7;                   /* saturate */
  return sign | c;
}

/* ---------------------------------------------------------------- E4M3 ---- */

/* E4M3 ("fn" variant of OFP8): sign bit 7, exponent bits 6..3 (bias 7),
 * mantissa bits 2..0; exponent 0 is subnormal; S.1111.111 is NaN; no Inf. */
EXPORT double oracle_e4m3_decode(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
  return s ? -mag : mag;
}

/* Bits of an E4M3 value known to be exactly representable (|v| <= 448). */
static int e4m3_bits_of_exact(double v) {
  int s = signbit(v) ? 0x80 : 0;
  double a = fabs(v);
  if (a == 0.0) return s;
  if (a < ldexp(1.0, -6)) return s | (int)(a / ldexp(1.0, -9)); /* subnormal: m * 2^-9 */
  int ex;
  double f = frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
  int e = ex - 1 + 7;       /* biased exponent of 2^(ex-1) */
  int m = (int)((f * 2.0 - 1.0) * 8.0);
  return s | (e << 3) | m;
}

/* E4M3 encode, round-to-nearest-even onto the grid of representable values,
 * saturating to +-448 (never NaN).  The grid spacing is 2^-9 below 2^-6 and
 * 2^(E-3) in the binade [2^E, 2^(E+1)).  Rounding is done on the real value
 * r / spacing (exact in double, since spacing is a power of two), with ties to
 * the even integer; a carry into the next binade stays on the grid. */
EXPORT int oracle_e4m3_encode(float r) {
  double a = fabs((double)r);
  int neg = signbit(r) ? 1 : 0;
  double v;
  if (a >= 448.0) {
    v = 448.0;
  } else {
    double spacing;
    if (a < ldexp(1.0, -6)) {
      spacing = ldexp(1.0, -9);
    } else {
      int ex;
      (void)frexp(a, &ex); /* a in [2^(ex-1), 2^ex) */
      spacing = ldexp(1.0, ex - 1 - 3);
    }
    double n = a / spacing; /* exact */
    double fl = floor(n), frac = n - fl;
    double rn;
    if (frac > 0.5) rn = fl + 1.0;
    else if (frac < 0.5) rn = fl;
    else rn = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    v = rn * spacing;
    if (v > 448.0) v = 448.0;
  }
  int bits = e4m3_bits_of_exact(v);
  if (neg) bits |= 0x80;
  return bits;
}

/* ---------------------------------------------------------------- BF16 ---- */

/* Round a double to the nearest bfloat16 (ties to even) and return its bits.
 * bfloat16 keeps 8 significant bits and the float exponent range; below 2^-126
 * the grid is the subnormal spacing 2^-133.  Overflow goes to +-Inf. */
EXPORT uint16_t oracle_bf16_bits_from_double(double x) {
  if (isnan(x)) return 0x7FC0;
  int neg = signbit(x) ? 1 : 0;
  double a = fabs(x);
  double spacing;
  if (a < ldexp(1.0, -126)) {
    spacing = ldexp(1.0, -133);
  } else {
    int ex;
    (void)frexp(a, &ex); /* a in [2^(ex-1), 2^ex) */
    spacing = ldexp(1.0, ex - 1 - 7);
  }
  double n = a / spacing;
  double fl = floor(n), frac = n - fl;
  double rn;
  if (frac > 0.5) rn = fl + 1.0;
  else if (frac < 0.5) rn = fl;
  else rn = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
  double v = rn * spacing;
  uint16_t bits;
  if (v >= ldexp(1.0, 128)) {
    bits = 0x7F80;
  } else {
    float f = (float)v; /* exact: v has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    bits = (uint16_t)(u >> 16);
  }
  if (neg) bits |= 0x8000;
  return bits;
}

/* --------------------------------------------------------------- Quantise - */

/* NVFP4 quantisation of a row-major FP32 matrix x[rows][ld_x] (first k columns
 * used; k a multiple of 16).
 *   1. Tensor scale g (FP32 decode multiplier).  dynamic != 0:
 *        g = amax > 0 ? fl(amax / 2688) : 1     (2688 = 6 * 448)
 *      and g is written to *g_inout; otherwise g = *g_inout as given.
 *   2. Per row and per block of 16 consecutive elements:
 *        amax_b = max |x|;  r = fl(amax_b / fl(6 * g));  sf = E4M3enc(r);
 *        s = fl(E4M3dec(sf) * g)
 *   3. Per element: y = (s == 0) ? +0 : fl(x / s);  code = E2M1enc(y)
 *   4. Pack: q[row][i] = code[2i] | code[2i+1] << 4.
 * fl() is one IEEE single operation, round-to-nearest-even.  The pages give
 * only the packing density (two per byte) and the 16-element FP8 block scale
 * ("Peering into the CUTLASS SharedStorage", section "Input Knowledge",
 * item 3); steps 1-3 are this library's reading of what they leave open.
 * Returns 0, or -1 on a bad argument. */
EXPORT int oracle_quantize(const float* x, int64_t rows, int64_t k, int64_t ld_x,
                           float* g_inout, int dynamic, uint8_t* q, uint8_t* sf) {
  if (k % 16 != 0 || rows < 0 || ld_x < k || !g_inout) return -1;
  float g;
  if (dynamic) {
    float amax = 0.0f;
    for (int64_t r = 0; r < rows; ++r)
      for (int64_t i = 0; i < k; ++i) {
        float a = fabsf(x[r * ld_x + i]);
        if (a > amax) amax = a;
      }
    g = (amax > 0.0f) ? amax / 2688.0f : 1.0f;
    *g_inout = g;
  } else {
    g = *g_inout;
  }
  const float six_g = 6.0f * g;
  const int64_t nb = k / 16;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const float* xb = x + r * ld_x + b * 16;
      float amax_b = 0.0f;
      for (int i = 0; i < 16; ++i) {
        float a = fabsf(xb[i]);
        if (a > amax_b) amax_b = a;
      }
      float rr = amax_b / six_g;
      int code_sf = oracle_e4m3_encode(rr);
      float s = (float)oracle_e4m3_decode(code_sf) * g;
      sf[r * nb + b] = (uint8_t)code_sf;
      int codes[16];
      for (int i = 0; i < 16; ++i) {
        float y = (s == 0.0f) ? 0.0f : xb[i] / s;
        codes[i] = oracle_e2m1_encode(y);
      }
      for (int i = 0; i < 8; ++i)
        q[r * (k / 2) + b * 8 + i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
    }
  }
  return 0;
}

/* ------------------------------------------------------------ Grouped GEMM - */

/* Twice the E2M1 value of each code: an integer in [-12, 12]. */
static int e2m1_times2(int code) {
  double v = oracle_e2m1_decode(code) * 2.0;
  return (int)v;
}
/* 512 times the E4M3 value of a finite code: an integer, |.| <= 229376. */
static int64_t e4m3_times512(int code) {
  double v = oracle_e4m3_decode(code) * 512.0;
  return (int64_t)v;
}

/* Find the expert that owns output row r: the e with off[e] <= r < off[e+1]. */
static int owner_expert(const int32_t* off, int32_t num_experts, int64_t r) {
  for (int32_t e = 0; e < num_experts; ++e)
    if (off[e] <= r && r < off[e + 1]) return e;
  return -1;
}

/* Grouped block-scaled GEMM, exact definition.
 * For expert e, output rows r in [off[e], off[e+1]), column j in [0, n):
 *   R[r][j] = a_scale * w_scale[e] * sum_k A(r, k) * W(e, j, k)
 * where A(r, k) = E2M1(a code) * E4M3(a block scale of block k/16) for
 * activation row src = a_row_index ? a_row_index[r] : r, and
 * W(e, j, k) = E2M1(w code) * E4M3(w block scale) of weight row j of expert e.
 * Layouts: a_q [a_rows][k/2], a_sf [a_rows][k/16], w_q [E][n][k/2],
 * w_sf [E][n][k/16]; element 2i in the low nibble of byte i.
 * The sum is formed exactly: per 16-block, sum_k (2a)(2w) is an integer, times
 * (512 sa)(512 sw), accumulated in int64; the value is acc * 2^-20.  It is then
 * scaled in double.  The grouped problem: one product per expert over the rows
 * routed to it ("Peering into the CUTLASS Kernel Cache", section "Knowledge
 * Required", the MoE grouped GEMM item), all experts in one call ("Peering into
 * the CUTLASS Kernel", section "Input Knowledge Required", item 4).
 * Only the listed output rows (rows_sel[0..nsel), or all m_total rows when
 * rows_sel is NULL) are computed; R_out and bf16_out are indexed
 * [sel_index][n].  Either output may be NULL.  Returns 0 or -1. */
EXPORT int oracle_grouped_gemm_exact(
    const uint8_t* a_q, const uint8_t* a_sf, float a_scale, int64_t a_rows,
    const int32_t* a_row_index, const uint8_t* w_q, const uint8_t* w_sf,
    const float* w_scale, const int32_t* offsets, int32_t num_experts,
    int64_t m_total, int64_t n, int64_t k, const int64_t* rows_sel, int64_t nsel,
    double* R_out, uint16_t* bf16_out) {
  if (k % 16 != 0 || n < 1 || num_experts < 1 || m_total < 0) return -1;
  if (!rows_sel) nsel = m_total;
  const int64_t nb = k / 16, kb = k / 2;
  /* Per-code integer values, filled from the decode functions above. */
  int j2[16];
  int64_t k512[256];
  for (int c = 0; c < 16; ++c) j2[c] = e2m1_times2(c);
  for (int c = 0; c < 256; ++c) k512[c] = ((c & 0x7F) == 0x7F) ? 0 : e4m3_times512(c);
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t t = 0; t < nsel; ++t) {
    int64_t r = rows_sel ? rows_sel[t] : t;
    int e = owner_expert(offsets, num_experts, r);
    if (e < 0) { bad |= 1; continue; }
    int64_t src = a_row_index ? a_row_index[r] : r;
    if (src < 0 || src >= a_rows) { bad |= 1; continue; }
    const uint8_t* aq = a_q + src * kb;
    const uint8_t* as = a_sf + src * nb;
    double alpha = (double)a_scale * (double)w_scale[e];
    for (int64_t j = 0; j < n; ++j) {
      const uint8_t* wq = w_q + ((int64_t)e * n + j) * kb;
      const uint8_t* ws = w_sf + ((int64_t)e * n + j) * nb;
      int64_t acc = 0;
      for (int64_t b = 0; b < nb; ++b) {
        int64_t p = 0;
        for (int i = 0; i < 16; ++i) {
          int64_t kk = b * 16 + i;
          int ca = (aq[kk / 2] >> (4 * (kk % 2))) & 15;
          int cw = (wq[kk / 2] >> (4 * (kk % 2))) & 15;
          p += (int64_t)j2[ca] * j2[cw];
        }
        acc += k512[as[b]] * k512[ws[b]] * p;
      }
      double R = ldexp((double)acc, -20) * alpha;
      if (R_out) R_out[t * n + j] = R;
      if (bf16_out) bf16_out[t * n + j] = oracle_bf16_bits_from_double(R);
    }
  }
  return bad ? -1 : 0;
}

/* Second, independent evaluation of the same definition: every element is
 * decoded to a double (E2M1 value times E4M3 value; exact), the products are
 * summed over k in natural order in double, and the sum is scaled.  Used to
 * cross-check the exact path; same arguments and layout. */
EXPORT int oracle_grouped_gemm_f64(
    const uint8_t* a_q, const uint8_t* a_sf, float a_scale, int64_t a_rows,
    const int32_t* a_row_index, const uint8_t* w_q, const uint8_t* w_sf,
    const float* w_scale, const int32_t* offsets, int32_t num_experts,
    int64_t m_total, int64_t n, int64_t k, const int64_t* rows_sel, int64_t nsel,
    double* R_out) {
  if (k % 16 != 0 || n < 1 || num_experts < 1 || m_total < 0 || !R_out) return -1;
  if (!rows_sel) nsel = m_total;
  const int64_t nb = k / 16, kb = k / 2;
  /* Per-code values, filled from the decode functions above. */
  double ev[16], sv[256];
  for (int c = 0; c < 16; ++c) ev[c] = oracle_e2m1_decode(c);
  for (int c = 0; c < 256; ++c) sv[c] = oracle_e4m3_decode(c);
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t t = 0; t < nsel; ++t) {
    int64_t r = rows_sel ? rows_sel[t] : t;
    int e = owner_expert(offsets, num_experts, r);
    if (e < 0) { bad |= 1; continue; }
    int64_t src = a_row_index ? a_row_index[r] : r;
    if (src < 0 || src >= a_rows) { bad |= 1; continue; }
    double* arow = (double*)malloc(sizeof(double) * k);
    for (int64_t kk = 0; kk < k; ++kk) {
      int ca = (a_q[src * kb + kk / 2] >> (4 * (kk % 2))) & 15;
      arow[kk] = ev[ca] * sv[a_sf[src * nb + kk / 16]];
    }
    for (int64_t j = 0; j < n; ++j) {
      const uint8_t* wq = w_q + ((int64_t)e * n + j) * kb;
      const uint8_t* ws = w_sf + ((int64_t)e * n + j) * nb;
      double sum = 0.0;
      for (int64_t kk = 0; kk < k; ++kk) {
        int cw = (wq[kk / 2] >> (4 * (kk % 2))) & 15;
        sum += arow[kk] * (ev[cw] * sv[ws[kk / 16]]);
      }
      R_out[t * n + j] = sum * (double)a_scale * (double)w_scale[e];
    }
    free(arow);
  }
  return bad ? -1 : 0;
}
