/*
 * oracle.c -- plain, slow, obviously-correct CPU model of block-scaled FP8
 * (OCP e4m3) W8A8 GEMM with 1x128 per-token UE8M0 activation scales packed four
 * to a 32-bit word, 128x128 weight block scales, and bf16 output.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code, header, table or constant generator with
 * the HIP library; every value here is derived from the definitions below.
 *
 * Arithmetic is done in double (fp64).  Every e4m3 value, every power-of-two
 * scale and every product of two e4m3 values is exact in double, and a sum of
 * 128 such products is exact too (their significands span < 53 bits), so the
 * per-block dot products below are the exact mathematical values.
 *
 * Sources (the pages this method is described on):
 *  - vLLM PR #29546 "Deepgemm fused layout kernel for activations", Purpose:
 *    per-token-group quant that packs the UE8M0 scales into a uint32 in the same
 *    pass; review comment on the "UE8M0-packed int32 scales".
 *  - vLLM PR #19885 "Optimize the little operations in the DeepGEMM + DeepEP low
 *    latency case", Summary: fused silu-mul-quant that skips padded tokens.
 *  - vLLM PR #19111 "Integrate batched/masked deepgemm kernel": masked grouped
 *    GEMM over [experts, max_tokens, K] with per-expert valid counts.
 *  - vLLM DeepGEMM FP8 block GEMM benchmark post, section 4.1 (scale = amax /
 *    fp8_max, rounded UP to a power of two when UE8M0 is used; 128x128 weight
 *    blocks, 1x128 activation groups), section 4.2 (per-K-block scale-then-
 *    accumulate), section 4.4 (calc_diff).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 * e4m3 = OCP E4M3FN (max 448, no infinities, NaN = S.1111.111); encoding is
 * round-to-nearest-even and saturates at +-448; the sign of zero is kept; the
 * UE8M0 byte is e + 127; the amax of a group is floored at 1e-10; the four
 * bytes of groups 4w..4w+3 go into word w little-endian; the activation-scale
 * tensor is stored M-major ([word][row]).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* e4m3 (OCP E4M3FN) decode: sign s, 4-bit exponent E (bias 7), 3-bit mantissa m.
 * E == 0: subnormal m * 2^-9.  E == 15 && m == 7: NaN.  Otherwise (1 + m/8) * 2^(E-7). */
double orc_e4m3_decode(uint8_t b) {
  int s = b >> 7, E = (b >> 3) & 15, m = b & 7;
  double v;
  if (E == 15 && m == 7) return NAN;
  if (E == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, E - 7);
  return s ? -v : v;
}

static double g_dec[256];
static int g_dec_ready = 0;
static void init_tables(void) {
  if (g_dec_ready) return;
  for (int b = 0; b < 256; ++b) g_dec[b] = orc_e4m3_decode((uint8_t)b);
  g_dec_ready = 1;
}

/* e4m3 encode, round to nearest with ties to even, saturating at 448.
 * The non-negative finite codes 0x00..0x7E decode to strictly increasing values,
 * so the nearest code is found by bisection over them; on an exact tie the code
 * with an even mantissa (LSB 0) wins.  The sign bit is copied from v (so -0 and
 * negatives that round to zero give 0x80).  NaN input is outside the contract. */
uint8_t orc_e4m3_encode(double v) {
  init_tables();
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs(v);
  if (isnan(v)) return (uint8_t)(0x7F | sign);
  if (a >= 448.0) return (uint8_t)(0x7E | sign);
  /* largest code lo in [0, 0x7E] with dec(lo) <= a */
  int lo = 0, hi = 0x7E;
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (g_dec[mid] <= a) lo = mid; else hi = mid - 1;
  }
  int code;
  if (g_dec[lo] == a) {
    code = lo;
  } else {
    double dlo = a - g_dec[lo], dhi = g_dec[lo + 1] - a;
    if (dlo < dhi) code = lo;
    else if (dhi < dlo) code = lo + 1;
    else code = (lo & 1) ? lo + 1 : lo;
  }
  return (uint8_t)(code | sign);
}

/* ------------------------------------------------------------------------ */
/* UE8M0 exponent of a group: the scale is amax / 448 rounded UP to a power of two,
 * i.e. the smallest integer e with 448 * 2^e >= amax', amax' = max(amax, 1e-10).
 * Found with exact double comparisons (no log2/ceil). */
int orc_ue8m0_exponent(double amax) {
  double a = amax > 1e-10 ? amax : 1e-10;
  int x;
  frexp(a, &x);     /* a = f * 2^x, f in [0.5, 1) */
  int e = x - 9;    /* 448 = 0.875 * 2^9, so 448 * 2^(x-9) is within a factor 2 of a */
  while (ldexp(448.0, e) < a) ++e;
  while (ldexp(448.0, e - 1) >= a) --e;
  return e;
}

static double bf16_to_double(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

/* Round a double to the nearest bf16 (ties to even), returning the bits. */
uint16_t orc_bf16_rne(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int x;
  frexp(a, &x);                      /* a in [2^(x-1), 2^x) */
  int q = x - 8;                     /* 8 significant bits: spacing 2^(x-8) */
  if (q < -133) q = -133;            /* bf16 subnormal spacing */
  double r = ldexp(nearbyint(ldexp(a, -q)), q);  /* default rounding mode: nearest-even */
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
  float f = (float)r;                /* exact: r has <= 8 significant bits */
  uint32_t bits;
  memcpy(&bits, &f, 4);
  return (uint16_t)(sign | ((bits >> 16) & 0x7FFF));
}

/* ------------------------------------------------------------------------ */
/* Per-token-group quant + UE8M0 pack.
 * x: bf16 [M][ldx];  q: e4m3 [M][ldq];  sf: uint32 [W][ld_sf], W = ceil(K/512).
 * For row r and group g (columns 128g..128g+127): e = ue8m0(amax), q = enc(x * 2^-e),
 * byte (e + 127) goes to bits 8*(g%4) of sf[(g/4)*ld_sf + r]; bytes of groups that
 * do not exist (K % 512 != 0) are zero.  Rows >= M of sf are not written. */
void orc_quant_group_pack(const uint16_t* x, int64_t ldx, int64_t M, int64_t K,
                          uint8_t* q, int64_t ldq, uint32_t* sf, int64_t ld_sf) {
  init_tables();
  int64_t G = K / 128, W = (G + 3) / 4;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < M; ++r) {
    for (int64_t w = 0; w < W; ++w) sf[w * ld_sf + r] = 0;
    for (int64_t g = 0; g < G; ++g) {
      double amax = 0.0;
      for (int64_t k = 128 * g; k < 128 * g + 128; ++k) {
        double v = fabs(bf16_to_double(x[r * ldx + k]));
        if (v > amax) amax = v;
      }
      int e = orc_ue8m0_exponent(amax);
      for (int64_t k = 128 * g; k < 128 * g + 128; ++k)
        q[r * ldq + k] = orc_e4m3_encode(ldexp(bf16_to_double(x[r * ldx + k]), -e));
      sf[(g / 4) * ld_sf + r] |= (uint32_t)(e + 127) << (8 * (g % 4));
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Fused SiLU-and-mul + per-token-group quant + pack over a masked batch.
 * x: bf16 [E][M_max][2H], gate = columns [0, H), up = columns [H, 2H).
 * Row r of expert e is processed only if r < c_e = clamp(masked_m[e], 0, M_max).
 * y = silu(g) * u = g / (1 + exp(-g)) * u, evaluated in double and then rounded to
 * fp32, the precision in which the GPU kernel holds y and takes the quantization
 * decision; then the 1x128 quant/pack above on y.
 * q: e4m3 [E][M_max][H];  sf: uint32 [E][W][M_max], W = ceil(H/512).
 * y_out (optional, may be NULL): the double y before the fp32 rounding, [E][M_max][H].
 * Rows r >= c_e of q, sf and y_out are not written. */
void orc_silu_mul_quant_group_pack(const uint16_t* x, const int32_t* masked_m, int64_t E,
                                   int64_t M_max, int64_t H, uint8_t* q, uint32_t* sf,
                                   double* y_out) {
  init_tables();
  int64_t G = H / 128, W = (G + 3) / 4;
  for (int64_t e = 0; e < E; ++e) {
    int64_t c = masked_m[e];
    if (c < 0) c = 0;
    if (c > M_max) c = M_max;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < c; ++r) {
      const uint16_t* row = x + (e * M_max + r) * 2 * H;
      uint8_t* qrow = q + (e * M_max + r) * H;
      for (int64_t w = 0; w < W; ++w) sf[(e * W + w) * M_max + r] = 0;
      for (int64_t g = 0; g < G; ++g) {
        float y32[128];
        double amax = 0.0;
        for (int64_t j = 0; j < 128; ++j) {
          int64_t k = 128 * g + j;
          double gv = bf16_to_double(row[k]);
          double uv = bf16_to_double(row[H + k]);
          double yd = gv / (1.0 + exp(-gv)) * uv;
          if (y_out) y_out[(e * M_max + r) * H + k] = yd;
          y32[j] = (float)yd;
          double a = fabs((double)y32[j]);
          if (a > amax) amax = a;
        }
        int ex = orc_ue8m0_exponent(amax);
        for (int64_t j = 0; j < 128; ++j)
          qrow[128 * g + j] = orc_e4m3_encode(ldexp((double)y32[j], -ex));
        sf[(e * W + g / 4) * M_max + r] |= (uint32_t)(ex + 127) << (8 * (g % 4));
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Weight block quant (offline step): per 128x128 block of w (bf16 [N][K], the last
 * row block may be partial), e = ue8m0(amax of the block), q = enc(w * 2^-e) and
 * sfb[nb][kb] = 2^e as fp32.  sfb is [ceil(N/128)][K/128] row-major. */
void orc_block_quant_128x128(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* sfb) {
  init_tables();
  int64_t NB = (N + 127) / 128, KB = K / 128;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t nb = 0; nb < NB; ++nb) {
    int64_t n1 = (nb + 1) * 128 < N ? (nb + 1) * 128 : N;
    for (int64_t kb = 0; kb < KB; ++kb) {
      double amax = 0.0;
      for (int64_t n = nb * 128; n < n1; ++n)
        for (int64_t k = kb * 128; k < kb * 128 + 128; ++k) {
          double v = fabs(bf16_to_double(w[n * K + k]));
          if (v > amax) amax = v;
        }
      int e = orc_ue8m0_exponent(amax);
      for (int64_t n = nb * 128; n < n1; ++n)
        for (int64_t k = kb * 128; k < kb * 128 + 128; ++k)
          q[n * K + k] = orc_e4m3_encode(ldexp(bf16_to_double(w[n * K + k]), -e));
      sfb[nb * KB + kb] = (float)ldexp(1.0, e);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Float-scale (non-UE8M0) format, benchmark post section 4.1: the scale of a group
 * or block is amax / fp8_max itself (rounding up to a power of two happens only for
 * UE8M0).  The pages' implementations compute in fp32, so these steps are fp32 IEEE
 * operations, each rounded to nearest even (C float arithmetic, no contraction):
 *   s = max(amax, 1e-10f) / 448,  y = x / s,  y clamped to [-448, 448],
 *   q = e4m3 RNE of y (exact decision: y is converted to double without rounding). */
static float float_scale(float amax) {
  float a = amax > 1e-10f ? amax : 1e-10f;
  return a / 448.0f;
}

static uint8_t float_quant(float x, float s) {
  float y = x / s;
  if (y > 448.0f) y = 448.0f;
  if (y < -448.0f) y = -448.0f;
  return orc_e4m3_encode((double)y);
}

/* 1x128 groups of bf16 x [M][ldx] -> q e4m3 [M][ldq], sf fp32 [K/128][ld_sf] (M-major). */
void orc_quant_group_float(const uint16_t* x, int64_t ldx, int64_t M, int64_t K, uint8_t* q, int64_t ldq,
                           float* sf, int64_t ld_sf) {
  init_tables();
  int64_t G = K / 128;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < M; ++r) {
    for (int64_t g = 0; g < G; ++g) {
      float amax = 0.0f;
      for (int64_t k = 128 * g; k < 128 * g + 128; ++k) {
        float v = fabsf((float)bf16_to_double(x[r * ldx + k]));
        if (v > amax) amax = v;
      }
      float s = float_scale(amax);
      for (int64_t k = 128 * g; k < 128 * g + 128; ++k)
        q[r * ldq + k] = float_quant((float)bf16_to_double(x[r * ldx + k]), s);
      sf[g * ld_sf + r] = s;
    }
  }
}

/* 128x128 blocks of bf16 w [N][K] -> q e4m3 [N][K], sfb fp32 [ceil(N/128)][K/128]. */
void orc_block_quant_128x128_float(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* sfb) {
  init_tables();
  int64_t NB = (N + 127) / 128, KB = K / 128;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t nb = 0; nb < NB; ++nb) {
    int64_t n1 = (nb + 1) * 128 < N ? (nb + 1) * 128 : N;
    for (int64_t kb = 0; kb < KB; ++kb) {
      float amax = 0.0f;
      for (int64_t n = nb * 128; n < n1; ++n)
        for (int64_t k = kb * 128; k < kb * 128 + 128; ++k) {
          float v = fabsf((float)bf16_to_double(w[n * K + k]));
          if (v > amax) amax = v;
        }
      float s = float_scale(amax);
      for (int64_t n = nb * 128; n < n1; ++n)
        for (int64_t k = kb * 128; k < kb * 128 + 128; ++k)
          q[n * K + k] = float_quant((float)bf16_to_double(w[n * K + k]), s);
      sfb[nb * KB + kb] = s;
    }
  }
}

/* Per-token group quant into the masked expert layout of routed tokens (the
 * quantization of FP8 dispatch: PR #19885, Summary item 1; PR #19111 review, the
 * TODO asking for a batched quant).  Pair p = t * topk + j goes to expert ids[p]
 * when 0 <= ids[p] < E; its slot is the number of earlier pairs (in p order) routed
 * to the same expert.  Invalid ids and slots >= M_max give slot -1 and write nothing.
 * Every routed token is quantized as orc_quant_group_pack quantizes a row and copied
 * to row `slot` of its expert.  q: e4m3 [E][M_max][K], sf: uint32 [E][W][M_max],
 * masked_m: int32 [E] = min(pairs routed to e, M_max), slot_of: int32 [T * topk]. */
void orc_quant_group_pack_to_experts(const uint16_t* x, int64_t ldx, int64_t T, int64_t K,
                                     const int32_t* ids, int64_t topk, int64_t E, int64_t M_max,
                                     uint8_t* q, uint32_t* sf, int32_t* masked_m, int32_t* slot_of) {
  int64_t W = (K / 128 + 3) / 4;
  int64_t* count = (int64_t*)calloc((size_t)(E > 0 ? E : 1), sizeof(int64_t));
  uint8_t* qrow = (uint8_t*)malloc((size_t)(K > 0 ? K : 1));
  uint32_t* sfrow = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(W > 0 ? W : 1));
  for (int64_t t = 0; t < T; ++t) {
    int quantized = 0;
    for (int64_t j = 0; j < topk; ++j) {
      int64_t pidx = t * topk + j;
      int64_t e = ids[pidx];
      if (e < 0 || e >= E) { slot_of[pidx] = -1; continue; }
      int64_t slot = count[e]++;
      if (slot >= M_max) { slot_of[pidx] = -1; continue; }
      slot_of[pidx] = (int32_t)slot;
      if (!quantized) {
        orc_quant_group_pack(x + t * ldx, ldx, 1, K, qrow, K, sfrow, 1);
        quantized = 1;
      }
      memcpy(q + (e * M_max + slot) * K, qrow, (size_t)K);
      for (int64_t w = 0; w < W; ++w) sf[(e * W + w) * M_max + slot] = sfrow[w];
    }
  }
  for (int64_t e = 0; e < E; ++e) masked_m[e] = (int32_t)(count[e] < M_max ? count[e] : M_max);
  free(count);
  free(qrow);
  free(sfrow);
}

/* ------------------------------------------------------------------------ */
/* Block-scaled GEMM, NT form: for each selected row m and column n,
 *   C[m][n] = sum over K-blocks kb of  2^(ea[m][kb]) * sfb[n/128][kb]
 *             * sum_{k in block kb} dec(qa[m][k]) * dec(qb[n][k])
 * where ea[m][kb] = byte kb%4 of word sfa[(kb/4)*ld_sfa + m], minus 127.
 * qa: e4m3 [M][lda], qb: e4m3 [N][ldb], sfb: fp32 [ceil(N/128)][K/128].
 * rows/cols select which outputs to compute (NULL = all M rows / all N columns);
 * out is double [nrows][ncols]. */
void orc_gemm_nt(const uint8_t* qa, int64_t lda, const uint32_t* sfa, int64_t ld_sfa,
                 const uint8_t* qb, int64_t ldb, const float* sfb,
                 int64_t M, int64_t N, int64_t K,
                 const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                 double* out) {
  init_tables();
  int64_t KB = K / 128;
  if (!rows) nrows = M;
  if (!cols) ncols = N;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t m = rows ? rows[i] : i;
    for (int64_t j = 0; j < ncols; ++j) {
      int64_t n = cols ? cols[j] : j;
      double acc = 0.0;
      for (int64_t kb = 0; kb < KB; ++kb) {
        double dot = 0.0;
        for (int64_t k = kb * 128; k < kb * 128 + 128; ++k)
          dot += g_dec[qa[m * lda + k]] * g_dec[qb[n * ldb + k]];
        int ea = (int)((sfa[(kb / 4) * ld_sfa + m] >> (8 * (kb % 4))) & 0xFF) - 127;
        acc += ldexp(1.0, ea) * (double)sfb[(n / 128) * KB + kb] * dot;
      }
      out[i * ncols + j] = acc;
    }
  }
}

/* Block-scaled GEMM with float scales (benchmark post section 4.2, the accumulate
 * rule read as acc += dot_kb * s_a[m] * s_b[n-block]): for each selected row m, column n
 *   C[m][n] = sum over K-blocks kb of sfa[kb][m] * sfb[n/128][kb]
 *             * sum_{k in block kb} dec(qa[m][k]) * dec(qb[n][k])
 * in double (the products of the two fp32 scales and the block sums are exact or
 * rounded once in double).  sfa: fp32 [K/128][ld_sfa]. */
void orc_gemm_nt_float_scales(const uint8_t* qa, int64_t lda, const float* sfa, int64_t ld_sfa,
                              const uint8_t* qb, int64_t ldb, const float* sfb,
                              int64_t M, int64_t N, int64_t K,
                              const int64_t* rows, int64_t nrows, const int64_t* cols, int64_t ncols,
                              double* out) {
  init_tables();
  int64_t KB = K / 128;
  if (!rows) nrows = M;
  if (!cols) ncols = N;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t m = rows ? rows[i] : i;
    for (int64_t j = 0; j < ncols; ++j) {
      int64_t n = cols ? cols[j] : j;
      double acc = 0.0;
      for (int64_t kb = 0; kb < KB; ++kb) {
        double dot = 0.0;
        for (int64_t k = kb * 128; k < kb * 128 + 128; ++k)
          dot += g_dec[qa[m * lda + k]] * g_dec[qb[n * ldb + k]];
        acc += (double)sfa[kb * ld_sfa + m] * (double)sfb[(n / 128) * KB + kb] * dot;
      }
      out[i * ncols + j] = acc;
    }
  }
}

/* Masked grouped GEMM: expert e multiplies its first c_e = clamp(masked_m[e], 0, M_max)
 * rows.  a: e4m3 [E][M_max][K], sfa: uint32 [E][W][M_max], b: e4m3 [E][N][K],
 * sfb: fp32 [E][ceil(N/128)][K/128], out: double [E][M_max][N].  rows (optional)
 * restricts the rows computed in every expert; rows >= c_e are skipped and their
 * outputs are not written. */
void orc_gemm_grouped_masked(const uint8_t* a, const uint32_t* sfa, const uint8_t* b,
                             const float* sfb, const int32_t* masked_m,
                             int64_t E, int64_t M_max, int64_t N, int64_t K,
                             const int64_t* rows, int64_t nrows, double* out) {
  int64_t W = (K / 128 + 3) / 4, NB = (N + 127) / 128, KB = K / 128;
  int64_t* sel = (int64_t*)malloc(sizeof(int64_t) * (size_t)(M_max > 0 ? M_max : 1));
  for (int64_t e = 0; e < E; ++e) {
    int64_t c = masked_m[e];
    if (c < 0) c = 0;
    if (c > M_max) c = M_max;
    int64_t ns = 0;
    if (rows) {
      for (int64_t i = 0; i < nrows; ++i)
        if (rows[i] >= 0 && rows[i] < c && ns < M_max) sel[ns++] = rows[i];
    } else {
      for (int64_t r = 0; r < c; ++r) sel[ns++] = r;
    }
    if (ns == 0) continue;
    double* tmp = (double*)malloc(sizeof(double) * (size_t)(ns * N));
    orc_gemm_nt(a + e * M_max * K, K, sfa + e * W * M_max, M_max,
                b + e * N * K, K, sfb + e * NB * KB, M_max, N, K,
                sel, ns, (const int64_t*)0, N, tmp);
    for (int64_t i = 0; i < ns; ++i)
      memcpy(out + (e * M_max + sel[i]) * N, tmp + i * N, sizeof(double) * (size_t)N);
    free(tmp);
  }
  free(sel);
}

/* Contiguous grouped GEMM (the high-throughput MoE layout; the PR #19111 page names
 * that path, the layout is read plainly): row m of A is multiplied with the weights
 * of group g = m_indices[m] when 0 <= g < E; rows with any other value are padding
 * and are not computed.  a: e4m3 [M][K], sfa: uint32 [W][ld_sfa], b: e4m3 [E][N][K],
 * sfb: fp32 [E][ceil(N/128)][K/128], out: double [M][N] (padding rows untouched).
 * rows (optional) restricts the rows computed. */
void orc_gemm_grouped_contiguous(const uint8_t* a, const uint32_t* sfa, int64_t ld_sfa, const uint8_t* b,
                                 const float* sfb, const int32_t* m_indices, int64_t E, int64_t M,
                                 int64_t N, int64_t K, const int64_t* rows, int64_t nrows, double* out) {
  int64_t NB = (N + 127) / 128, KB = K / 128;
  int64_t n_sel = rows ? nrows : M;
  int64_t* sel = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_sel > 0 ? n_sel : 1));
  for (int64_t g = 0; g < E; ++g) {
    int64_t ns = 0;
    for (int64_t i = 0; i < n_sel; ++i) {
      int64_t m = rows ? rows[i] : i;
      if (m >= 0 && m < M && m_indices[m] == g) sel[ns++] = m;
    }
    if (ns == 0) continue;
    double* tmp = (double*)malloc(sizeof(double) * (size_t)(ns * N));
    orc_gemm_nt(a, K, sfa, ld_sfa, b + g * N * K, K, sfb + g * NB * KB, M, N, K,
                sel, ns, (const int64_t*)0, N, tmp);
    for (int64_t i = 0; i < ns; ++i)
      memcpy(out + sel[i] * N, tmp + i * N, sizeof(double) * (size_t)N);
    free(tmp);
  }
  free(sel);
}

/* calc_diff of the benchmark post (section 4.4): 1 - 2*sum(x*y) / sum(x*x + y*y), in double. */
/*
 * Pre-shuffled weight layout.  Not a step of the method: a byte permutation of
 * e4m3 weights [rows][K] that the GEMM library declares for its decode kernel
 * (fp8_weight_preshuffle).  Byte i of 16-byte chunk l of load q of K-block kb of
 * 32-row group g sits at ((g*KB + kb)*4 + q)*1024 + l*16 + i and holds weight
 * row 32g + (l mod 32), column 128kb + 64*(q div 2) + 32*(l div 32) + 16*(q mod 2) + i.
 * Written here as the plain loop over that definition; rows % 32 == 0, K % 128 == 0.
 */
void orc_weight_preshuffle(const uint8_t* w, int64_t rows, int64_t K, uint8_t* out) {
  const int64_t KB = K / 128;
  for (int64_t g = 0; g < rows / 32; ++g)
    for (int64_t kb = 0; kb < KB; ++kb)
      for (int q = 0; q < 4; ++q)
        for (int l = 0; l < 64; ++l)
          for (int i = 0; i < 16; ++i) {
            const int64_t row = 32 * g + (l % 32);
            const int64_t col = 128 * kb + 64 * (q / 2) + 32 * (l / 32) + 16 * (q % 2) + i;
            out[(((g * KB + kb) * 4 + q) * 64 + l) * 16 + i] = w[row * K + col];
          }
}

double orc_calc_diff(const double* x, const double* y, int64_t n) {
  double num = 0.0, den = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    num += x[i] * y[i];
    den += x[i] * x[i] + y[i] * y[i];
  }
  return 1.0 - 2.0 * num / den;
}

/* Thread count for the OpenMP loops above (timing only: results do not depend on it). */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
