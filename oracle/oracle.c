/*
 * CPU oracle for the GEMM engine -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test-suite, the smoke check and the bench's CPU-baseline leg may
 * load this library. It shares no code with the GPU path (no headers, no
 * helpers, no tables); the only thing both sides see is the seeded input
 * arrays built by the `synth` package.
 *
 * What it computes is the operation stated on the page "InternLM Lmdeploy
 * Gemm Interface" (Description, and the Run signature / I/O Contract):
 *
 *     D = alpha * (A @ B) + beta * C
 *
 * written out as a plain triple loop, in fp64, summing serially over k:
 *
 *     acc(i,j)    = sum_k  a(i,k) * b(j,k)
 *     absdot(i,j) = sum_k |a(i,k) * b(j,k)|
 *     ref(i,j)    = alpha * acc(i,j) + (beta != 0 ? beta * c(i,j) : 0)
 *
 * B is the operand stored N x K (K contiguous), so (A@B)(i,j) = sum_k A[i,k]B[j,k]
 * (the same orientation as the stream-K kernel's transpose_B operand in the
 * TileLang tutorial "gemm_variants.py", function gemm_streamk).
 *
 * Decoded operand values (the "U, V quantization scale operands" of the
 * I/O Contract on the Gemm Interface page; the group stepping along K of the
 * page "InternLM Lmdeploy Gemm MainloopSm80V2", Description):
 *   bf16 / fp16 / fp32 : exact widening of the stored value
 *   int8               : the integer
 *   int4 (weight only) : b(j,k) = (q(j,k) - zero_point) * s(j, k / group_k),
 *                        s an fp16 scale, q the nibble k%8 of word k/8 of row j
 *                        (bits [4*(k%8), 4*(k%8)+4)); asymmetric: zero_point
 *                        = U(j, k / group_k), one byte per column and group
 *   fp8 OCP E4M3       : a(i,k) = dec(qa) * U(i / group_m, k / group_k),
 *                        b(j,k) = dec(qb) * V(e, j / group_n, k / group_k)
 * Grouped (MoE) problems: row r of A and D belongs to the expert e with
 * offsets[e] <= r < offsets[e+1], and uses B_e (and V_e).
 *
 * Epilogue (the fused GEMM + bias + activation and the fused output
 * quantisation of the DeepGEMM write-up, section 6), applied to ref in fp64:
 *   bias (flag 1):  ref += bias(j)
 *   ReLU (flag 2):  ref  = max(ref, 0)
 *   GELU (flag 4):  ref  = ref * Phi(ref) = 0.5 ref (1 + erf(ref / sqrt 2))
 *   quantisation (flag 8), or_quant_codes: t = ref * row_scale(i) + zero_point,
 *                   code = min(max(round_half_even(t), -128), 127)
 *
 * Split mode (self-check only): the K range is cut into `splits` contiguous
 * chunks of ceil(K/splits); each chunk is summed in fp64 on its own and the
 * chunk sums are then added in chunk order.
 *
 * Pins: every function here is checked by the CPU test-suite against
 * closed forms, brute force in exact rational arithmetic, library decoders
 * and invariants (identity / permutation B, linearity in alpha and beta,
 * beta-only pass-through, split invariance, grouped = per-expert dense).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_E4M3 = 3, OR_I8 = 4, OR_I32 = 5, OR_U4 = 6 };
enum { OR_Q_NONE = 0, OR_Q_INT4 = 1, OR_Q_BLOCK = 2 };

typedef struct {
  int64_t M, N, K;
  int32_t ta, tb, tc;  /* tc < 0: no C operand */
  int32_t qa, qb;      /* OR_Q_* */
  const void* A; int64_t lda;  /* elements */
  const void* B; int64_t ldb;  /* elements; uint32 words for int4 */
  const void* C; int64_t ldc;
  const void* U; int64_t ldu;  /* fp32 scales of A: [ceil(M/gm_a), ldu] */
  const void* V; int64_t ldv;  /* int4: fp16 [N, ldv]; fp8: fp32 [ceil(N/gn_b), ldv] */
  int32_t gm_a, gk_a, gn_b, gk_b;
  int32_t zero_point;
  double alpha, beta;
  int32_t E;                   /* > 0: grouped problem with E experts */
  const int32_t* offsets;      /* E + 1 row offsets into A / D */
  int64_t b_batch, v_batch;    /* per-expert strides of B (elements or words) and V */
  int32_t splits;              /* >= 1 */
  int32_t epi;                 /* epilogue flags: bias 1, relu 2, gelu 4, quantise 8 */
  int32_t bias_type;           /* OR_F32 / OR_BF16 / OR_F16 */
  const void* bias;            /* N values */
  const float* row_scale;      /* one per row of D */
  double out_zero_point;
} or_problem;

/* ---- scalar decoders ---------------------------------------------------- */

double or_dec_bf16(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double or_dec_f16(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

/* OCP 8-bit E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 fraction bits;
 * exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities. */
double or_dec_e4m3(uint8_t c) {
  int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}

static double dec_plain(int t, const void* p, int64_t idx) {
  switch (t) {
    case OR_F32: return (double)((const float*)p)[idx];
    case OR_F16: return or_dec_f16(((const uint16_t*)p)[idx]);
    case OR_BF16: return or_dec_bf16(((const uint16_t*)p)[idx]);
    case OR_E4M3: return or_dec_e4m3(((const uint8_t*)p)[idx]);
    case OR_I8: return (double)((const int8_t*)p)[idx];
    case OR_I32: return (double)((const int32_t*)p)[idx];
    default: return NAN;
  }
}

static double a_value(const or_problem* p, int64_t i, int64_t k) {
  double v = dec_plain(p->ta, p->A, i * p->lda + k);
  if (p->qa == OR_Q_BLOCK)
    v *= (double)((const float*)p->U)[(i / p->gm_a) * p->ldu + k / p->gk_a];
  return v;
}

static double b_value(const or_problem* p, int64_t e, int64_t j, int64_t k) {
  if (p->tb == OR_U4) {
    const uint32_t* w = (const uint32_t*)p->B + e * p->b_batch;
    uint32_t word = w[j * p->ldb + k / 8];
    int q = (int)((word >> (4 * (k % 8))) & 15u);
    const uint16_t* s = (const uint16_t*)p->V + e * p->v_batch;
    /* asymmetric: a zero point per column and group, bytes in U */
    int zp = p->U ? (int)((const int8_t*)p->U)[j * p->ldu + k / p->gk_b] : p->zero_point;
    return (double)(q - zp) * or_dec_f16(s[j * p->ldv + k / p->gk_b]);
  }
  int64_t esz = (p->tb == OR_F32) ? 4 : (p->tb == OR_F16 || p->tb == OR_BF16) ? 2 : 1;
  const char* base = (const char*)p->B + e * p->b_batch * esz;
  double v = dec_plain(p->tb, base, j * p->ldb + k);
  if (p->qb == OR_Q_BLOCK) {
    const float* s = (const float*)p->V + e * p->v_batch;
    v *= (double)s[(j / p->gn_b) * p->ldv + k / p->gk_b];
  }
  return v;
}

static int64_t expert_of_row(const or_problem* p, int64_t r) {
  if (p->E <= 0) return 0;
  for (int64_t e = 0; e < p->E; ++e)
    if (r >= p->offsets[e] && r < p->offsets[e + 1]) return e;
  return -1;
}

/* One output element, exactly as the definition in the header. */
static void one_output(const or_problem* p, int64_t i, int64_t j, double* ref, double* absdot) {
  int64_t e = expert_of_row(p, i);
  int64_t S = p->splits > 0 ? p->splits : 1;
  int64_t chunk = (p->K + S - 1) / S;
  double acc = 0.0, ad = 0.0;
  if (e >= 0) {
    for (int64_t c = 0; c < S; ++c) {
      int64_t k0 = c * chunk, k1 = k0 + chunk < p->K ? k0 + chunk : p->K;
      double part = 0.0;
      for (int64_t k = k0; k < k1; ++k) {
        double prod = a_value(p, i, k) * b_value(p, e, j, k);
        part += prod;
        ad += fabs(prod);
      }
      acc += part;
    }
  }
  double r = p->alpha * acc;
  if (p->beta != 0.0 && p->tc >= 0) r += p->beta * dec_plain(p->tc, p->C, i * p->ldc + j);
  if (p->epi & 1) r += dec_plain(p->bias_type, p->bias, j);
  if (p->epi & 2) r = r > 0.0 ? r : 0.0;
  if (p->epi & 4) r = 0.5 * r * (1.0 + erf(r / sqrt(2.0)));
  *ref = r;
  *absdot = ad;
}

/* Computes ref and absdot for the listed rows (rows == NULL: every row 0..M-1),
 * all N columns each; outputs are [nrows, N] row-major. Returns 0, or -1 on a
 * malformed problem. Rows are spread over OpenMP threads. */
int or_gemm(const or_problem* p, const int64_t* rows, int64_t nrows, double* ref, double* absdot) {
  if (!p || p->M < 0 || p->N < 0 || p->K < 0) return -1;
  if (!rows) nrows = p->M;
  int64_t total = nrows * p->N;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t t = 0; t < total; ++t) {
    int64_t r = t / p->N, j = t % p->N;
    int64_t i = rows ? rows[r] : r;
    one_output(p, i, j, &ref[t], &absdot[t]);
  }
  return 0;
}

/* Output quantisation of already computed outputs ref [nrows, N] (rows as in
 * or_gemm): pre = ref * row_scale(i) + zero_point, code = saturated
 * round-half-even of pre. */
int or_quant_codes(const or_problem* p, const int64_t* rows, int64_t nrows, const double* ref, double* pre,
                   int32_t* code) {
  if (!p || !p->row_scale) return -1;
  if (!rows) nrows = p->M;
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t i = rows ? rows[r] : r;
    double s = (double)p->row_scale[i];
    for (int64_t j = 0; j < p->N; ++j) {
      double t = ref[r * p->N + j] * s + p->out_zero_point;
      double q = nearbyint(t); /* the default rounding mode: to nearest, ties to even */
      if (q < -128.0) q = -128.0;
      if (q > 127.0) q = 127.0;
      pre[r * p->N + j] = t;
      code[r * p->N + j] = (int32_t)q;
    }
  }
  return 0;
}

int or_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the number of OpenMP threads of later calls made from the calling
 * thread (n >= 1); used to time the oracle single-threaded. */
void or_set_num_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
