/*
 * CPU oracle for the all-gather matmul — TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code, header or constant with the HIP
 * library; both only receive the same raw input bits.
 *
 * What it computes (plain definition, written out):
 *   tpu-inference "all_gather_matmul.py", `all_gather_matmul` docstring: the
 *   result is all-gather(x, axis=0) @ y, where x is row-sharded over the
 *   devices and y is column-sharded, so one device produces
 *   C[m, n_local] = concat_r(A_r) @ B[:, n_local].
 *   Triton-distributed-Ascend "AllGather-GEMM", golden `torch_allgather_gemm`:
 *   all-gather the shards, concatenate along dim 0, then matmul.
 *   With rhs_transpose (tpu-inference `_do_mxu`, the dot_general that
 *   contracts dim 1 of both operands) B is stored [n_local, k] and
 *   C = A_gathered @ B^T.
 *
 * Arithmetic: every stored value is widened to double by decoding its bits
 * here; products of bf16/fp16/fp32 values are exact in double, and the sum
 * over t runs in increasing t in double.  The result is left in double (never
 * rounded to the storage dtype).
 *
 * Pins (checked by the CPU tests): brute force in exact rationals on tiny
 * shapes, numpy float64 matmul, per-shard row blocks, shard permutation,
 * B = identity, linearity in B, layout (transpose) consistency, and the
 * decoders against numpy/torch conversions.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_BF16 0
#define OR_FP16 1
#define OR_FP32 2

#define OR_OK 0
#define OR_EINVAL 1
#define OR_ENOMEM 3

/* bfloat16: the upper 16 bits of an IEEE binary32. */
static double or_decode_bf16(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double or_decode_fp16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int frac = h & 0x3FF;
  double v;
  if (e == 0) {
    v = ldexp((double)frac, -24); /* subnormal: frac * 2^(1-15-10) */
  } else if (e == 31) {
    v = frac ? NAN : INFINITY;
  } else {
    v = ldexp((double)(frac + 1024), e - 25); /* (1.frac) * 2^(e-15) */
  }
  return sign ? -v : v;
}

static double or_decode_fp32(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static size_t or_elem_bytes(int dtype) {
  return dtype == OR_FP32 ? 4 : 2;
}

/* Decode `count` stored values of `dtype` into doubles. */
int agmm_oracle_decode(int dtype, const void *src, int64_t count, double *dst) {
  if (!src || !dst || count < 0) return OR_EINVAL;
  if (dtype == OR_BF16) {
    const uint16_t *s = (const uint16_t *)src;
    for (int64_t i = 0; i < count; ++i) dst[i] = or_decode_bf16(s[i]);
  } else if (dtype == OR_FP16) {
    const uint16_t *s = (const uint16_t *)src;
    for (int64_t i = 0; i < count; ++i) dst[i] = or_decode_fp16(s[i]);
  } else if (dtype == OR_FP32) {
    const uint32_t *s = (const uint32_t *)src;
    for (int64_t i = 0; i < count; ++i) dst[i] = or_decode_fp32(s[i]);
  } else {
    return OR_EINVAL;
  }
  return OR_OK;
}

/*
 * The all-gathered operand: row r*m_s + i of the result is row i of shard r,
 * copied bit for bit (Ascend tutorial, golden: torch.cat of the gathered list
 * along dim 0; tpu-inference `_do_o_local_copy`: rows of shard d land at
 * offset m_per_device*d).
 */
int agmm_oracle_gather(int num_shards, int64_t m_s, int64_t k, int dtype,
                       const void *const *shards, void *gathered) {
  if (num_shards < 1 || m_s < 0 || k < 0 || !shards || !gathered) return OR_EINVAL;
  if (dtype < OR_BF16 || dtype > OR_FP32) return OR_EINVAL;
  size_t row_bytes = (size_t)k * or_elem_bytes(dtype);
  char *out = (char *)gathered;
  for (int r = 0; r < num_shards; ++r) {
    if (!shards[r]) return OR_EINVAL;
    const char *src = (const char *)shards[r];
    for (int64_t i = 0; i < m_s; ++i)
      memcpy(out + ((size_t)r * m_s + i) * row_bytes, src + (size_t)i * row_bytes, row_bytes);
  }
  return OR_OK;
}

/*
 * C rows of the all-gather matmul, in double.
 *
 *   rows   : global output row indices to compute (row = r*m_s + i means
 *            shard r, local row i), or NULL for all num_shards*m_s rows in
 *            order.
 *   nrows  : number of entries of `rows` (ignored when rows == NULL).
 *   C      : [nrows_out, n] doubles, row-major.
 *
 * For each requested row and each column j:
 *   C[row][j] = sum_{t=0}^{k-1} A_r[i][t] * Bv(t, j)     (t increasing)
 *   Bv(t, j)  = rhs_transpose ? B[j][t] : B[t][j]
 */
int agmm_oracle_f64(int num_shards, int64_t m_s, int64_t k, int64_t n, int dtype,
                    int rhs_transpose, const void *const *shards, const void *B,
                    const int64_t *rows, int64_t nrows, double *C) {
  if (num_shards < 1 || m_s < 0 || k < 0 || n < 0) return OR_EINVAL;
  if (dtype < OR_BF16 || dtype > OR_FP32) return OR_EINVAL;
  if (!shards || !B || !C) return OR_EINVAL;
  int64_t m = (int64_t)num_shards * m_s;
  int64_t nout = rows ? nrows : m;
  if (nout < 0) return OR_EINVAL;
  for (int64_t q = 0; rows && q < nout; ++q)
    if (rows[q] < 0 || rows[q] >= m) return OR_EINVAL;
  for (int r = 0; r < num_shards; ++r)
    if (!shards[r]) return OR_EINVAL;

  size_t eb = or_elem_bytes(dtype);
  /* B widened once: Bd[t*n + j] = Bv(t, j) (logical k x n). */
  double *Bd = (double *)malloc(sizeof(double) * (size_t)(k * n > 0 ? k * n : 1));
  if (!Bd) return OR_ENOMEM;
  {
    double *tmp = (double *)malloc(sizeof(double) * (size_t)(k * n > 0 ? k * n : 1));
    if (!tmp) { free(Bd); return OR_ENOMEM; }
    agmm_oracle_decode(dtype, B, k * n, tmp);
    for (int64_t t = 0; t < k; ++t)
      for (int64_t j = 0; j < n; ++j)
        Bd[t * n + j] = rhs_transpose ? tmp[j * k + t] : tmp[t * n + j];
    free(tmp);
  }

  int status = OR_OK;
#pragma omp parallel
  {
    double *arow = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
    if (!arow) {
#pragma omp atomic write
      status = OR_ENOMEM;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t q = 0; q < nout; ++q) {
        int64_t row = rows ? rows[q] : q;
        int64_t r = row / m_s;       /* owning shard */
        int64_t i = row - r * m_s;   /* row inside the shard */
        const char *src = (const char *)shards[r] + (size_t)i * (size_t)k * eb;
        agmm_oracle_decode(dtype, src, k, arow);
        double *out = C + (size_t)q * (size_t)n;
        for (int64_t j = 0; j < n; ++j) out[j] = 0.0;
        /* out[j] collects A_r[i][t] * Bv(t, j) for t = 0, 1, ..., k-1. */
        for (int64_t t = 0; t < k; ++t) {
          double a = arow[t];
          const double *brow = Bd + (size_t)t * (size_t)n;
          for (int64_t j = 0; j < n; ++j) out[j] += a * brow[j];
        }
      }
      free(arow);
    }
  }
  free(Bd);
  return status;
}

/* Number of OpenMP threads a parallel region uses here (for reporting). */
int agmm_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads the following oracle calls use (n >= 1); for timing the oracle on
 * one host core as well as on all of them.  Does not change what it computes:
 * every output element is one sequential sum in either case. */
void agmm_oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
