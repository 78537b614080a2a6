/*
 * CPU oracle for paged decode attention and its companion copies.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * statement of what the GPU path computes.  It is loaded by the tests, by the
 * smoke check and by the benchmark's CPU-baseline leg; the product library
 * never links, loads or calls it, and it shares no code, header or table with
 * the GPU path.
 *
 * What it follows (pages as published; sections named, not line numbers):
 *  - "How PagedAttention Powers vLLM's KV Cache", section "PagedAttention:
 *    paging, borrowed from the operating system": a block holds the keys and
 *    values of a fixed number of tokens; each sequence's block table maps
 *    logical block j to the physical block that holds it.
 *  - same page, section "The attention kernel has to read scattered blocks":
 *    attention walks the block table and gathers keys and values block by
 *    block.
 *  - attention-lab "PagedAttention" page, widget "Measure memory use across
 *    requests" and reference entry "How it works": paging changes where the
 *    cache lives, not the attention equation.
 * Hence the oracle gathers each sequence's K/V through its table into a
 * contiguous copy and runs textbook softmax attention on it, in double.
 *
 * Pool layout (an interface fact the pages leave open; this build fixes it):
 *   K pool: [num_blocks][num_kv_heads][block_size][head_dim]   (token-major)
 *   V pool: [num_blocks][num_kv_heads][head_dim][block_size]   (dim-major)
 * Element types: 0 = IEEE fp32, 1 = bf16 (upper 16 bits of an fp32),
 * 2 = 8-bit float cache (OCP FP8 E4M3 codes with one bf16 scale per token,
 * kv head and side).  For type 2 the K buffer holds, per (block, kv head), a
 * region of B*d code bytes (token-major [B][d]) followed by the scales of
 * that (block, kv head): for each group of 4 token slots, their 4 K scales
 * then their 4 V scales, as bf16 (B*4 bytes); the V buffer holds, per
 * (block, kv head), only the B*d V codes (dim-major [d][B]).  A stored
 * element's value is decode(code) * scale of its token and side.  Queries,
 * outputs and the tokens handed to the slot write are bf16 for type 2.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_FP8 2

/*
 * OCP 8-bit floating point, E4M3 ("OCP 8-bit Floating Point Specification",
 * the E4M3 format): sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
 * exponent field 0 holds subnormals m * 2^-9; S.1111.111 is NaN; there are
 * no infinities, so the largest magnitude is S.1111.110 = 448.
 */
static double orc_e4m3_decode(uint8_t c) {
  const int sign = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
  double v;
  if (e == 0xF && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -v : v;
}

/*
 * Round an fp32 value to the nearest E4M3 code, ties to even; magnitudes at
 * or past 464 (the midpoint between 448 and the next power of two's first
 * step, which E4M3 lacks) saturate to 448.  Written on the fp32 bit pattern.
 */
static uint8_t orc_e4m3_encode(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  const uint8_t sign = (uint8_t)((u >> 24) & 0x80);
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7F;  /* NaN */
  if (a >= 0x43E80000u) return sign | 0x7E; /* |x| >= 464: saturate to 448 */
  if (a < 0x3C800000u) {                    /* |x| < 2^-6: subnormal or zero */
    float t;
    memcpy(&t, &a, sizeof t);
    return sign | (uint8_t)rintf(t * 512.0f); /* m = RNE(|x| / 2^-9); 8 is 2^-6 */
  }
  const uint32_t e = (a >> 23) - 120u;       /* biased E4M3 exponent, 1..15 */
  const uint32_t m3 = (a >> 20) & 7u;        /* top three mantissa bits */
  const uint32_t rest = a & 0xfffffu;        /* the 20 bits below them */
  uint32_t code = (e << 3) | m3;
  if (rest > 0x80000u || (rest == 0x80000u && (m3 & 1u))) code += 1; /* carries into e */
  return sign | (uint8_t)code;
}

/* Bytes of one (block, kv head) region of an 8-bit K buffer / V buffer. */
static size_t orc_fp8_k_region(int B, int d) { return (size_t)B * d + 4u * (size_t)B; }
static size_t orc_fp8_v_region(int B, int d) { return (size_t)B * d; }

/* Byte offset, inside a K region, of the bf16 scale of token slot r, side
 * v (0 = K, 1 = V): groups of 4 slots hold 4 K scales then 4 V scales. */
static size_t orc_fp8_scale_at(int B, int d, int r, int v) {
  return (size_t)B * d + 16u * (size_t)(r / 4) + 8u * (size_t)v + 2u * (size_t)(r % 4);
}

static double orc_fp8_scale(const void* k_pool, size_t k_region_base, int B, int d, int r,
                            int v) {
  uint16_t h;
  memcpy(&h, (const char*)k_pool + k_region_base + orc_fp8_scale_at(B, d, r, v), sizeof h);
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Widen one stored element to double, exactly. */
static double orc_load(int dtype, const void* base, size_t idx) {
  if (dtype == ORC_BF16) {
    uint16_t bits = ((const uint16_t*)base)[idx];
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[idx];
}

static size_t orc_elem_size(int dtype) { return dtype == ORC_BF16 ? 2u : 4u; }

static size_t k_index(int nkv, int B, int d, int32_t blk, int g, int r, int i) {
  return (((size_t)blk * nkv + g) * B + r) * (size_t)d + i;
}
static size_t v_index(int nkv, int B, int d, int32_t blk, int g, int r, int i) {
  return (((size_t)blk * nkv + g) * d + i) * (size_t)B + r;
}

/* Element i of token slot r of (block, kv head g), widened to double.  An
 * 8-bit V element needs the K buffer too: its scale is stored there. */
static double orc_k_elem(int dtype, int nkv, int B, int d, const void* k_pool, int32_t blk,
                         int g, int r, int i) {
  if (dtype == ORC_FP8) {
    const size_t base = ((size_t)blk * nkv + g) * orc_fp8_k_region(B, d);
    const uint8_t c = ((const uint8_t*)k_pool)[base + (size_t)r * d + i];
    return orc_e4m3_decode(c) * orc_fp8_scale(k_pool, base, B, d, r, 0);
  }
  return orc_load(dtype, k_pool, k_index(nkv, B, d, blk, g, r, i));
}
static double orc_v_elem(int dtype, int nkv, int B, int d, const void* k_pool,
                         const void* v_pool, int32_t blk, int g, int r, int i) {
  if (dtype == ORC_FP8) {
    const size_t vbase = ((size_t)blk * nkv + g) * orc_fp8_v_region(B, d);
    const size_t kbase = ((size_t)blk * nkv + g) * orc_fp8_k_region(B, d);
    const uint8_t c = ((const uint8_t*)v_pool)[vbase + (size_t)i * B + r];
    return orc_e4m3_decode(c) * orc_fp8_scale(k_pool, kbase, B, d, r, 1);
  }
  return orc_load(dtype, v_pool, v_index(nkv, B, d, blk, g, r, i));
}

/* Element type of queries and outputs for a pool type. */
static int orc_q_dtype(int dtype) { return dtype == ORC_FP8 ? ORC_BF16 : dtype; }

/*
 * Gather logical tokens [0, L) of (sequence s, kv head g) into contiguous
 * double arrays Kc[L][d], Vc[L][d]: token t lives in physical block
 * table[t / B], slot t % B.
 */
static void orc_gather(int dtype, int nkv, int B, int d, const void* k_pool,
                       const void* v_pool, const int32_t* table_row, int g,
                       int L, double* Kc, double* Vc) {
  for (int t = 0; t < L; ++t) {
    int32_t blk = table_row[t / B];
    int r = t % B;
    for (int i = 0; i < d; ++i) {
      Kc[(size_t)t * d + i] = orc_k_elem(dtype, nkv, B, d, k_pool, blk, g, r, i);
      Vc[(size_t)t * d + i] = orc_v_elem(dtype, nkv, B, d, k_pool, v_pool, blk, g, r, i);
    }
  }
}

/*
 * Textbook softmax attention of one query row over tokens [t0, t1) of a
 * contiguous K/V copy.  Writes the unnormalised partial state:
 *   m = max_t s_t,  l = sum_t exp(s_t - m),  o[i] = sum_t exp(s_t - m) V[t][i],
 * with s_t = scale * sum_i q[i] K[t][i].  Subtracting the maximum is exact
 * algebra and keeps exp() finite.
 */
static void orc_attend_range(const double* qd, const double* Kc, const double* Vc,
                             int d, int t0, int t1, double scale, double* scores,
                             double* m_out, double* l_out, double* o) {
  double m = -INFINITY;
  for (int t = t0; t < t1; ++t) {
    double acc = 0.0;
    for (int i = 0; i < d; ++i) acc += qd[i] * Kc[(size_t)t * d + i];
    scores[t - t0] = scale * acc;
    if (scores[t - t0] > m) m = scores[t - t0];
  }
  double l = 0.0;
  for (int i = 0; i < d; ++i) o[i] = 0.0;
  for (int t = t0; t < t1; ++t) {
    double e = exp(scores[t - t0] - m);
    l += e;
    for (int i = 0; i < d; ++i) o[i] += e * Vc[(size_t)t * d + i];
  }
  *m_out = m;
  *l_out = l;
}

/* Full attention over [0, L): out = o / l. */
static void orc_attend(const double* qd, const double* Kc, const double* Vc, int d,
                       int L, double scale, double* scores, double* out) {
  double m, l;
  orc_attend_range(qd, Kc, Vc, d, 0, L, scale, scores, &m, &l, out);
  for (int i = 0; i < d; ++i) out[i] /= l;
}

static int check_geometry(int dtype, int num_blocks, int B, int nkv, int d, int nq) {
  if (dtype != ORC_F32 && dtype != ORC_BF16 && dtype != ORC_FP8) return 1;
  if (num_blocks <= 0 || B <= 0 || nkv <= 0 || d <= 0 || nq <= 0) return 1;
  if (nq % nkv != 0) return 1;
  return 0;
}

static void set_threads(int num_threads) {
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#else
  (void)num_threads;
#endif
}

/*
 * Paged decode attention for a list of (sequence, query head) pairs.
 * out: [n_pairs][d] doubles.  Returns 0, or 1 on bad arguments, 2 on a
 * block id or length out of range, 3 on allocation failure.
 */
int oracle_decode_pairs(int dtype, int num_blocks, int block_size, int num_kv_heads,
                        int head_dim, const void* k_pool, const void* v_pool,
                        const void* q, int num_seqs, int num_q_heads,
                        const int32_t* block_tables, int max_blocks_per_seq,
                        const int32_t* context_lens, double scale,
                        const int32_t* pairs, int n_pairs, double* out,
                        int num_threads) {
  if (check_geometry(dtype, num_blocks, block_size, num_kv_heads, head_dim, num_q_heads))
    return 1;
  const int B = block_size, d = head_dim, nkv = num_kv_heads;
  const int G = num_q_heads / num_kv_heads;
  for (int p = 0; p < n_pairs; ++p) {
    int s = pairs[2 * p], h = pairs[2 * p + 1];
    if (s < 0 || s >= num_seqs || h < 0 || h >= num_q_heads) return 1;
    int L = context_lens[s];
    if (L <= 0 || L > max_blocks_per_seq * B) return 2;
    for (int j = 0; j < (L + B - 1) / B; ++j) {
      int32_t b = block_tables[(size_t)s * max_blocks_per_seq + j];
      if (b < 0 || b >= num_blocks) return 2;
    }
  }
  set_threads(num_threads);
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int p = 0; p < n_pairs; ++p) {
    int s = pairs[2 * p], h = pairs[2 * p + 1];
    int g = h / G;
    int L = context_lens[s];
    double* Kc = (double*)malloc(sizeof(double) * (size_t)L * d);
    double* Vc = (double*)malloc(sizeof(double) * (size_t)L * d);
    double* sc = (double*)malloc(sizeof(double) * (size_t)L);
    double* qd = (double*)malloc(sizeof(double) * (size_t)d);
    if (!Kc || !Vc || !sc || !qd) {
#pragma omp atomic write
      failed = 1;
    } else {
      for (int i = 0; i < d; ++i)
        qd[i] = orc_load(orc_q_dtype(dtype), q, ((size_t)s * num_q_heads + h) * d + i);
      orc_gather(dtype, nkv, B, d, k_pool, v_pool,
                 block_tables + (size_t)s * max_blocks_per_seq, g, L, Kc, Vc);
      orc_attend(qd, Kc, Vc, d, L, scale, sc, out + (size_t)p * d);
    }
    free(Kc);
    free(Vc);
    free(sc);
    free(qd);
  }
  return failed ? 3 : 0;
}

/* Paged decode attention for every (sequence, query head); out [S][Hq][d]. */
int oracle_decode(int dtype, int num_blocks, int block_size, int num_kv_heads,
                  int head_dim, const void* k_pool, const void* v_pool, const void* q,
                  int num_seqs, int num_q_heads, const int32_t* block_tables,
                  int max_blocks_per_seq, const int32_t* context_lens, double scale,
                  double* out, int num_threads) {
  if (num_seqs < 0 || num_q_heads <= 0) return 1;
  int n = num_seqs * num_q_heads;
  int32_t* pairs = (int32_t*)malloc(sizeof(int32_t) * 2 * (size_t)(n > 0 ? n : 1));
  if (!pairs) return 3;
  for (int s = 0; s < num_seqs; ++s)
    for (int h = 0; h < num_q_heads; ++h) {
      pairs[2 * (s * num_q_heads + h)] = s;
      pairs[2 * (s * num_q_heads + h) + 1] = h;
    }
  int rc = oracle_decode_pairs(dtype, num_blocks, block_size, num_kv_heads, head_dim,
                               k_pool, v_pool, q, num_seqs, num_q_heads, block_tables,
                               max_blocks_per_seq, context_lens, scale, pairs, n, out,
                               num_threads);
  free(pairs);
  return rc;
}

/*
 * The same attention on an unpaged, contiguous layout:
 *   k_dense, v_dense: [num_seqs][num_kv_heads][max_len][head_dim].
 * Paging must not change outputs, so for the same logical data this equals
 * oracle_decode bit for bit (same arithmetic, same order).
 */
int oracle_decode_dense(int dtype, int num_kv_heads, int head_dim, const void* k_dense,
                        const void* v_dense, int max_len, const void* q, int num_seqs,
                        int num_q_heads, const int32_t* context_lens, double scale,
                        double* out, int num_threads) {
  if (check_geometry(dtype, 1, 1, num_kv_heads, head_dim, num_q_heads)) return 1;
  if (dtype == ORC_FP8) return 1; /* dense copies are plain fp32 / bf16 arrays */
  const int d = head_dim, G = num_q_heads / num_kv_heads;
  for (int s = 0; s < num_seqs; ++s)
    if (context_lens[s] <= 0 || context_lens[s] > max_len) return 2;
  set_threads(num_threads);
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int p = 0; p < num_seqs * num_q_heads; ++p) {
    int s = p / num_q_heads, h = p % num_q_heads, g = h / G;
    int L = context_lens[s];
    double* Kc = (double*)malloc(sizeof(double) * (size_t)L * d);
    double* Vc = (double*)malloc(sizeof(double) * (size_t)L * d);
    double* sc = (double*)malloc(sizeof(double) * (size_t)L);
    double* qd = (double*)malloc(sizeof(double) * (size_t)d);
    if (!Kc || !Vc || !sc || !qd) {
#pragma omp atomic write
      failed = 1;
    } else {
      for (int i = 0; i < d; ++i)
        qd[i] = orc_load(orc_q_dtype(dtype), q, ((size_t)s * num_q_heads + h) * d + i);
      size_t base = ((size_t)s * num_kv_heads + g) * (size_t)max_len * d;
      for (int t = 0; t < L; ++t)
        for (int i = 0; i < d; ++i) {
          Kc[(size_t)t * d + i] = orc_load(dtype, k_dense, base + (size_t)t * d + i);
          Vc[(size_t)t * d + i] = orc_load(dtype, v_dense, base + (size_t)t * d + i);
        }
      orc_attend(qd, Kc, Vc, d, L, scale, sc, out + (size_t)p * d);
    }
    free(Kc);
    free(Vc);
    free(sc);
    free(qd);
  }
  return failed ? 3 : 0;
}

/*
 * Split-context form of the same attention, used only to check the split
 * identity: tokens [0, L) are cut into partitions [pP, min((p+1)P, L)); each
 * partition keeps (m_p, l_p, o_p) unnormalised and they are combined as
 *   M = max_p m_p,  out = sum_p e^{m_p - M} o_p / sum_p e^{m_p - M} l_p.
 */
int oracle_decode_split(int dtype, int num_blocks, int block_size, int num_kv_heads,
                        int head_dim, const void* k_pool, const void* v_pool,
                        const void* q, int num_seqs, int num_q_heads,
                        const int32_t* block_tables, int max_blocks_per_seq,
                        const int32_t* context_lens, double scale, int partition_tokens,
                        double* out, int num_threads) {
  if (check_geometry(dtype, num_blocks, block_size, num_kv_heads, head_dim, num_q_heads))
    return 1;
  if (partition_tokens <= 0) return 1;
  const int B = block_size, d = head_dim, nkv = num_kv_heads;
  const int G = num_q_heads / num_kv_heads, P = partition_tokens;
  for (int s = 0; s < num_seqs; ++s) {
    int L = context_lens[s];
    if (L <= 0 || L > max_blocks_per_seq * B) return 2;
    for (int j = 0; j < (L + B - 1) / B; ++j) {
      int32_t b = block_tables[(size_t)s * max_blocks_per_seq + j];
      if (b < 0 || b >= num_blocks) return 2;
    }
  }
  set_threads(num_threads);
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int p = 0; p < num_seqs * num_q_heads; ++p) {
    int s = p / num_q_heads, h = p % num_q_heads, g = h / G;
    int L = context_lens[s];
    int np = (L + P - 1) / P;
    double* Kc = (double*)malloc(sizeof(double) * (size_t)L * d);
    double* Vc = (double*)malloc(sizeof(double) * (size_t)L * d);
    double* sc = (double*)malloc(sizeof(double) * (size_t)P);
    double* qd = (double*)malloc(sizeof(double) * (size_t)d);
    double* mp = (double*)malloc(sizeof(double) * (size_t)np);
    double* lp = (double*)malloc(sizeof(double) * (size_t)np);
    double* op = (double*)malloc(sizeof(double) * (size_t)np * d);
    if (!Kc || !Vc || !sc || !qd || !mp || !lp || !op) {
#pragma omp atomic write
      failed = 1;
    } else {
      for (int i = 0; i < d; ++i)
        qd[i] = orc_load(orc_q_dtype(dtype), q, ((size_t)s * num_q_heads + h) * d + i);
      orc_gather(dtype, nkv, B, d, k_pool, v_pool,
                 block_tables + (size_t)s * max_blocks_per_seq, g, L, Kc, Vc);
      double M = -INFINITY;
      for (int k = 0; k < np; ++k) {
        int t0 = k * P, t1 = (k + 1) * P < L ? (k + 1) * P : L;
        orc_attend_range(qd, Kc, Vc, d, t0, t1, scale, sc, &mp[k], &lp[k],
                         op + (size_t)k * d);
        if (mp[k] > M) M = mp[k];
      }
      double den = 0.0;
      double* o = out + (size_t)p * d;
      for (int i = 0; i < d; ++i) o[i] = 0.0;
      for (int k = 0; k < np; ++k) {
        double w = exp(mp[k] - M);
        den += w * lp[k];
        for (int i = 0; i < d; ++i) o[i] += w * op[(size_t)k * d + i];
      }
      for (int i = 0; i < d; ++i) o[i] /= den;
    }
    free(Kc);
    free(Vc);
    free(sc);
    free(qd);
    free(mp);
    free(lp);
    free(op);
  }
  return failed ? 3 : 0;
}

/*
 * Gather one (sequence, kv head) into contiguous doubles Kc[L][d], Vc[L][d]:
 * exposes the block-table walk itself so it can be checked against the
 * pages' worked example of a table that keeps pages in order.
 */
int oracle_gather(int dtype, int num_blocks, int block_size, int num_kv_heads,
                  int head_dim, const void* k_pool, const void* v_pool,
                  const int32_t* table_row, int n_entries, int kv_head, int len,
                  double* Kc, double* Vc) {
  if (check_geometry(dtype, num_blocks, block_size, num_kv_heads, head_dim, num_kv_heads))
    return 1;
  if (kv_head < 0 || kv_head >= num_kv_heads || len < 0) return 1;
  if ((len + block_size - 1) / block_size > n_entries) return 2;
  for (int j = 0; j < (len + block_size - 1) / block_size; ++j)
    if (table_row[j] < 0 || table_row[j] >= num_blocks) return 2;
  orc_gather(dtype, num_kv_heads, block_size, head_dim, k_pool, v_pool, table_row,
             kv_head, len, Kc, Vc);
  return 0;
}

/* fp32 -> bf16 bits, round to nearest even (inputs here are finite). */
static uint16_t orc_bf16_rne(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/*
 * Slot write into an 8-bit pool: each token's bf16 K row and V row of each
 * kv head are quantised on their own.  amax = max |x| over the row; the
 * scale is amax / 448 computed in fp32 and rounded to bf16 (nearest even);
 * code_e = E4M3(x_e / scale) in fp32, rounded to nearest even (x_e / scale
 * may exceed 448 by the scale's rounding, at most 448 * (1 + 2^-8), which
 * still rounds to 448); a zero scale gives zero codes.  Codes go to the
 * token's slot, the scale to the token's K or V entry of the scale group in
 * the K buffer.  Same slot rules as below.
 */
static int orc_kv_write_fp8(int B, int d, int nkv, uint8_t* k_pool, uint8_t* v_pool,
                            const uint16_t* k_new, const uint16_t* v_new,
                            const int64_t* slot_mapping, int T) {
  for (int i = 0; i < T; ++i) {
    int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    int32_t blk = (int32_t)(slot / B);
    int r = (int)(slot % B);
    for (int g = 0; g < nkv; ++g) {
      const size_t kbase = ((size_t)blk * nkv + g) * orc_fp8_k_region(B, d);
      const size_t vbase = ((size_t)blk * nkv + g) * orc_fp8_v_region(B, d);
      for (int kv = 0; kv < 2; ++kv) {
        const uint16_t* src = (kv == 0 ? k_new : v_new) + ((size_t)i * nkv + g) * d;
        float amax = 0.0f;
        for (int e = 0; e < d; ++e) {
          float x = (float)orc_load(ORC_BF16, src, (size_t)e);
          if (fabsf(x) > amax) amax = fabsf(x);
        }
        const uint16_t sbits = orc_bf16_rne(amax / 448.0f);
        const float scale = (float)orc_load(ORC_BF16, &sbits, 0);
        for (int e = 0; e < d; ++e) {
          float x = (float)orc_load(ORC_BF16, src, (size_t)e);
          uint8_t c = scale > 0.0f ? orc_e4m3_encode(x / scale) : 0;
          if (kv == 0)
            k_pool[kbase + (size_t)r * d + e] = c;
          else
            v_pool[vbase + (size_t)e * B + r] = c;
        }
        memcpy(k_pool + kbase + orc_fp8_scale_at(B, d, r, kv), &sbits, sizeof sbits);
      }
    }
  }
  return 0;
}

/*
 * Slot write ("Dynamic Growth" on the glossary page: a sequence grows token
 * by token into the block its table names).  For every i with
 * slot_mapping[i] >= 0: block = slot / B, offset = slot % B, and for every kv
 * head g the token's K row and V row are copied bit for bit into that slot.
 * k_new, v_new: [T][num_kv_heads][head_dim].  Pools are host arrays updated
 * in place.  Returns 2 if a slot is past the pool.
 */
int oracle_kv_write(int dtype, int num_blocks, int block_size, int num_kv_heads,
                    int head_dim, void* k_pool, void* v_pool, const void* k_new,
                    const void* v_new, const int64_t* slot_mapping, int T) {
  if (check_geometry(dtype, num_blocks, block_size, num_kv_heads, head_dim, num_kv_heads))
    return 1;
  const int B = block_size, d = head_dim, nkv = num_kv_heads;
  const size_t es = orc_elem_size(dtype);
  for (int i = 0; i < T; ++i)
    if (slot_mapping[i] >= (int64_t)num_blocks * B) return 2;
  if (dtype == ORC_FP8) return orc_kv_write_fp8(B, d, nkv, (uint8_t*)k_pool, (uint8_t*)v_pool,
                                                (const uint16_t*)k_new, (const uint16_t*)v_new,
                                                slot_mapping, T);
  for (int i = 0; i < T; ++i) {
    int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    int32_t blk = (int32_t)(slot / B);
    int r = (int)(slot % B);
    for (int g = 0; g < nkv; ++g)
      for (int e = 0; e < d; ++e) {
        size_t src = ((size_t)i * nkv + g) * d + e;
        memcpy((char*)k_pool + k_index(nkv, B, d, blk, g, r, e) * es,
               (const char*)k_new + src * es, es);
        memcpy((char*)v_pool + v_index(nkv, B, d, blk, g, r, e) * es,
               (const char*)v_new + src * es, es);
      }
  }
  return 0;
}

/*
 * Copy-on-write block copy ("Shared blocks and copy-on-write": before a
 * request modifies a shared block it receives a private copy).  For each
 * (src, dst) pair, every kv head and every slot of block src is copied bit
 * for bit into block dst, for K and for V.  Pairs are applied in order.
 */
int oracle_block_copy(int dtype, int num_blocks, int block_size, int num_kv_heads,
                      int head_dim, void* k_pool, void* v_pool, const int32_t* pairs,
                      int num_pairs) {
  if (check_geometry(dtype, num_blocks, block_size, num_kv_heads, head_dim, num_kv_heads))
    return 1;
  const size_t plain = (size_t)num_kv_heads * block_size * head_dim * orc_elem_size(dtype);
  const size_t k_bytes =
      dtype == ORC_FP8 ? (size_t)num_kv_heads * orc_fp8_k_region(block_size, head_dim) : plain;
  const size_t v_bytes =
      dtype == ORC_FP8 ? (size_t)num_kv_heads * orc_fp8_v_region(block_size, head_dim) : plain;
  for (int p = 0; p < num_pairs; ++p) {
    int32_t src = pairs[2 * p], dst = pairs[2 * p + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return 2;
  }
  for (int p = 0; p < num_pairs; ++p) {
    int32_t src = pairs[2 * p], dst = pairs[2 * p + 1];
    memmove((char*)k_pool + (size_t)dst * k_bytes, (const char*)k_pool + (size_t)src * k_bytes,
            k_bytes);
    memmove((char*)v_pool + (size_t)dst * v_bytes, (const char*)v_pool + (size_t)src * v_bytes,
            v_bytes);
  }
  return 0;
}

/*
 * Multi-token attention with a causal mask (extend / chunked prefill):
 * sequence s brings n_s = q_start[s+1] - q_start[s] query rows whose tokens
 * are already counted in L = context_lens[s]; query j is at position
 * p = L - n_s + j and attends to tokens [0, p] exactly as decode attends to
 * [0, L) (gather through the table, textbook softmax in double).  The pages
 * describe the table-driven gather for any logical order (glossary entry,
 * "Complex Attention Patterns"); the causal range is the plainest reading of
 * appending tokens one by one ("Dynamic Growth").  q, out: [total][nq][d].
 */
int oracle_extend(int dtype, int num_blocks, int block_size, int num_kv_heads, int head_dim,
                  const void* k_pool, const void* v_pool, const void* q,
                  const int32_t* q_start, int num_seqs, int num_q_heads,
                  const int32_t* block_tables, int max_blocks_per_seq,
                  const int32_t* context_lens, double scale, double* out, int num_threads) {
  if (check_geometry(dtype, num_blocks, block_size, num_kv_heads, head_dim, num_q_heads))
    return 1;
  const int B = block_size, d = head_dim, nkv = num_kv_heads, G = num_q_heads / num_kv_heads;
  if (num_seqs < 0 || q_start[0] != 0) return 2;
  for (int s = 0; s < num_seqs; ++s) {
    const int n = q_start[s + 1] - q_start[s], L = context_lens[s];
    if (n < 0 || (n > 0 && (L < n || L > max_blocks_per_seq * B))) return 2;
    for (int j = 0; n > 0 && j < (L + B - 1) / B; ++j) {
      int32_t b = block_tables[(size_t)s * max_blocks_per_seq + j];
      if (b < 0 || b >= num_blocks) return 2;
    }
  }
  const int total = q_start[num_seqs];
  set_threads(num_threads);
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int p = 0; p < total * num_q_heads; ++p) {
    const int row = p / num_q_heads, h = p % num_q_heads, g = h / G;
    int s = 0;
    while (q_start[s + 1] <= row) ++s;
    const int n = q_start[s + 1] - q_start[s], L = context_lens[s];
    const int pos = L - n + (row - q_start[s]);
    const int len = pos + 1;
    double* Kc = (double*)malloc(sizeof(double) * (size_t)len * d);
    double* Vc = (double*)malloc(sizeof(double) * (size_t)len * d);
    double* sc = (double*)malloc(sizeof(double) * (size_t)len);
    double* qd = (double*)malloc(sizeof(double) * (size_t)d);
    if (!Kc || !Vc || !sc || !qd) {
#pragma omp atomic write
      failed = 1;
    } else {
      for (int i = 0; i < d; ++i)
        qd[i] = orc_load(orc_q_dtype(dtype), q, ((size_t)row * num_q_heads + h) * d + i);
      orc_gather(dtype, nkv, B, d, k_pool, v_pool,
                 block_tables + (size_t)s * max_blocks_per_seq, g, len, Kc, Vc);
      orc_attend(qd, Kc, Vc, d, len, scale, sc, out + (size_t)p * d);
    }
    free(Kc);
    free(Vc);
    free(sc);
    free(qd);
  }
  return failed ? 3 : 0;
}

/*
 * Block swap between a device pool and a host pool (preemption by swapping:
 * vLLM post, "Where it bites"; glossary entry, "Flexible Management").  For
 * each (src, dst) pair, the whole block src of the source pools (the device
 * pools for dir 0, the host pools for dir 1) is copied bit for bit to block
 * dst of the other pools, K and V.  Returns 2 on an index out of range.
 */
int oracle_block_swap(int dtype, int num_blocks, int block_size, int num_kv_heads, int head_dim,
                      void* k_pool, void* v_pool, void* host_k, void* host_v,
                      int num_host_blocks, const int32_t* pairs, int num_pairs, int dir) {
  if (check_geometry(dtype, num_blocks, block_size, num_kv_heads, head_dim, num_kv_heads))
    return 1;
  if (dir != 0 && dir != 1) return 1;
  const size_t plain = (size_t)num_kv_heads * block_size * head_dim * orc_elem_size(dtype);
  const size_t k_bytes =
      dtype == ORC_FP8 ? (size_t)num_kv_heads * orc_fp8_k_region(block_size, head_dim) : plain;
  const size_t v_bytes =
      dtype == ORC_FP8 ? (size_t)num_kv_heads * orc_fp8_v_region(block_size, head_dim) : plain;
  const int n_src = dir == 0 ? num_blocks : num_host_blocks;
  const int n_dst = dir == 0 ? num_host_blocks : num_blocks;
  for (int p = 0; p < num_pairs; ++p)
    if (pairs[2 * p] < 0 || pairs[2 * p] >= n_src || pairs[2 * p + 1] < 0 ||
        pairs[2 * p + 1] >= n_dst)
      return 2;
  char* sk = (char*)(dir == 0 ? k_pool : host_k);
  char* sv = (char*)(dir == 0 ? v_pool : host_v);
  char* dk = (char*)(dir == 0 ? host_k : k_pool);
  char* dv = (char*)(dir == 0 ? host_v : v_pool);
  for (int p = 0; p < num_pairs; ++p) {
    const size_t src = (size_t)pairs[2 * p], dst = (size_t)pairs[2 * p + 1];
    memcpy(dk + dst * k_bytes, sk + src * k_bytes, k_bytes);
    memcpy(dv + dst * v_bytes, sv + src * v_bytes, v_bytes);
  }
  return 0;
}

/* The E4M3 codec over arrays (for pinning it against the format). */
void oracle_e4m3_encode(const float* x, uint8_t* codes, int n) {
  for (int i = 0; i < n; ++i) codes[i] = orc_e4m3_encode(x[i]);
}
void oracle_e4m3_decode(const uint8_t* codes, double* x, int n) {
  for (int i = 0; i < n; ++i) x[i] = orc_e4m3_decode(codes[i]);
}

/* Threads OpenMP will use for the calls above (for reporting). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
