/*
 * oracle.c -- plain, slow, fp64 CPU oracle for paged attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the bench's CPU
 * baseline do.  It shares no code, header, table or helper with the HIP
 * library: every conversion, gather and sum below is written out here.
 *
 * What it computes (the plain definition; the GPU reaches it by online
 * softmax over fixed-size key splits, an exact rewrite up to rounding):
 *
 *   Vosti: Specifying, Implementing, and Verifying Deterministic LLM
 *   Inference, App. A.1: a query row i of an invocation with query length s
 *   and key length n sits at logical position p = n - s + i (also §5.3,
 *   "The causal contract"), and key row j of the logical cache is row
 *   j mod P of physical page pi(floor(j / P)).  App. A.2: the output row is
 *   softmax over keys 0..p of the scaled scores, applied to V.
 *
 * Physical page layout (a choice of this project; the pages are silent):
 *   K page: [num_pages][Hkv][d/8][P][8]   (8-element chunks, one slot per
 *           token: see k_slot for the order of the slots)
 *   V page: [num_pages][Hkv][d][P]        (dim-major, tokens contiguous)
 * The oracle implements its own gather for that layout.
 *
 * fp8: OCP e4m3 ("e4m3fn": bias 7, no infinities, S.1111.111 is NaN, max
 * finite 448).  Dequantised value = decoded code * per-KV-head scale; the
 * quantiser is code = RNE_e4m3(clamp(fp32(x / s), -448, 448)) -- static
 * per-head scales, as the Detent page requires for batch-invariant fp8
 * (its discussion of fp8 scales), and e4m3 products are exact while their
 * sums are order dependent (The Integer Alibi, §III (iii)).
 *
 * Every floating-point step is fp64 unless the definition fixes another
 * precision (bf16 inputs are exact in fp64; the fp8 quantiser's division is
 * defined in fp32).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- scalars */

/* bf16 bit pattern -> exact double: bf16 is the top half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP e4m3 (fn) code -> exact double.  Sign bit 7, exponent bits 6..3
 * (bias 7), mantissa bits 2..0; exponent 0 is subnormal (m/8 * 2^-6);
 * S.1111.111 is NaN; there is no infinity. */
double oracle_e4m3_to_f64(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 7;
  double v;
  if (e == 0xF && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* fp32 -> OCP e4m3 code, round to nearest even, saturating at +-448.
 * Written as a search over the 127 non-negative finite codes so that the
 * rounding rule is visible: pick the nearest representable magnitude, and on
 * a tie the one whose code is even (even mantissa). */
uint8_t oracle_f32_to_e4m3(float x) {
  double a = fabs((double)x);
  int neg = signbit(x) ? 1 : 0;
  if (a >= 448.0) return (uint8_t)((neg << 7) | 0x7E);
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double v = oracle_e4m3_to_f64((uint8_t)c);
    double err = fabs(v - a);
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)((neg << 7) | best);
}

/* The quantiser: stored code for value x under static scale s.  The division
 * is IEEE fp32 (computed in fp64 and rounded once to fp32, which equals the
 * correctly rounded fp32 quotient because 53 >= 2*24 + 2). */
uint8_t oracle_quantize_e4m3(float x, float s) {
  float q = (float)((double)x / (double)s);
  return oracle_f32_to_e4m3(q);
}

/* ------------------------------------------------------------- page layout */

/* K slot of token tok of a page: inside every whole group of 16 tokens, bits
 * 2 and 3 of tok are exchanged (a 16-token page stores tokens 0-3, 8-11, 4-7,
 * 12-15 in slots 0..15); tokens of a group that the page does not hold whole
 * keep their own index (so pages of fewer than 16 tokens are in token order). */
static int k_slot(int tok, int P) {
  if ((tok | 15) >= P) return tok;
  return (tok & ~12) | ((tok >> 1) & 4) | ((tok << 1) & 8);
}

static size_t k_index(int64_t page, int kvh, int tok, int dim, int Hkv, int d, int P) {
  return ((((size_t)page * Hkv + kvh) * (size_t)(d / 8) + (size_t)(dim / 8)) * P + k_slot(tok, P)) * 8 + (dim % 8);
}

static size_t v_index(int64_t page, int kvh, int tok, int dim, int Hkv, int d, int P) {
  return (((size_t)page * Hkv + kvh) * (size_t)d + dim) * P + tok;
}

/*
 * kv_append, the definition: new row t of K and V ([T][Hkv][d] bf16) goes to
 * slot slot_mapping[t] = page * P + offset of both caches.  Defining
 * passage: Defeating Nondeterminism in LLM Inference (summary page),
 * Overview -- the KV cache is updated before the attention kernel, which
 * then reads every key through the cache.  Slots < 0 are skipped (padding).
 * kv_fp8 != 0 stores e4m3 codes quantised with k_scale/v_scale [Hkv].
 */
int oracle_kv_append(const uint16_t* k_new, const uint16_t* v_new, const int64_t* slot_mapping,
                     int32_t T, int32_t Hkv, int32_t d, int32_t P, int32_t num_pages, int kv_fp8,
                     const float* k_scale, const float* v_scale, void* k_cache, void* v_cache) {
  if (d % 8 != 0) return 1;
  for (int32_t t = 0; t < T; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    int64_t page = slot / P;
    int tok = (int)(slot % P);
    if (page >= num_pages) return 2;
    for (int h = 0; h < Hkv; ++h) {
      for (int c = 0; c < d; ++c) {
        uint16_t kb = k_new[((size_t)t * Hkv + h) * d + c];
        uint16_t vb = v_new[((size_t)t * Hkv + h) * d + c];
        size_t ki = k_index(page, h, tok, c, Hkv, d, P);
        size_t vi = v_index(page, h, tok, c, Hkv, d, P);
        if (kv_fp8) {
          ((uint8_t*)k_cache)[ki] = oracle_quantize_e4m3((float)oracle_bf16_to_f64(kb), k_scale[h]);
          ((uint8_t*)v_cache)[vi] = oracle_quantize_e4m3((float)oracle_bf16_to_f64(vb), v_scale[h]);
        } else {
          ((uint16_t*)k_cache)[ki] = kb;
          ((uint16_t*)v_cache)[vi] = vb;
        }
      }
    }
  }
  return 0;
}

/* Gathered logical key / value element (exact in fp64). */
static double load_kv(const void* cache, int kv_fp8, size_t idx, double scale) {
  if (kv_fp8) return oracle_e4m3_to_f64(((const uint8_t*)cache)[idx]) * scale;
  return oracle_bf16_to_f64(((const uint16_t*)cache)[idx]);
}

typedef struct {
  const uint16_t* q;
  const int32_t* cu_q_lens;
  const int32_t* seq_lens;
  const void* k_cache;
  const void* v_cache;
  int kv_fp8;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  int32_t bt_stride, B, Hq, Hkv, d, P;
  double scale;
} attn_args;

/* Gathers the logical prefix 0..p of one (sequence, kv head) into dense fp64
 * arrays K[p+1][d], V[p+1][d]: K_X[j,:] = K_phys[pi(floor(j/P)), j mod P, :]
 * (Vosti, App. A.1). */
static void gather_prefix(const attn_args* a, int b, int kvh, int p, double* K, double* V) {
  const int32_t* bt = a->block_table + (size_t)b * a->bt_stride;
  double ks = a->kv_fp8 ? (double)a->k_scale[kvh] : 1.0;
  double vs = a->kv_fp8 ? (double)a->v_scale[kvh] : 1.0;
  for (int j = 0; j <= p; ++j) {
    int64_t page = bt[j / a->P];
    int tok = j % a->P;
    for (int c = 0; c < a->d; ++c) {
      K[(size_t)j * a->d + c] = load_kv(a->k_cache, a->kv_fp8, k_index(page, kvh, tok, c, a->Hkv, a->d, a->P), ks);
      V[(size_t)j * a->d + c] = load_kv(a->v_cache, a->kv_fp8, v_index(page, kvh, tok, c, a->Hkv, a->d, a->P), vs);
    }
  }
}

/* First key a query at position p sees: 0 for full causal attention; with a
 * sliding window of w > 0 keys, key j is visible iff p - w < j <= p (Vosti,
 * App. A.5: sliding-window attention adds the mask term j > p - w). */
static int first_key(int p, int window) {
  if (window <= 0) return 0;
  return p - window + 1 > 0 ? p - window + 1 : 0;
}

/* One output row by the plain definition: scores s_j = scale * <q, k_j> for
 * the visible keys j = lo..p, weights exp(s_j - max s),
 * O = sum_j w_j v_j / sum_j w_j. */
static void attend_plain(const double* qrow, const double* K, const double* V, int lo, int p, int d,
                         double scale, double* s, double* out) {
  double mx = -INFINITY;
  for (int j = lo; j <= p; ++j) {
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += qrow[c] * K[(size_t)j * d + c];
    s[j] = scale * acc;
    if (s[j] > mx) mx = s[j];
  }
  double den = 0.0;
  for (int c = 0; c < d; ++c) out[c] = 0.0;
  for (int j = lo; j <= p; ++j) {
    double w = exp(s[j] - mx);
    den += w;
    for (int c = 0; c < d; ++c) out[c] += w * V[(size_t)j * d + c];
  }
  for (int c = 0; c < d; ++c) out[c] /= den;
}

/* The same row computed as fixed-size split-KV (flash-decoding): keys are cut
 * at absolute multiples of S; each split gives (max m_s, sum l_s, weighted
 * sum o_s) and the splits are combined in ascending order by the LSE merge
 * M = max m_s, num = sum e^{m_s - M} o_s, den = sum e^{m_s - M} l_s
 * (Deterministic inference: results independent of the batch, the split-KV
 * decode example and the "Attention" rule of "Batch invariance: fixed splits
 * that don't change with load").  Used to cross-check the merge algebra.
 * Only splits holding visible keys (lo..p) take part. */
static void attend_split(const double* qrow, const double* K, const double* V, int lo, int p, int d,
                         double scale, int S, double* s, double* out, double* tmp) {
  int s0 = lo / S, nsplit = p / S + 1;
  double M = -INFINITY;
  for (int j = lo; j <= p; ++j) {
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += qrow[c] * K[(size_t)j * d + c];
    s[j] = scale * acc;
  }
  /* per-split maxima, then the global maximum over splits */
  for (int sp = s0; sp < nsplit; ++sp) {
    double m = -INFINITY;
    for (int j = sp * S > lo ? sp * S : lo; j <= p && j < (sp + 1) * S; ++j) m = s[j] > m ? s[j] : m;
    if (m > M) M = m;
  }
  double den = 0.0;
  for (int c = 0; c < d; ++c) out[c] = 0.0;
  for (int sp = s0; sp < nsplit; ++sp) {
    double m = -INFINITY;
    for (int j = sp * S > lo ? sp * S : lo; j <= p && j < (sp + 1) * S; ++j) m = s[j] > m ? s[j] : m;
    double l = 0.0;
    for (int c = 0; c < d; ++c) tmp[c] = 0.0;
    for (int j = sp * S > lo ? sp * S : lo; j <= p && j < (sp + 1) * S; ++j) {
      double w = exp(s[j] - m);
      l += w;
      for (int c = 0; c < d; ++c) tmp[c] += w * V[(size_t)j * d + c];
    }
    double f = exp(m - M);
    den += f * l;
    for (int c = 0; c < d; ++c) out[c] += f * tmp[c];
  }
  for (int c = 0; c < d; ++c) out[c] /= den;
}

static int run_attention(const attn_args* a, int split_tokens, int window, double* out, int nthreads) {
  if (a->Hkv <= 0 || a->Hq % a->Hkv != 0 || a->d % 8 != 0 || a->P <= 0) return 1;
  int g = a->Hq / a->Hkv;
  int max_n = 0;
  for (int b = 0; b < a->B; ++b) max_n = a->seq_lens[b] > max_n ? a->seq_lens[b] : max_n;
  for (int b = 0; b < a->B; ++b) {
    int s_len = a->cu_q_lens[b + 1] - a->cu_q_lens[b];
    if (s_len < 0 || s_len > a->seq_lens[b]) return 2;
  }
  int err = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  /* Parallel over (sequence, kv head); every task gathers its own prefix. */
#pragma omp parallel for schedule(dynamic, 1)
  for (int task = 0; task < a->B * a->Hkv; ++task) {
    int b = task / a->Hkv, kvh = task % a->Hkv;
    int n = a->seq_lens[b];
    int q0 = a->cu_q_lens[b], s_len = a->cu_q_lens[b + 1] - q0;
    if (s_len == 0) continue;
    int pmax = n - 1;
    double* K = (double*)malloc(sizeof(double) * (size_t)(pmax + 1) * a->d);
    double* V = (double*)malloc(sizeof(double) * (size_t)(pmax + 1) * a->d);
    double* sc = (double*)malloc(sizeof(double) * (size_t)(pmax + 1));
    double* qrow = (double*)malloc(sizeof(double) * a->d);
    double* tmp = (double*)malloc(sizeof(double) * a->d);
    if (!K || !V || !sc || !qrow || !tmp) {
#pragma omp atomic write
      err = 3;
    } else {
      gather_prefix(a, b, kvh, pmax, K, V);
      for (int i = 0; i < s_len; ++i) {
        int p = n - s_len + i; /* logical position of query row i */
        for (int hh = 0; hh < g; ++hh) {
          int h = kvh * g + hh; /* contiguous GQA groups: kv head = floor(h / g) */
          const uint16_t* qb = a->q + ((size_t)(q0 + i) * a->Hq + h) * a->d;
          for (int c = 0; c < a->d; ++c) qrow[c] = oracle_bf16_to_f64(qb[c]);
          double* o = out + ((size_t)(q0 + i) * a->Hq + h) * a->d;
          const int lo = first_key(p, window);
          if (split_tokens > 0)
            attend_split(qrow, K, V, lo, p, a->d, a->scale, split_tokens, sc, o, tmp);
          else
            attend_plain(qrow, K, V, lo, p, a->d, a->scale, sc, o);
        }
      }
    }
    free(K); free(V); free(sc); free(qrow); free(tmp);
  }
  (void)max_n;
  return err;
}

/*
 * Paged attention over ragged packed queries.  Decode is the case
 * cu_q_lens = 0,1,..,B.  q: [total_q][Hq][d] bf16; out: [total_q][Hq][d]
 * fp64.  window = 0 is full causal attention, window = w > 0 a sliding window
 * of w keys.  split_tokens = 0 gives the plain definition; > 0 computes the same
 * rows through fixed-size splits merged in ascending order.
 */
int oracle_paged_attention(const uint16_t* q, const int32_t* cu_q_lens, const int32_t* seq_lens,
                           const void* k_cache, const void* v_cache, int kv_fp8, const float* k_scale,
                           const float* v_scale, const int32_t* block_table, int32_t bt_stride, int32_t B,
                           int32_t Hq, int32_t Hkv, int32_t d, int32_t P, double scale, int32_t split_tokens,
                           int32_t window, double* out, int32_t nthreads) {
  attn_args a = {q, cu_q_lens, seq_lens, k_cache, v_cache, kv_fp8, k_scale, v_scale, block_table,
                 bt_stride, B, Hq, Hkv, d, P, scale};
  return run_attention(&a, split_tokens, window, out, nthreads);
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
