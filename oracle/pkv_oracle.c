/*
 * pkv_oracle.c - TEST INFRASTRUCTURE.  The CPU oracle for paged decode
 * attention (and the causal multi-query prefill over the same cache).  Only tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this file's library; the product path never does.
 *
 * What it computes is the plain definition the pages give, written out with
 * no blocking, fusion or reordering:
 *   - iThome ithelp article 10405755 on PagedAttention, section
 *     "PagedAttention 的核心想法": paging leaves the attention formula
 *     unchanged; the kernel only finds K,V through the block table.
 *   - Fanyi Pu, "Infra: PagedAttention", section "按 Block 分配": position t
 *     lives in logical block t/B at offset t%B, found through the table; the
 *     score of token i is s_i = q.k_i / sqrt(d) and the softmax normalises over
 *     every token the query can see.
 * So each sequence's K and V rows are first gathered into logical (position)
 * order, then ordinary dense softmax attention runs over them, in fp64:
 *     s_t = scale * sum_d q[d] k_t[d]          (d ascending)
 *     m   = max_t s_t
 *     Z   = sum_t exp(s_t - m)                 (t ascending)
 *     o   = sum_t exp(s_t - m) v_t / Z
 * A sequence with no tokens yields a zero row.  Query head h uses KV head
 * h / G with G = Hq / Hkv (consecutive query heads share a KV head).
 *
 * Cache layout read here (the library's documented layout, restated):
 *   k_cache bf16 [P, Hkv, B, D]; v_cache bf16 [P, Hkv, D, B].
 * Inputs are bf16 bit patterns; they widen exactly to double.
 *
 * Parallelism: one OpenMP work item per (sequence, KV head); nothing else.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double widen_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Dense softmax attention of one query row over T gathered rows (each row of
 * length D, consecutive rows `stride` doubles apart). */
static void dense_attention_row(const double* qrow, const double* K, const double* V,
                                int64_t T, int64_t stride, int32_t D, double scale,
                                double* s, double* out) {
  if (T == 0) {
    for (int32_t d = 0; d < D; d++) out[d] = 0.0;
    return;
  }
  double m = -INFINITY;
  for (int64_t t = 0; t < T; t++) {
    double acc = 0.0;
    for (int32_t d = 0; d < D; d++) acc += qrow[d] * K[t * stride + d];
    s[t] = scale * acc;
    if (s[t] > m) m = s[t];
  }
  double Z = 0.0;
  for (int64_t t = 0; t < T; t++) {
    s[t] = exp(s[t] - m);
    Z += s[t];
  }
  for (int32_t d = 0; d < D; d++) {
    double acc = 0.0;
    for (int64_t t = 0; t < T; t++) acc += s[t] * V[t * stride + d];
    out[d] = acc / Z;
  }
}

/* Paged decode attention.  out: fp64 [S, Hq, D].  Returns 0, or -1 on bad
 * sizes, -2 on allocation failure. */
int oracle_paged_decode(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                        const int32_t* block_tables, const int32_t* seq_lens, int32_t S,
                        int32_t Hq, int32_t Hkv, int32_t D, int32_t B, int32_t max_blocks,
                        double scale, double* out, int32_t num_threads) {
  if (S < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || B <= 0) return -1;
  const int32_t G = Hq / Hkv;
  const int64_t units = (int64_t)S * Hkv;
  int status = 0;
#ifdef _OPENMP
  if (num_threads <= 0) num_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads)
#endif
  for (int64_t u = 0; u < units; u++) {
    const int32_t b = (int32_t)(u / Hkv), h = (int32_t)(u % Hkv);
    const int64_t T = seq_lens[b];
    double* K = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * D);
    double* V = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * D);
    double* s = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
    if (!K || !V || !s || !qrow) {
      status = -2;
    } else {
      /* gather this sequence's rows for KV head h into position order */
      for (int64_t t = 0; t < T; t++) {
        const int64_t p = block_tables[(int64_t)b * max_blocks + t / B];
        const int64_t o = t % B;
        for (int32_t d = 0; d < D; d++) {
          K[t * D + d] = widen_bf16(k_cache[((p * Hkv + h) * B + o) * D + d]);
          V[t * D + d] = widen_bf16(v_cache[((p * Hkv + h) * D + d) * B + o]);
        }
      }
      for (int32_t g = 0; g < G; g++) {
        const int32_t hq = h * G + g;
        for (int32_t d = 0; d < D; d++)
          qrow[d] = widen_bf16(q[((int64_t)b * Hq + hq) * D + d]);
        dense_attention_row(qrow, K, V, T, D, D, scale, s,
                            out + ((int64_t)b * Hq + hq) * D);
      }
    }
    free(K);
    free(V);
    free(s);
    free(qrow);
  }
  return status;
}

/* The same attention from rows already in position order (no cache):
 * k_tok, v_tok bf16 [sum_b T_b, Hkv, D] sequence-major, cu_seqlens[S+1]. */
int oracle_dense_decode(const uint16_t* q, const uint16_t* k_tok, const uint16_t* v_tok,
                        const int64_t* cu_seqlens, int32_t S, int32_t Hq, int32_t Hkv,
                        int32_t D, double scale, double* out, int32_t num_threads) {
  if (S < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0) return -1;
  const int32_t G = Hq / Hkv;
  const int64_t units = (int64_t)S * Hkv;
  int status = 0;
#ifdef _OPENMP
  if (num_threads <= 0) num_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads)
#endif
  for (int64_t u = 0; u < units; u++) {
    const int32_t b = (int32_t)(u / Hkv), h = (int32_t)(u % Hkv);
    const int64_t t0 = cu_seqlens[b], T = cu_seqlens[b + 1] - cu_seqlens[b];
    double* K = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * D);
    double* V = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * D);
    double* s = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
    if (!K || !V || !s || !qrow) {
      status = -2;
    } else {
      for (int64_t t = 0; t < T; t++)
        for (int32_t d = 0; d < D; d++) {
          K[t * D + d] = widen_bf16(k_tok[((t0 + t) * Hkv + h) * D + d]);
          V[t * D + d] = widen_bf16(v_tok[((t0 + t) * Hkv + h) * D + d]);
        }
      for (int32_t g = 0; g < G; g++) {
        const int32_t hq = h * G + g;
        for (int32_t d = 0; d < D; d++)
          qrow[d] = widen_bf16(q[((int64_t)b * Hq + hq) * D + d]);
        dense_attention_row(qrow, K, V, T, D, D, scale, s,
                            out + ((int64_t)b * Hq + hq) * D);
      }
    }
    free(K);
    free(V);
    free(s);
    free(qrow);
  }
  return status;
}

/* Paged prefill (causal multi-query) attention.  The new tokens of sequence b
 * are the last q_len_b = cu_q[b+1] - cu_q[b] of its T_b cached tokens (their
 * K,V already in the cache); new token i sits at position p = T_b - q_len_b + i
 * and, as causal attention, sees the tokens at positions 0 .. p ([PU] "KV
 * Cache 为什么会浪费显存": in causal attention a token attends to the tokens
 * before it, whose K,V the cache keeps; [PU] "Continuous Batching": paging
 * and FlashAttention both keep the dense attention semantics).  So each new
 * token's row is the dense attention above over the first p + 1 gathered rows.
 * q bf16 [N, Hq, D] (N = cu_q[S]), out fp64 [N, Hq, D].  Returns 0, or -1 on
 * bad sizes (including q_len_b > T_b), -2 on allocation failure. */
int oracle_paged_prefill(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens,
                         const int64_t* cu_q, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                         int32_t B, int32_t max_blocks, double scale, double* out,
                         int32_t num_threads) {
  if (S < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || B <= 0) return -1;
  for (int32_t b = 0; b < S; b++)
    if (cu_q[b + 1] - cu_q[b] < 0 || cu_q[b + 1] - cu_q[b] > seq_lens[b]) return -1;
  const int32_t G = Hq / Hkv;
  const int64_t units = (int64_t)S * Hkv;
  int status = 0;
#ifdef _OPENMP
  if (num_threads <= 0) num_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads)
#endif
  for (int64_t u = 0; u < units; u++) {
    const int32_t b = (int32_t)(u / Hkv), h = (int32_t)(u % Hkv);
    const int64_t T = seq_lens[b];
    const int64_t nq = cu_q[b + 1] - cu_q[b];
    double* K = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * D);
    double* V = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * D);
    double* s = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
    if (!K || !V || !s || !qrow) {
      status = -2;
    } else {
      for (int64_t t = 0; t < T; t++) {
        const int64_t p = block_tables[(int64_t)b * max_blocks + t / B];
        const int64_t o = t % B;
        for (int32_t d = 0; d < D; d++) {
          K[t * D + d] = widen_bf16(k_cache[((p * Hkv + h) * B + o) * D + d]);
          V[t * D + d] = widen_bf16(v_cache[((p * Hkv + h) * D + d) * B + o]);
        }
      }
      for (int64_t i = 0; i < nq; i++) {
        const int64_t pos = T - nq + i; /* this token's position */
        const int64_t n = cu_q[b] + i;  /* its row in q and out */
        for (int32_t g = 0; g < G; g++) {
          const int32_t hq = h * G + g;
          for (int32_t d = 0; d < D; d++) qrow[d] = widen_bf16(q[(n * Hq + hq) * D + d]);
          dense_attention_row(qrow, K, V, pos + 1, D, D, scale, s, out + (n * Hq + hq) * D);
        }
      }
    }
    free(K);
    free(V);
    free(s);
    free(qrow);
  }
  return status;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
