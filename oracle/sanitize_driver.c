/*
 * sanitize_driver.c - TEST INFRASTRUCTURE.  A stand-alone driver that runs
 * every entry point of pkv_oracle.c once on a tiny paged cache, for a build
 * with the address and undefined-behaviour sanitizers (tests build and run it
 * on the host only).  Every buffer is allocated at exactly its documented
 * size, so a read or write past any of them is reported.
 *
 * The case is the tiny paged layout of the iThome ithelp article 10405755 on
 * PagedAttention, section "手動畫一次 block table" (block size 4, tables
 * [7,1] and [3,0,4]) plus one more sequence and an empty one; the values are
 * arbitrary bf16 bit patterns from a fixed linear congruential sequence, and
 * every slot no sequence uses holds a NaN pattern.  Exit status 0 means every
 * call returned 0 and the paged and dense decodes agree bit for bit (they run
 * the same fp64 arithmetic on the same rows).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_paged_decode(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                        const int32_t* block_tables, const int32_t* seq_lens, int32_t S,
                        int32_t Hq, int32_t Hkv, int32_t D, int32_t B, int32_t max_blocks,
                        double scale, double* out, int32_t num_threads);
int oracle_dense_decode(const uint16_t* q, const uint16_t* k_tok, const uint16_t* v_tok,
                        const int64_t* cu_seqlens, int32_t S, int32_t Hq, int32_t Hkv,
                        int32_t D, double scale, double* out, int32_t num_threads);
int oracle_paged_prefill(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens,
                         const int64_t* cu_q, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                         int32_t B, int32_t max_blocks, double scale, double* out,
                         int32_t num_threads);
int oracle_max_threads(void);

enum { S = 4, HQ = 4, HKV = 2, D = 16, B = 4, P = 8, MB = 3 };
static const int32_t kLens[S] = {7, 9, 4, 0};
static const int32_t kTables[S][MB] = {{7, 1, 5}, {3, 0, 4}, {2, 5, 5}, {5, 5, 5}};
static const int32_t kQLens[S] = {3, 9, 1, 0}; /* prefill: new tokens per sequence */

static uint32_t lcg_state = 12345u;
static uint16_t next_bits(void) {
  lcg_state = lcg_state * 1664525u + 1013904223u;
  /* sign, a small exponent range around 1.0 and 7 mantissa bits */
  const uint32_t r = lcg_state >> 8;
  return (uint16_t)(((r & 1u) << 15) | ((124u + (r >> 1) % 6u) << 7) | ((r >> 4) & 0x7fu));
}

static void* exact(size_t n, size_t size) {
  void* p = malloc(n * size);
  if (p == NULL) {
    fprintf(stderr, "allocation failed\n");
    exit(2);
  }
  return p;
}

int main(void) {
  const uint16_t nan_bits = 0x7fc0;
  const size_t ncache = (size_t)P * HKV * B * D;
  uint16_t* kc = exact(ncache, sizeof(uint16_t));
  uint16_t* vc = exact(ncache, sizeof(uint16_t));
  for (size_t i = 0; i < ncache; i++) kc[i] = vc[i] = nan_bits;

  int64_t cu[S + 1];
  cu[0] = 0;
  for (int b = 0; b < S; b++) cu[b + 1] = cu[b] + kLens[b];
  const size_t ntok = (size_t)cu[S];
  uint16_t* kt = exact(ntok * HKV * D, sizeof(uint16_t));
  uint16_t* vt = exact(ntok * HKV * D, sizeof(uint16_t));
  /* token t of sequence b: row cu[b] + t of kt/vt, slot (table[t/B], t%B) of the cache */
  for (int b = 0; b < S; b++)
    for (int t = 0; t < kLens[b]; t++)
      for (int h = 0; h < HKV; h++)
        for (int d = 0; d < D; d++) {
          const uint16_t kb = next_bits(), vb = next_bits();
          const size_t row = ((size_t)(cu[b] + t) * HKV + h) * D + d;
          const size_t p = (size_t)kTables[b][t / B], o = (size_t)(t % B);
          kt[row] = kb;
          vt[row] = vb;
          kc[((p * HKV + h) * B + o) * D + d] = kb;
          vc[((p * HKV + h) * D + d) * B + o] = vb;
        }

  int32_t* bt = exact((size_t)S * MB, sizeof(int32_t));
  int32_t* lens = exact(S, sizeof(int32_t));
  for (int b = 0; b < S; b++) {
    lens[b] = kLens[b];
    for (int j = 0; j < MB; j++) bt[b * MB + j] = kTables[b][j];
  }
  uint16_t* q = exact((size_t)S * HQ * D, sizeof(uint16_t));
  for (size_t i = 0; i < (size_t)S * HQ * D; i++) q[i] = next_bits();
  double* out_paged = exact((size_t)S * HQ * D, sizeof(double));
  double* out_dense = exact((size_t)S * HQ * D, sizeof(double));
  const double scale = 0.25;

  int bad = 0;
  if (oracle_paged_decode(q, kc, vc, bt, lens, S, HQ, HKV, D, B, MB, scale, out_paged, 1) != 0)
    bad |= 1;
  if (oracle_dense_decode(q, kt, vt, cu, S, HQ, HKV, D, scale, out_dense, 1) != 0) bad |= 2;
  if (memcmp(out_paged, out_dense, sizeof(double) * S * HQ * D) != 0) bad |= 4;
  for (size_t i = 0; i < (size_t)S * HQ * D; i++)
    if (!isfinite(out_paged[i])) bad |= 8;
  for (size_t i = (size_t)3 * HQ * D; i < (size_t)S * HQ * D; i++)
    if (out_paged[i] != 0.0) bad |= 16; /* the empty sequence's row */

  int64_t cuq[S + 1];
  cuq[0] = 0;
  for (int b = 0; b < S; b++) cuq[b + 1] = cuq[b] + kQLens[b];
  const size_t nq = (size_t)cuq[S];
  uint16_t* qp = exact(nq * HQ * D, sizeof(uint16_t));
  for (size_t i = 0; i < nq * HQ * D; i++) qp[i] = next_bits();
  double* out_pf = exact(nq * HQ * D, sizeof(double));
  if (oracle_paged_prefill(qp, kc, vc, bt, lens, cuq, S, HQ, HKV, D, B, MB, scale, out_pf, 1) !=
      0)
    bad |= 32;
  for (size_t i = 0; i < nq * HQ * D; i++)
    if (!isfinite(out_pf[i])) bad |= 64;
  if (oracle_max_threads() < 1) bad |= 128;

  free(kc);
  free(vc);
  free(kt);
  free(vt);
  free(bt);
  free(lens);
  free(q);
  free(out_paged);
  free(out_dense);
  free(qp);
  free(out_pf);
  printf("sanitize_driver: status %d\n", bad);
  return bad;
}
