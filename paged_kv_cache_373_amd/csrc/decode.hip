// decode.hip - paged decode attention kernels for gfx950 (CDNA4).
//
// Sources (by title and section):
//   [ITH] iThome ithelp article 10405755 on PagedAttention,
//         section "PagedAttention 的核心想法": the formula is unchanged; the
//         kernel looks the block table up and reads K,V in the physical blocks.
//   [PU]  Fanyi Pu, "Infra: PagedAttention", section "按 Block 分配":
//         s_i = q.k_i / sqrt(d); the softmax spans every visible token; segment
//         results merge by o = (Z1 o1 + Z2 o2) / (Z1 + Z2) once every segment's
//         statistics are rescaled to a common maximum; segments need not match
//         physical blocks; lookup, KV read and compute belong in one kernel,
//         neighbouring threads should read neighbouring data and the merge
//         should synchronise little.
//
// Kernel families
//   decode_mfma     one workgroup per (partition, KV head, sequence); its NW
//                   wavefronts stride over 32-token chunks of the partition.
//                   QK^T and P.V run on v_mfma_f32_16x16x32_bf16; the online
//                   softmax runs on the vector ALU; waves merge through LDS.
//   decode_generic  one wavefront per (partition, q head, sequence), scalar
//                   fp32 online softmax; any head_dim <= 256, any block size.
//   merge_states    one wavefront per (sequence, q head): combines partition
//                   results (o_r, ln Z_r) into the output.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// A running maximum is only raised when a chunk's maximum exceeds it by more
// than this many powers of two.  Until then probabilities are formed against
// the stale maximum and stay <= 2^8, which fp32 sums hold exactly as well as
// values <= 1; the final division by the same-based sum makes the result
// identical in exact arithmetic.  Rescaling the accumulators (a cross-lane
// exchange) therefore happens a handful of times per partition, not per chunk.
constexpr float kRescaleThreshold = 8.0f;

// 32-token chunks each wavefront of the matrix-core kernel keeps in flight.
#ifndef PKV_PIPELINE_DEPTH
#define PKV_PIPELINE_DEPTH 2
#endif
constexpr int kDepth = PKV_PIPELINE_DEPTH;

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  // v_cvt_pk_bf16_f32 rounds to nearest even
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Device-coherent accesses for data that workgroups hand to each other inside
// one launch (split-KV partials): atomic at agent scope, so each access is
// coherent across the chip's L2 caches by itself and no cache-wide write-back
// or invalidation is needed.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_out(void* out, size_t idx, float v, int out_f32) {
  if (out_f32)
    static_cast<float*>(out)[idx] = v;
  else
    static_cast<uint16_t*>(out)[idx] = float_to_bf16_bits(v);
}

// Finishes one (sequence, q head) row of a partition: either the final output
// (single partition) or the partition's (o_r, ln Z_r).  `m2` is the maximum in
// base-2 units, `den` the sum of 2^(x - m2).
__device__ __forceinline__ void write_partition_result(const DecodeParams& prm, int b, int hq,
                                                       int p, int nparts, int d, float o,
                                                       float m2, float den, bool empty) {
  const int D = prm.head_dim;
  if (nparts <= 1) {
    store_out(prm.out, (static_cast<size_t>(b) * prm.num_q_heads + hq) * D + d,
              empty ? 0.0f : o, prm.out_f32);
  } else {
    const size_t row = static_cast<size_t>(b) * prm.num_q_heads + hq;
    prm.part_out[(row * prm.num_partitions + p) * D + d] = o;
    if (d == 0) prm.part_lse[row * prm.num_partitions + p] = (m2 + __log2f(den)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Matrix-core kernel.
//
// One workgroup per (partition, KV head, sequence); its NW wavefronts take the
// partition's 32-token chunks round robin (wave w: chunks w, w + NW, ...).
//
// Lane roles inside a wavefront (lane = 16 c + r, c in 0..3, r in 0..15):
//   QK^T   S^T[t][g] = sum_d K[t][d] Q[g][d] as two 16x16x32 MFMAs per 16-token
//          half u of a 32-token chunk and per 32-wide slice of d.
//          A operand (K): lane (c, r) holds 8 dims [32 hs + 8 c, +8) of token
//          tok(u, r) = 8 (r / 4) + 4 u + r % 4 (one 16-byte load).
//          B operand (Q): lane (c, r) holds the same 8 dims of query head g = r
//          (zero for r >= G).
//          Result: lane (c, g) holds scores of tokens 8 c + 4 u + i, i = 0..3.
//   P.V    O[g][d] = sum_t P[g][t] V[t][d] as one 16x16x32 MFMA per 16-wide
//          slice of d over the whole chunk.
//          A operand (P): lane (c, g) holds P[g][8 c + e], e = 4 u + i, which
//          is exactly the QK^T result layout: no data moves between lanes.
//          B operand (V): lane (c, r) holds tokens 8 c .. 8 c + 7 of feature
//          16 nt + r; in the transposed V tile this is one 16-byte load.
//          A third MFMA against a ones operand sums P per head (the softmax
//          denominator) from the same bf16-rounded P the numerator uses.
//   Result rows: lane (c, r) holds O[g = 4 c + i][16 nt + r].
// Every K load instruction covers 64 contiguous bytes of each of 16 token
// rows; every V load instruction covers whole 32-byte token runs of 16
// feature rows of one or two tiles, so a chunk's loads touch only the bytes
// of its blocks, each once.
//
// Latency: the sequence length, the partition's slice of the block table (one
// entry per lane, at most 128 entries) and the query group are requested
// together before anything waits; chunk addresses then come from the table
// slice by lane reads, so no load in the streaming loop waits on another
// load.  Each wave keeps kDepth chunks (8 KiB each at head_dim 64) in flight.
//
// Split-KV: a partition's result (unnormalised accumulator, maximum and
// denominator) goes to the workspace; the last workgroup of a (sequence, KV
// head) to finish - found with a counter that it returns to zero afterwards -
// merges all partitions by the rescaled segment rule and writes the output, so
// no second kernel runs.
template <int D, int BS, int NW>
__global__ void __launch_bounds__(NW * 64)
    decode_mfma(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
                const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
                const int32_t* __restrict__ seq_lens, const DecodeParams prm) {
  static_assert(D % 32 == 0 && D <= 128, "head_dim");
  static_assert(BS == 8 || BS == 16 || BS == 32, "block_size");
  constexpr int HS = D / 32;                  // 32-wide slices of d (QK^T k-steps)
  constexpr int NT = D / 16;                  // 16-wide slices of d (P.V n-tiles)
  constexpr int NB = BS >= 32 ? 1 : 32 / BS;  // physical blocks per 32-token chunk
  constexpr int DEPTH = kDepth;
  constexpr size_t kTile = static_cast<size_t>(BS) * D;  // elements per (block, head) tile

  __shared__ float s_m[NW][16];
  __shared__ float s_l[NW][16];
  __shared__ float s_acc[NW][16][D];
  __shared__ int s_last;

  const int p = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane >> 4;
  const int r = lane & 15;
  const int G = prm.group;
  const int Hkv = prm.num_kv_heads;
  const int PS = prm.partition_size;
  const int MB = prm.max_blocks_per_seq;
  const bool balanced = prm.balanced != 0;
  const int32_t* btrow = block_tables + static_cast<size_t>(b) * MB;

  // The partition's slice of the block table, one entry per lane (<= 128).
  int tb0 = 0, tb1 = 0;
  auto load_slice = [&](int lb0, int n) {
    if (lane < n && lb0 + lane < MB) tb0 = btrow[lb0 + lane];
    if (lane + 64 < n && lb0 + lane + 64 < MB) tb1 = btrow[lb0 + lane + 64];
  };
  // Fixed-size partitions: the slice, the query group and the length are
  // requested together before anything waits.
  if (!balanced) load_slice(p * (PS / BS), PS / BS);
  bf16x8_t qop[HS];
  {
    const uint16_t* qrow =
        q + (static_cast<size_t>(b) * prm.num_q_heads + h * G + (r < G ? r : 0)) * D + 8 * c;
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) qop[hs] = load_bf16x8(qrow + 32 * hs);
    if (r >= G) {
#pragma unroll
      for (int hs = 0; hs < HS; ++hs) qop[hs] = bf16x8_t{};
    }
  }
  const int T = seq_lens[b];
  const int nparts = (T + PS - 1) / PS;
  if (p >= (nparts > 0 ? nparts : 1)) return;

  // Balanced partitions: the sequence's ceil(T / 32) chunks are dealt out
  // evenly over its nparts partitions (each then holds at most PS tokens), so
  // no workgroup is left with a short remainder while others run long.
  const int part_len =
      (balanced && nparts > 0) ? 32 * ((((T + 31) >> 5) + nparts - 1) / nparts) : PS;
  const int t_begin = p * part_len;
  const int t_end = min(t_begin + part_len, T);
  if (balanced) load_slice(t_begin / BS, part_len / BS);
  const int span = t_end - t_begin;             // tokens of this partition (0 only if T == 0)
  const int nch = (span + 31) >> 5;             // 32-token chunks
  const int last_blk = (span + BS - 1) / BS - 1;  // last table entry of the slice in use
  const float sl = prm.scale_log2;
  const size_t head_off = static_cast<size_t>(h) * kTile;
  const size_t blk_stride = static_cast<size_t>(Hkv) * kTile;

  float m2 = -INFINITY;  // running max of head g = r, base-2 units
  f32x4_t acc[NT];
  f32x4_t lsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // lane-constant parts of the addresses
  int kj[2], koff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int tok = 8 * (r >> 2) + 4 * u + (r & 3);
    kj[u] = tok / BS;
    koff[u] = (tok % BS) * D + 8 * c;
  }
  const int vj = (8 * c) / BS;
  const int voff = r * BS + (8 * c) % BS;

  // Physical block of partition-relative block lb (uniform).  Entries past
  // the last one holding tokens are never used: the index is clamped to it,
  // so every address stays inside a tile the table names, and the tokens
  // concerned are masked by selection.
  auto entry = [&](int lb) -> int {
    lb = min(lb, last_blk);
    return lb < 64 ? __builtin_amdgcn_readlane(tb0, lb) : __builtin_amdgcn_readlane(tb1, lb - 64);
  };
  auto load_chunk = [&](int k, bf16x8_t (&kr)[2][HS], bf16x8_t (&vr)[NT]) {
    const int lbc = (32 * k) / BS;
    size_t base[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
      base[j] = static_cast<size_t>(entry(lbc + j)) * blk_stride + head_off;
    auto pick = [&](int j) {
      size_t v = base[0];
#pragma unroll
      for (int jj = 1; jj < NB; ++jj) v = (j == jj) ? base[jj] : v;
      return v;
    };
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint16_t* kp = k_cache + pick(kj[u]) + koff[u];
#pragma unroll
      for (int hs = 0; hs < HS; ++hs) kr[u][hs] = load_bf16x8(kp + 32 * hs);
    }
    const uint16_t* vp = v_cache + pick(vj) + voff;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) vr[nt] = load_bf16x8(vp + 16 * nt * BS);
  };

  const bf16x8_t ones = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
  auto process_chunk = [&](int k, bf16x8_t (&kr)[2][HS], bf16x8_t (&vr)[NT]) {
    const int t = 32 * k;  // partition-relative
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[0][hs], qop[hs], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[1][hs], qop[hs], s1, 0, 0, 0);
    }
    // x[e]: score of token t + 8 c + e in base-2 units, e = 4 u + i
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = s0[i] * sl;
      x[4 + i] = s1[i] * sl;
    }
    const bool tail = t + 32 > span;  // wave-uniform
    const int valid = span - t - 8 * c;  // tokens of this lane group still in range
    if (tail) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (e < valid) ? x[e] : -INFINITY;
    }
    float cm = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, x[e]);
    cm = fmaxf(cm, __shfl_xor(cm, 16));
    cm = fmaxf(cm, __shfl_xor(cm, 32));
    // every lane of head g now holds the chunk maximum of head g
    if (__ballot(cm > m2 + kRescaleThreshold) != 0) {
      const float mn = fmaxf(m2, cm);
      const float alpha = fast_exp2(m2 - mn);  // 0 on the first chunk (m2 = -inf)
      m2 = mn;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = __shfl(alpha, 4 * c + i);  // factor of head 4 c + i
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][i] *= a;
        lsum[i] *= a;
      }
    }
    bf16x8_t pa;
#pragma unroll
    for (int e = 0; e < 8; ++e) pa[e] = static_cast<__bf16>(fast_exp2(x[e] - m2));
    if (tail) {
      // V rows of tokens >= T may hold anything (NaN included): select 0
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          vr[nt][e] = (e < valid) ? vr[nt][e] : static_cast<__bf16>(0.f);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vr[nt], acc[nt], 0, 0, 0);
    lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, ones, lsum, 0, 0, 0);
  };

  // Software pipeline over this wave's chunks w, w + NW, ...: ring slot s
  // holds chunk i with i % DEPTH == s and is refilled with chunk i + DEPTH as
  // soon as chunk i has been consumed.  In the steady-state loop every refill
  // is unconditional, so the compiler's wait counts stay exact (each wait
  // leaves the younger DEPTH - 1 chunks in flight); only the final drain has
  // conditional refills.
  const int my_n = w < nch ? (nch - 1 - w) / NW + 1 : 0;
  bf16x8_t kr[DEPTH][2][HS], vr[DEPTH][NT];
  if (my_n >= DEPTH) {
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) load_chunk(w + NW * s, kr[s], vr[s]);
    int i = 0;
    for (; i + 2 * DEPTH - 1 < my_n; i += DEPTH) {
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) {
        process_chunk(w + NW * (i + s), kr[s], vr[s]);
        load_chunk(w + NW * (i + s + DEPTH), kr[s], vr[s]);
      }
    }
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) {
      process_chunk(w + NW * (i + s), kr[s], vr[s]);
      if (i + s + DEPTH < my_n) load_chunk(w + NW * (i + s + DEPTH), kr[s], vr[s]);
    }
#pragma unroll
    for (int s = 0; s < DEPTH; ++s)
      if (i + s + DEPTH < my_n) process_chunk(w + NW * (i + s + DEPTH), kr[s], vr[s]);
  } else {
#pragma unroll
    for (int s = 0; s < DEPTH; ++s)
      if (s < my_n) load_chunk(w + NW * s, kr[s], vr[s]);
#pragma unroll
    for (int s = 0; s < DEPTH; ++s)
      if (s < my_n) process_chunk(w + NW * s, kr[s], vr[s]);
  }

  // Merge the wavefronts' (m, l, acc) in LDS by the rescaled segment rule.
  if (c == 0) s_m[w][r] = m2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = 4 * c + i;
    if (g < G) {
      if (r == 0) s_l[w][g] = lsum[i];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) s_acc[w][g][16 * nt + r] = acc[nt][i];
    }
  }
  __syncthreads();
  const bool split = nparts > 1;
  const int Hq = prm.num_q_heads;
  const int NP = prm.num_partitions;
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int g = idx / D;
    const int d = idx - g * D;
    float mx = s_m[0][g];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) mx = fmaxf(mx, s_m[ww][g]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float f = (s_m[ww][g] == -INFINITY) ? 0.f : fast_exp2(s_m[ww][g] - mx);
      num += f * s_acc[ww][g][d];
      den += f * s_l[ww][g];
    }
    const size_t row = static_cast<size_t>(b) * Hq + h * G + g;
    if (!split) {
      store_out(prm.out, row * D + d, T == 0 ? 0.f : num / den, prm.out_f32);
    } else {
      store_coherent(prm.part_out + (row * NP + p) * D + d, num);
      if (d == 0) {
        store_coherent(prm.part_ml + (row * NP + p) * 2, mx);
        store_coherent(prm.part_ml + (row * NP + p) * 2 + 1, den);
      }
    }
  }
  if (!split) return;

  // Publish this partition, then count it; the last of the nparts arrivals
  // merges.  Every thread waits until its coherent stores have completed
  // before the barrier, so they are visible chip-wide before the count is.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t* counter = prm.counters + static_cast<size_t>(b) * Hkv + h;
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == static_cast<uint32_t>(nparts - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (s_last == 0) return;
  // Every other partition's stores completed before its count, and this
  // workgroup's reads below are issued after the count it observed; the
  // reads are coherent, so they see those stores.
  // Stage every partition's (max, sum) pair in LDS (the per-wave staging area
  // is free again), then each (head, feature) thread reduces over partitions
  // with its accumulator loads all independent of each other.
  float* s_pm = &s_acc[0][0][0];
  constexpr int kStage = (NW * 16 * D) / 2;  // pairs the staging area holds
  const bool staged = G * nparts <= kStage;
  if (staged) {
    for (int idx = threadIdx.x; idx < G * nparts; idx += NW * 64) {
      const int g = idx / nparts;
      const int pp = idx - g * nparts;
      const size_t row = static_cast<size_t>(b) * Hq + h * G + g;
      s_pm[idx] = load_coherent(prm.part_ml + (row * NP + pp) * 2);
      s_pm[kStage + idx] = load_coherent(prm.part_ml + (row * NP + pp) * 2 + 1);
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int g = idx / D;
    const int d = idx - g * D;
    const size_t row = static_cast<size_t>(b) * Hq + h * G + g;
    const float* po = prm.part_out + row * NP * D + d;
    float mx = -INFINITY, num = 0.f, den = 0.f;
    if (staged) {
      const float* pm = s_pm + g * nparts;
      const float* pl = s_pm + kStage + g * nparts;
      for (int pp = 0; pp < nparts; ++pp) mx = fmaxf(mx, pm[pp]);
#pragma unroll 16
      for (int pp = 0; pp < nparts; ++pp) {
        const float f = fast_exp2(pm[pp] - mx);
        num += f * load_coherent(po + static_cast<size_t>(pp) * D);
        den += f * pl[pp];
      }
    } else {
      const float* ml = prm.part_ml + row * NP * 2;
      for (int pp = 0; pp < nparts; ++pp) mx = fmaxf(mx, load_coherent(ml + 2 * pp));
      for (int pp = 0; pp < nparts; ++pp) {
        const float f = fast_exp2(load_coherent(ml + 2 * pp) - mx);
        num += f * load_coherent(po + static_cast<size_t>(pp) * D);
        den += f * load_coherent(ml + 2 * pp + 1);
      }
    }
    store_out(prm.out, row * D + d, num / den, prm.out_f32);
  }
  // every arrival has been counted: leave the counter at zero for the next call
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Generic vector kernel: one wavefront per (partition, q head, sequence).
// Lane l owns features l, l + 64, ...; each token's score is a wavefront sum.
template <int DPL>
__global__ void __launch_bounds__(64)
    decode_generic(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
                   const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
                   const int32_t* __restrict__ seq_lens, const DecodeParams prm) {
  const int p = blockIdx.x;
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int T = seq_lens[b];
  const int PS = prm.partition_size;
  const int nparts = (T + PS - 1) / PS;
  if (p >= (nparts > 0 ? nparts : 1)) return;
  const int D = prm.head_dim;
  const int BS = prm.block_size;
  const int h = hq / prm.group;
  const int lane = threadIdx.x;
  const size_t tile = static_cast<size_t>(BS) * D;
  const int32_t* btrow = block_tables + static_cast<size_t>(b) * prm.max_blocks_per_seq;

  float qv[DPL], acc[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const int d = lane + 64 * k;
    qv[k] = d < D ? bf16_bits_to_float(q[(static_cast<size_t>(b) * prm.num_q_heads + hq) * D + d]) *
                        prm.scale_log2
                  : 0.f;
    acc[k] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int t_begin = p * PS;
  const int t_end = min(t_begin + PS, T);
  for (int t = t_begin; t < t_end; ++t) {
    const int phys = btrow[t / BS];
    const int o = t % BS;
    const size_t base = (static_cast<size_t>(phys) * prm.num_kv_heads + h) * tile;
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int d = lane + 64 * k;
      if (d < D) s += qv[k] * bf16_bits_to_float(k_cache[base + static_cast<size_t>(o) * D + d]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    const float mn = fmaxf(m, s);
    const float alpha = fast_exp2(m - mn);
    const float pe = fast_exp2(s - mn);
    l = l * alpha + pe;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int d = lane + 64 * k;
      const float v = d < D ? bf16_bits_to_float(v_cache[base + static_cast<size_t>(d) * BS + o]) : 0.f;
      acc[k] = acc[k] * alpha + pe * v;
    }
    m = mn;
  }
  const bool empty = (T == 0);
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const int d = lane + 64 * k;
    if (d < D) write_partition_result(prm, b, hq, p, nparts, d, empty ? 0.f : acc[k] / l, m, l, empty);
  }
}

// ---------------------------------------------------------------------------
// Merge: out = sum_r w_r o_r / sum_r w_r, w_r = exp(ln Z_r - max_r ln Z_r).
// Empty segments (ln Z_r = -inf) are skipped by selection, so whatever their
// o_r holds never reaches the sum.
template <int DPL>
__global__ void __launch_bounds__(64)
    merge_states(const float* __restrict__ part_out, const float* __restrict__ part_lse,
                 int32_t part_stride, int32_t num_parts, int32_t D,
                 const int32_t* __restrict__ seq_lens, int32_t rows_per_seq, int32_t PS,
                 void* out, int out_f32) {
  const int row = blockIdx.x;
  int n = num_parts;
  if (seq_lens != nullptr) {
    const int T = seq_lens[row / rows_per_seq];
    n = (T + PS - 1) / PS;
    if (n <= 1) return;
  }
  const float* lse = part_lse + static_cast<size_t>(row) * part_stride;
  const float* po = part_out + static_cast<size_t>(row) * part_stride * D;
  float mx = -INFINITY;
  for (int i = 0; i < n; ++i) mx = fmaxf(mx, lse[i]);
  const int lane = threadIdx.x;
  float num[DPL], den = 0.f;
#pragma unroll
  for (int k = 0; k < DPL; ++k) num[k] = 0.f;
  if (mx != -INFINITY) {
    for (int i = 0; i < n; ++i) {
      const float li = lse[i];
      if (li == -INFINITY) continue;  // uniform: every lane reads the same lse
      const float wgt = fast_exp2((li - mx) * kLog2e);
      den += wgt;
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const int d = lane + 64 * k;
        if (d < D) num[k] += wgt * po[static_cast<size_t>(i) * D + d];
      }
    }
  }
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const int d = lane + 64 * k;
    if (d < D)
      store_out(out, static_cast<size_t>(row) * D + d, mx == -INFINITY ? 0.f : num[k] / den,
                out_f32);
  }
}

template <int D, int BS>
hipError_t launch_mfma_w(const DecodeLaunch& a, int waves, dim3 grid, hipStream_t stream) {
  switch (waves) {
    case 1:
      decode_mfma<D, BS, 1><<<grid, 64, 0, stream>>>(a.q, a.k_cache, a.v_cache, a.block_tables,
                                                     a.seq_lens, a.prm);
      break;
    case 2:
      decode_mfma<D, BS, 2><<<grid, 128, 0, stream>>>(a.q, a.k_cache, a.v_cache, a.block_tables,
                                                      a.seq_lens, a.prm);
      break;
    default:
      decode_mfma<D, BS, 4><<<grid, 256, 0, stream>>>(a.q, a.k_cache, a.v_cache, a.block_tables,
                                                      a.seq_lens, a.prm);
      break;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_mfma_bs(const DecodeLaunch& a, int waves, dim3 grid, hipStream_t stream) {
  switch (a.prm.block_size) {
    case 8: return launch_mfma_w<D, 8>(a, waves, grid, stream);
    case 16: return launch_mfma_w<D, 16>(a, waves, grid, stream);
    default: return launch_mfma_w<D, 32>(a, waves, grid, stream);
  }
}

hipError_t launch_merge_for(const DecodeLaunch& a, hipStream_t stream) {
  const DecodeParams& prm = a.prm;
  return launch_merge(prm.part_out, prm.part_lse, a.num_seqs * prm.num_q_heads,
                      prm.num_partitions, prm.num_partitions, prm.head_dim, a.seq_lens,
                      prm.num_q_heads, prm.partition_size, prm.out, prm.out_f32, stream);
}

}  // namespace

bool mfma_shape_supported(int head_dim, int block_size, int group, int partition_size) {
  return (head_dim == 64 || head_dim == 128) &&
         (block_size == 8 || block_size == 16 || block_size == 32) && group >= 1 &&
         group <= 16 && partition_size > 0 && partition_size % 32 == 0 &&
         partition_size / block_size <= 128;
}

bool generic_shape_supported(int head_dim, int block_size, int group) {
  return head_dim >= 1 && head_dim <= 256 && block_size >= 1 && group >= 1;
}

hipError_t launch_decode_mfma(const DecodeLaunch& a, int waves, hipStream_t stream) {
  const dim3 grid(a.prm.num_partitions, a.prm.num_kv_heads, a.num_seqs);
  return (a.prm.head_dim == 64) ? launch_mfma_bs<64>(a, waves, grid, stream)
                                : launch_mfma_bs<128>(a, waves, grid, stream);
}

hipError_t launch_decode_generic(const DecodeLaunch& a, hipStream_t stream) {
  const dim3 grid(a.prm.num_partitions, a.prm.num_q_heads, a.num_seqs);
  const int dpl = (a.prm.head_dim + 63) / 64;
  switch (dpl) {
    case 1:
      decode_generic<1><<<grid, 64, 0, stream>>>(a.q, a.k_cache, a.v_cache, a.block_tables,
                                                 a.seq_lens, a.prm);
      break;
    case 2:
      decode_generic<2><<<grid, 64, 0, stream>>>(a.q, a.k_cache, a.v_cache, a.block_tables,
                                                 a.seq_lens, a.prm);
      break;
    case 3:
      decode_generic<3><<<grid, 64, 0, stream>>>(a.q, a.k_cache, a.v_cache, a.block_tables,
                                                 a.seq_lens, a.prm);
      break;
    default:
      decode_generic<4><<<grid, 64, 0, stream>>>(a.q, a.k_cache, a.v_cache, a.block_tables,
                                                 a.seq_lens, a.prm);
      break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.prm.num_partitions <= 1) return e;
  return launch_merge_for(a, stream);
}

hipError_t launch_merge(const float* part_out, const float* part_lse, int32_t num_rows,
                        int32_t part_stride, int32_t num_parts, int32_t head_dim,
                        const int32_t* seq_lens, int32_t rows_per_seq, int32_t partition_size,
                        void* out, int out_f32, hipStream_t stream) {
  if (num_rows <= 0) return hipSuccess;
  const dim3 grid(num_rows);
  const int dpl = (head_dim + 63) / 64;
#define PKV_MERGE(N)                                                                         \
  merge_states<N><<<grid, 64, 0, stream>>>(part_out, part_lse, part_stride, num_parts,       \
                                           head_dim, seq_lens, rows_per_seq, partition_size, \
                                           out, out_f32)
  switch (dpl) {
    case 1: PKV_MERGE(1); break;
    case 2: PKV_MERGE(2); break;
    case 3: PKV_MERGE(3); break;
    default: PKV_MERGE(4); break;
  }
#undef PKV_MERGE
  return hipGetLastError();
}

}  // namespace pkv
