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
//   decode_stream   matrix-core kernel.  The work of a call - every
//                   (sequence, KV head) unit cut into 32-token chunks - is
//                   dealt out in equal contiguous shares to a fixed set of
//                   wavefronts, so all of them stream HBM until the end; a unit
//                   cut between wavefronts is merged by the last of them.  (The
//                   default, decode_wg in decode_wg.hip, deals the same work to
//                   whole workgroups.)
//   decode_mfma     matrix-core kernel over fixed partitions: one workgroup
//                   per (partition, KV head, sequence), its waves taking the
//                   partition's chunks round robin, split sequences merged by
//                   the last partition to finish.
//   decode_generic  one wavefront per (partition, q head, sequence), scalar
//                   fp32 online softmax; any head_dim <= 256, any block size.
//   merge_states    one wavefront per (sequence, q head): combines partition
//                   results (o_r, ln Z_r) into the output (vector kernel path
//                   and the standalone merge entry point).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "chunk.h"
#include "internal.h"

namespace pkv {
namespace {

// Finishes one (sequence, q head) row of a vector-kernel partition: either the
// final output (single partition) or the partition's (o_r, ln Z_r).  `m2` is
// the maximum in base-2 units, `den` the sum of 2^(x - m2).
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
// Stream kernel.
//
// Work units are (sequence b, KV head h) in the order u = b Hkv + h; unit u
// holds n_b = ceil(T_b / 32) chunks, and the C = Hkv sum_b n_b chunks of a
// call are numbered in unit order.  Wavefront g of the W launched takes chunks
// [g C / W', (g + 1) C / W') with W' = min(W, C), so every wavefront streams
// the same number of bytes, to one chunk.  The stretch of a unit inside one
// wavefront's range is a piece.  A piece that is a whole unit writes the
// output (held in LDS until the wavefront's last load when there is room, as
// is the range's first piece, the one that ends while chunks are still
// loading).  Otherwise it publishes (acc, max, sum) into workspace slot
// u + g (unique: ranges and units both advance with g, so two pieces with the
// same u + g cannot exist), counts itself on the unit's counter and, if it is
// the last of the unit's pieces (one per wavefront from the owner of the
// unit's first chunk to the owner of its last), merges them all by the
// rescaled segment rule into the output.
//
// Set-up: each workgroup puts the sequence lengths and the exclusive prefix
// of chunk counts in LDS.  Each wavefront then takes its range in batches of
// up to 64 chunks: lane i works out chunk i's unit, position in the unit,
// valid token count and physical blocks (one table read each), and the
// streaming loop reads these back by lane, with no memory access, kDepth
// chunks ahead of the one it folds in.
constexpr int kStreamWaves = 4;       // wavefronts per workgroup, each with its own range
constexpr int kStreamMaxSeqs = 2048;  // sequences whose lengths and prefix fit in LDS

template <int D, int BS, bool kStream>
__global__ void __launch_bounds__(kStreamWaves * 64)
    __attribute__((amdgpu_waves_per_eu(D <= 64 ? 2 : 1))) decode_stream(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
                  const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
                  const int32_t* __restrict__ seq_lens, const DecodeParams prm) {
  using M = Mfma<D, BS>;
  using Regs = typename M::Regs;
  constexpr int NB = M::NB;
  constexpr int HS = M::HS;
  constexpr int NT = M::NT;
  constexpr int DEPTH = kDepth;
  constexpr int NTH = kStreamWaves * 64;
  constexpr int kBlocksPerChunk = 32 / BS < 1 ? 1 : 32 / BS;
  __shared__ int s_len[kStreamMaxSeqs];
  __shared__ int s_pre[kStreamMaxSeqs + 1];
  __shared__ int s_wsum[kStreamWaves];
  constexpr int kMergeStage = 256;  // (max, sum) pairs a wavefront can stage for a merge
  __shared__ float s_mrg[kStreamWaves][2 * kMergeStage];
  // Output rows of whole units a wavefront holds back until its last load
  // (a store among the ring's loads holds up every later load until it is
  // acknowledged, the memory counter retiring them in issue order).
  constexpr int kStageFloats = 2048;
  constexpr int kStageUnits = 16;
  __shared__ float s_out[kStreamWaves][kStageFloats];
  __shared__ int s_orow[kStreamWaves][kStageUnits];

  const int S = prm.num_seqs;
  const int Hkv = prm.num_kv_heads;
  const int Hq = prm.num_q_heads;
  const int G = prm.group;
  const int MB = prm.max_blocks_per_seq;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane >> 4;
  const int r = lane & 15;

  // 1. Lengths, and the exclusive prefix of per-sequence chunk counts.
  chunk_prefix<NTH>(seq_lens, S, s_len, s_pre, s_wsum, tid);

  // 2. Sequences with no tokens get a zero output row.
  zero_empty_rows<D, NTH>(prm, s_len, tid);

  // 3. This wavefront's share of the chunks.  (No barrier below this point:
  // the wavefronts of a workgroup are independent from here on.)
  const int64_t C = static_cast<int64_t>(Hkv) * s_pre[S];
  const int64_t W = static_cast<int64_t>(gridDim.x) * kStreamWaves;
  const int64_t Weff = C < W ? C : W;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kStreamWaves + w;
  // A fused step's cache writes: wavefront gw of the grid writes the new
  // tokens of units gw, gw + (all wavefronts), ...  The memory counter retires
  // a wavefront's stores and loads in issue order, so a store issued among the
  // ring's loads would hold up every load behind it until it is acknowledged:
  // the first unit's rows are loaded now and written at the end, after the
  // pieces' publication, and any further units after that.
  const int fused = prm.k_new != nullptr ? 1 : 0;
  const int units = S * Hkv;
  const int gw = static_cast<int>(g);
  const int gwaves = static_cast<int>(W);
  if (g >= Weff) {  // no chunks here: only the writes
    if (fused)
      for (int u = gw; u < units; u += gwaves) {
        TokenWrite<D, BS> more;
        more.load(prm, block_tables, u, s_len[u / Hkv], lane);
        more.store(prm, lane);
      }
    return;
  }
  TokenWrite<D, BS> tw;
  if (fused && gw < units) tw.load(prm, block_tables, gw, s_len[gw / Hkv], lane);
  const int64_t start = g * C / Weff;
  const int64_t end = (g + 1) * C / Weff;

  const typename M::Lane ln(c, r);
  const float sl = prm.scale_log2;
  const size_t blk_stride = static_cast<size_t>(Hkv) * M::kTile;
  typename M::State st;
  st.reset();
  struct Slot {  // one ring entry: a chunk's K/V operands and its unit's query group
    Regs x;
    bf16x8_t q[HS];
    NewToken<D> nt;  // the new token of a fused decode step (zeros where none)
  };
  int pb = 0, ph = 0, plc0 = 0;  // the piece being folded: sequence, KV head, first chunk

  // The pieces of unit (sb, sh): one per wavefront from the owner of the
  // unit's first chunk (gf) to the owner of its last (gl).
  auto unit_span = [&](int sb, int sh, int64_t& gf, int64_t& gl) {
    const int nb = (s_len[sb] + 31) >> 5;
    const int64_t cu0 = static_cast<int64_t>(Hkv) * s_pre[sb] + static_cast<int64_t>(sh) * nb;
    gf = ((cu0 + 1) * Weff - 1) / C;
    gl = ((cu0 + nb) * Weff - 1) / C;
  };
  // Publishes the state of the current piece (a part of unit (pb, ph)) into
  // workspace slot u + g with device-coherent stores.
  auto publish = [&]() {
    const int64_t u = static_cast<int64_t>(pb) * Hkv + ph;
    float* pacc = prm.part_out + (u + g) * G * D;  // [G][D]
    float* pml = prm.part_ml + (u + g) * G * 2;    // [G][max, sum]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int gh = 4 * c + i;
      if (gh < G) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) store_coherent(pacc + gh * D + 16 * nt + r, st.acc[nt][i]);
        if (r == 0) store_coherent(pml + gh * 2 + 1, st.lsum[i]);
      }
    }
    if (c == 0 && r < G) store_coherent(pml + r * 2, st.m2);
  };
  // Counts a published piece of unit (sb, sh) whose stores have completed;
  // returns the count before this arrival.
  auto count = [&](int sb, int sh) -> uint32_t {
    uint32_t prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(prm.counters + static_cast<int64_t>(sb) * Hkv + sh, 1u,
                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return prev;
  };
  // Merges every piece of unit (sb, sh) - all published and counted - into
  // the output, in wavefront order, and leaves its counter at zero.
  auto merge_unit = [&](int sb, int sh) {
    const int64_t u = static_cast<int64_t>(sb) * Hkv + sh;
    const size_t row0 = static_cast<size_t>(sb) * Hq + static_cast<size_t>(sh) * G;
    int64_t gf, gl;
    unit_span(sb, sh, gf, gl);
    // Merge the unit's k pieces in wavefront order (so the result does not
    // depend on which piece arrived last).  Their (max, sum) pairs
    // go to this wavefront's LDS area, all loads in flight at once; then each
    // lane folds four adjacent features of one head, sixteen pieces' loads at
    // a time.
    const int k = static_cast<int>(gl - gf + 1);
    float* sm = s_mrg[w];
    float* sq = s_mrg[w] + kMergeStage;
    const bool staged = G * k <= kMergeStage;
    if (staged) {
      // the unit's k slots: acc [k][G][D] and (max, sum) [k][G][2]
      const CoherentReader racc(prm.part_out + (u + gf) * G * D,
                                static_cast<uint32_t>(k * G * D * sizeof(float)));
      const CoherentReader rml(prm.part_ml + (u + gf) * G * 2,
                               static_cast<uint32_t>(k * G * 2 * sizeof(float)));
      // G * k <= 256: at most four (head, piece) pairs per lane, loaded first
      float m4[4], l4[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int idx = min(lane + 64 * t, G * k - 1);
        const int gh = idx / k;
        const int j = idx - gh * k;
        const uint32_t off = static_cast<uint32_t>((j * G + gh) * 2 * sizeof(float));
        m4[t] = rml.f32(off);
        l4[t] = rml.f32(off + sizeof(float));
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int idx = lane + 64 * t;
        if (idx < G * k) {
          sm[idx] = m4[t];
          sq[idx] = l4[t];
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int e = lane; e < G * D / 4; e += 64) {
        const int gh = (4 * e) / D;
        const int d0 = 4 * e - gh * D;
        float mx = -INFINITY;
        for (int j = 0; j < k; ++j) mx = fmaxf(mx, sm[gh * k + j]);
        float den = 0.f;
        f32x4_t nm = {0.f, 0.f, 0.f, 0.f};
        // sixteen pieces' accumulators in flight at a time (the batches
        // depend on each other only through the sums)
        for (int j0 = 0; j0 < k; j0 += 16) {
          f32x4_t a[16];
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const int j = min(j0 + t, k - 1);
            a[t] = racc.f32x4(static_cast<uint32_t>(((j * G + gh) * D + d0) * sizeof(float)));
          }
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            if (j0 + t < k) {
              const float f = fast_exp2(sm[gh * k + j0 + t] - mx);
              den += f * sq[gh * k + j0 + t];
              nm += f * a[t];
            }
          }
        }
        const float inv = 1.0f / den;
        const size_t o = (row0 + gh) * D + d0;
        store_out(prm.out, o, nm[0] * inv, prm.out_f32);
        store_out(prm.out, o + 1, nm[1] * inv, prm.out_f32);
        store_out(prm.out, o + 2, nm[2] * inv, prm.out_f32);
        store_out(prm.out, o + 3, nm[3] * inv, prm.out_f32);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int gh = 4 * c + i;
        if (gh < G) {
          float mx = -INFINITY, den = 0.f, num[NT];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) num[nt] = 0.f;
          for (int64_t gg = gf; gg <= gl; ++gg) {
            const float* oml = prm.part_ml + ((u + gg) * G + gh) * 2;
            const float* oacc = prm.part_out + ((u + gg) * G + gh) * D + r;
            const float mj = load_coherent(oml);
            const float lj = load_coherent(oml + 1);
            const float mn = fmaxf(mx, mj);
            const float fo = fast_exp2(mx - mn);  // 0 for the first piece
            const float fj = fast_exp2(mj - mn);
            den = den * fo + lj * fj;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              num[nt] = num[nt] * fo + load_coherent(oacc + 16 * nt) * fj;
            mx = mn;
          }
          const float inv = 1.0f / den;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            store_out(prm.out, (row0 + gh) * D + 16 * nt + r, num[nt] * inv, prm.out_f32);
        }
      }
    }
    // every piece has been counted: leave the counter at zero for the next call
    if (lane == 0)
      __hip_atomic_store(prm.counters + u, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // A wavefront's range is contiguous, so only its first and its last piece
  // can be parts of units; every unit in between is whole.  Partial pieces
  // are published when they end and counted together once the range is done
  // - one wait for all stores, then both counts - so the chunk ring never
  // drains in mid-range.
  int np_pub = 0, pub_b0 = 0, pub_h0 = 0, pub_b1 = 0, pub_h1 = 0;
  // The range's first piece (a part of a unit) held back at the end of
  // s_out[w], laid out as its workspace slot ([G][D] then [G][max, sum]),
  // when it fits; whole units' rows held back in front of it: nst of at
  // most scap.
  const int pfl = G * D + 2 * G;
  const bool pfit = pfl <= kStageFloats;
  float* sp = s_out[w] + (pfit ? kStageFloats - pfl : 0);
  const int scap = min(kStageUnits, (kStageFloats - (pfit ? pfl : 0)) / (G * D));
  int nst = 0;
  int pheld = 0;
  // Ends the current piece whose last chunk is `last_lc` of its unit.
  auto finish_piece = [&](int last_lc) {
    const int T = s_len[pb];
    const int nb = (T + 31) >> 5;
    const size_t row0 = static_cast<size_t>(pb) * Hq + static_cast<size_t>(ph) * G;
    if (plc0 == 0 && last_lc == nb - 1 && nst < scap) {  // the whole unit, held back
      float* so = s_out[w] + nst * G * D;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int gh = 4 * c + i;
        if (gh < G) {
          const float inv = 1.0f / st.lsum[i];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) so[gh * D + 16 * nt + r] = st.acc[nt][i] * inv;
        }
      }
      if (lane == 0) s_orow[w][nst] = static_cast<int>(row0);
      ++nst;
      return;
    }
    if (plc0 == 0 && last_lc == nb - 1) {  // the whole unit, no room to hold it back
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int gh = 4 * c + i;
        if (gh < G) {
          const float inv = 1.0f / st.lsum[i];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            store_out(prm.out, (row0 + gh) * D + 16 * nt + r, st.acc[nt][i] * inv, prm.out_f32);
        }
      }
      return;
    }
    if (np_pub == 0 && pfit) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int gh = 4 * c + i;
        if (gh < G) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) sp[gh * D + 16 * nt + r] = st.acc[nt][i];
          if (r == 0) sp[G * D + gh * 2 + 1] = st.lsum[i];
        }
      }
      if (c == 0 && r < G) sp[G * D + r * 2] = st.m2;
      pheld = 1;
    } else {
      publish();
    }
    if (np_pub == 0) {
      pub_b0 = pb;
      pub_h0 = ph;
    } else {
      pub_b1 = pb;
      pub_h1 = ph;
    }
    ++np_pub;
  };

  for (int64_t bat = start; bat < end; bat += 64) {
    const int n = static_cast<int>(end - bat < 64 ? end - bat : 64);
    // Lane i describes chunk bat + i: sequence, KV head, chunk of the unit,
    // valid tokens, piece start / end flags and physical blocks.
    int cb = 0, chd = 0, clc = 0, cval = 0, cfl = 0;
    int ent[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) ent[j] = 0;
    if (lane < n) {
      const int64_t cc = bat + lane;
      int lo = 0, hi = S;  // largest lo with Hkv * s_pre[lo] <= cc
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (static_cast<int64_t>(Hkv) * s_pre[mid] <= cc)
          lo = mid;
        else
          hi = mid;
      }
      const int T = s_len[lo];
      const int nb = (T + 31) >> 5;
      const int rem = static_cast<int>(cc - static_cast<int64_t>(Hkv) * s_pre[lo]);
      cb = lo;
      chd = rem / nb;
      clc = rem - chd * nb;
      cval = min(32, T - 32 * clc);
      cfl = ((cc == start || clc == 0) ? 1 : 0) | ((cc == end - 1 || clc == nb - 1) ? 2 : 0) |
            (clc == nb - 1 ? 4 : 0);
      const int last_blk = (T + BS - 1) / BS - 1;
      const int32_t* row = block_tables + static_cast<size_t>(lo) * MB;
#pragma unroll
      for (int j = 0; j < NB; ++j) ent[j] = row[min(clc * kBlocksPerChunk + j, last_blk)];
    }

    auto issue = [&](int i, Slot& sl8) {
      const int hh = __builtin_amdgcn_readlane(chd, i);
      const size_t head_off = static_cast<size_t>(hh) * M::kTile;
      size_t base[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j)
        base[j] = static_cast<size_t>(__builtin_amdgcn_readlane(ent[j], i)) * blk_stride + head_off;
      M::template load<kStream>(k_cache, v_cache, base, ln, sl8.x);
      // the chunk's query group travels with it (512 bytes per unit, cached
      // after its first chunk), so a piece starting needs no load of its own
      M::load_q(q, Hq, G, __builtin_amdgcn_readlane(cb, i), hh, c, r, sl8.q);
      const bool fresh = prm.k_new != nullptr && (__builtin_amdgcn_readlane(cfl, i) & 4) != 0;
      const size_t row = (static_cast<size_t>(__builtin_amdgcn_readlane(cb, i)) * Hkv + hh) * D;
      sl8.nt.load(fresh ? prm.k_new + row : nullptr, fresh ? prm.v_new + row : nullptr, fresh, c,
                  r);
    };
    auto consume = [&](int i, Slot& sl8) {
      Regs& x = sl8.x;
      const int fl = __builtin_amdgcn_readlane(cfl, i);
      if (fl & 1) {  // a piece starts: a fresh state
        pb = __builtin_amdgcn_readlane(cb, i);
        ph = __builtin_amdgcn_readlane(chd, i);
        plc0 = __builtin_amdgcn_readlane(clc, i);
        st.reset();
      }
      const int valid = __builtin_amdgcn_readlane(cval, i);
      if ((fl & 4) && prm.k_new != nullptr) {
        // The unit's last chunk holds the new token (chunk position
        // valid - 1): its K/V, loaded with the chunk, replace the operands,
        // whether the slot was read before or after its write.
        patch_new_operands<D, BS>(x, sl8.nt, valid, lane);
      }
      M::step(sl8.q, x, valid, sl, c, st);
      if (fl & 2) finish_piece(__builtin_amdgcn_readlane(clc, i));
    };

    // Ring of DEPTH chunks in flight; the steady-state refills are
    // unconditional so the wait counts stay exact, only the drain is not.
    Slot ring[DEPTH];
    if (n >= DEPTH) {
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) issue(s, ring[s]);
      int i = 0;
      for (; i + 2 * DEPTH - 1 < n; i += DEPTH) {
#pragma unroll
        for (int s = 0; s < DEPTH; ++s) {
          consume(i + s, ring[s]);
          issue(i + s + DEPTH, ring[s]);
        }
      }
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) {
        consume(i + s, ring[s]);
        if (i + s + DEPTH < n) issue(i + s + DEPTH, ring[s]);
      }
#pragma unroll
      for (int s = 0; s < DEPTH; ++s)
        if (i + s + DEPTH < n) consume(i + s + DEPTH, ring[s]);
    } else {
#pragma unroll
      for (int s = 0; s < DEPTH; ++s)
        if (s < n) issue(s, ring[s]);
#pragma unroll
      for (int s = 0; s < DEPTH; ++s)
        if (s < n) consume(s, ring[s]);
    }
  }

  // Count the published pieces (their stores complete first) and merge each
  // unit this wavefront closed.
  if (pheld) {  // publish the held-back first piece
    const int64_t u = static_cast<int64_t>(pub_b0) * Hkv + pub_h0;
    float* pacc = prm.part_out + (u + g) * G * D;
    float* pml = prm.part_ml + (u + g) * G * 2;
    for (int e = lane; e < G * D; e += 64) store_coherent(pacc + e, sp[e]);
    if (lane < 2 * G) store_coherent(pml + lane, sp[G * D + lane]);
  }
  if (np_pub > 0) {
    __builtin_amdgcn_s_waitcnt(0);
    const uint32_t prev0 = count(pub_b0, pub_h0);
    const uint32_t prev1 = np_pub > 1 ? count(pub_b1, pub_h1) : 0u;
    for (int t = 0; t < np_pub; ++t) {
      const int sb = t == 0 ? pub_b0 : pub_b1;
      const int sh = t == 0 ? pub_h0 : pub_h1;
      int64_t gf, gl;
      unit_span(sb, sh, gf, gl);
      const uint32_t prev = __builtin_amdgcn_readfirstlane(t == 0 ? prev0 : prev1);
      if (prev == static_cast<uint32_t>(gl - gf)) merge_unit(sb, sh);
    }
  }
  // the held-back output rows (a unit's G rows are consecutive in the output)
  for (int k = 0; k < nst; ++k) {
    const size_t o = static_cast<size_t>(s_orow[w][k]) * D;
    const float* so = s_out[w] + k * G * D;
    for (int e = lane; e < G * D; e += 64) store_out(prm.out, o + e, so[e], prm.out_f32);
  }
  if (fused) {
    if (gw < units) tw.store(prm, lane);
    for (int u = gw + gwaves; u < units; u += gwaves) {
      TokenWrite<D, BS> more;
      more.load(prm, block_tables, u, s_len[u / Hkv], lane);
      more.store(prm, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// Partitioned kernel.
//
// One workgroup per (partition, KV head, sequence); its NW wavefronts take the
// partition's chunks round robin (wave w: chunks w, w + NW, ...) and merge
// through LDS.  Partitions hold partition_size tokens (a sequence's last one
// fewer), or - balanced - share the sequence's chunks evenly.  The
// partition's slice of the block table (at most 128 entries) is read with one
// load per lane and looked up by lane reads.  A split sequence's partitions
// publish (acc, max, sum) to the workspace and count themselves on the
// (sequence, KV head) counter; the last to arrive merges them all.
template <int D, int BS, int NW>
__global__ void __launch_bounds__(NW * 64)
    decode_mfma(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
                const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
                const int32_t* __restrict__ seq_lens, const DecodeParams prm) {
  using M = Mfma<D, BS>;
  using Regs = typename M::Regs;
  constexpr int NB = M::NB;
  constexpr int HS = M::HS;
  constexpr int NT = M::NT;
  constexpr int DEPTH = kDepth;

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
  const int Hq = prm.num_q_heads;
  const int PS = prm.partition_size;
  const int MB = prm.max_blocks_per_seq;
  const bool balanced = prm.balanced != 0;
  const int32_t* btrow = block_tables + static_cast<size_t>(b) * MB;

  // The partition's slice of the block table, one entry per lane (<= 128).
  int tb0 = 0, tb1 = 0;
  auto load_slice = [&](int lb0, int cnt) {
    if (lane < cnt && lb0 + lane < MB) tb0 = btrow[lb0 + lane];
    if (lane + 64 < cnt && lb0 + lane + 64 < MB) tb1 = btrow[lb0 + lane + 64];
  };
  // Fixed-size partitions: the slice, the query group and the length are
  // requested together before anything waits.
  if (!balanced) load_slice(p * (PS / BS), PS / BS);
  bf16x8_t qop[HS];
  M::load_q(q, Hq, G, b, h, c, r, qop);
  const int T = seq_lens[b];
  const int nparts = (T + PS - 1) / PS;
  if (p >= (nparts > 0 ? nparts : 1)) return;

  // Balanced partitions: the sequence's ceil(T / 32) chunks are dealt out
  // evenly over its nparts partitions (each then holds at most PS tokens).
  const int part_len =
      (balanced && nparts > 0) ? 32 * ((((T + 31) >> 5) + nparts - 1) / nparts) : PS;
  const int t_begin = p * part_len;
  const int t_end = min(t_begin + part_len, T);
  if (balanced) load_slice(t_begin / BS, part_len / BS);
  const int span = t_end - t_begin;               // tokens of this partition (0 only if T == 0)
  const int nch = (span + 31) >> 5;               // 32-token chunks
  const int last_blk = (span + BS - 1) / BS - 1;  // last table entry of the slice in use
  const float sl = prm.scale_log2;
  const size_t head_off = static_cast<size_t>(h) * M::kTile;
  const size_t blk_stride = static_cast<size_t>(Hkv) * M::kTile;
  const typename M::Lane ln(c, r);
  typename M::State st;
  st.reset();

  // Physical block of partition-relative block lb (uniform).  Entries past
  // the last one holding tokens are never used: the index is clamped to it,
  // so every address stays inside a tile the table names, and the tokens
  // concerned are masked by selection.
  auto entry = [&](int lb) -> int {
    lb = min(lb, last_blk);
    return lb < 64 ? __builtin_amdgcn_readlane(tb0, lb) : __builtin_amdgcn_readlane(tb1, lb - 64);
  };
  auto issue = [&](int k, Regs& x) {
    const int lbc = (32 * k) / BS;
    size_t base[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
      base[j] = static_cast<size_t>(entry(lbc + j)) * blk_stride + head_off;
    M::load(k_cache, v_cache, base, ln, x);
  };
  auto consume = [&](int k, Regs& x) { M::step(qop, x, min(32, span - 32 * k), sl, c, st); };

  // Ring over this wave's chunks w, w + NW, ...: slot s holds chunk i with
  // i % DEPTH == s and is refilled with chunk i + DEPTH as soon as chunk i has
  // been consumed.  Steady-state refills are unconditional, so the compiler's
  // wait counts stay exact; only the drain has conditional refills.
  const int my_n = w < nch ? (nch - 1 - w) / NW + 1 : 0;
  Regs ring[DEPTH];
  if (my_n >= DEPTH) {
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) issue(w + NW * s, ring[s]);
    int i = 0;
    for (; i + 2 * DEPTH - 1 < my_n; i += DEPTH) {
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) {
        consume(w + NW * (i + s), ring[s]);
        issue(w + NW * (i + s + DEPTH), ring[s]);
      }
    }
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) {
      consume(w + NW * (i + s), ring[s]);
      if (i + s + DEPTH < my_n) issue(w + NW * (i + s + DEPTH), ring[s]);
    }
#pragma unroll
    for (int s = 0; s < DEPTH; ++s)
      if (i + s + DEPTH < my_n) consume(w + NW * (i + s + DEPTH), ring[s]);
  } else {
#pragma unroll
    for (int s = 0; s < DEPTH; ++s)
      if (s < my_n) issue(w + NW * s, ring[s]);
#pragma unroll
    for (int s = 0; s < DEPTH; ++s)
      if (s < my_n) consume(w + NW * s, ring[s]);
  }

  // Merge the wavefronts' (m, l, acc) in LDS by the rescaled segment rule.
  if (c == 0) s_m[w][r] = st.m2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = 4 * c + i;
    if (g < G) {
      if (r == 0) s_l[w][g] = st.lsum[i];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) s_acc[w][g][16 * nt + r] = st.acc[nt][i];
    }
  }
  __syncthreads();
  const bool split = nparts > 1;
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
      const CoherentReader rml(prm.part_ml + row * NP * 2,
                               static_cast<uint32_t>(NP * 2 * sizeof(float)));
      s_pm[idx] = rml.f32(static_cast<uint32_t>(pp * 2 * sizeof(float)));
      s_pm[kStage + idx] = rml.f32(static_cast<uint32_t>((pp * 2 + 1) * sizeof(float)));
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
      const CoherentReader racc(prm.part_out + row * NP * D,
                                static_cast<uint32_t>(NP * D * sizeof(float)));
      for (int pp = 0; pp < nparts; ++pp) mx = fmaxf(mx, pm[pp]);
      // eight partitions' accumulators in flight at a time
      for (int p0 = 0; p0 < nparts; p0 += 8) {
        float a[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int pp = min(p0 + t, nparts - 1);
          a[t] = racc.f32(static_cast<uint32_t>((pp * D + d) * sizeof(float)));
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          if (p0 + t < nparts) {
            const float f = fast_exp2(pm[p0 + t] - mx);
            num += f * a[t];
            den += f * pl[p0 + t];
          }
        }
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

template <int D, int BS>
void launch_stream_k(const DecodeLaunch& a, dim3 grid, hipStream_t stream) {
  const dim3 block(kStreamWaves * 64);
  if (a.prm.stream_kv != 0)
    decode_stream<D, BS, true><<<grid, block, 0, stream>>>(a.q, a.k_cache, a.v_cache,
                                                           a.block_tables, a.seq_lens, a.prm);
  else
    decode_stream<D, BS, false><<<grid, block, 0, stream>>>(a.q, a.k_cache, a.v_cache,
                                                            a.block_tables, a.seq_lens, a.prm);
}

template <int D>
hipError_t launch_stream_bs(const DecodeLaunch& a, dim3 grid, hipStream_t stream) {
  switch (a.prm.block_size) {
    case 8: launch_stream_k<D, 8>(a, grid, stream); break;
    case 16: launch_stream_k<D, 16>(a, grid, stream); break;
    default: launch_stream_k<D, 32>(a, grid, stream); break;
  }
  return hipGetLastError();
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

bool stream_shape_supported(int head_dim, int block_size, int group, int num_seqs) {
  return (head_dim == 64 || head_dim == 128) &&
         (block_size == 8 || block_size == 16 || block_size == 32) && group >= 1 &&
         group <= 16 && num_seqs <= kStreamMaxSeqs;
}

int stream_waves_per_group() { return kStreamWaves; }

bool generic_shape_supported(int head_dim, int block_size, int group) {
  return head_dim >= 1 && head_dim <= 256 && block_size >= 1 && group >= 1;
}

hipError_t launch_decode_mfma(const DecodeLaunch& a, int waves, hipStream_t stream) {
  const dim3 grid(a.prm.num_partitions, a.prm.num_kv_heads, a.num_seqs);
  return (a.prm.head_dim == 64) ? launch_mfma_bs<64>(a, waves, grid, stream)
                                : launch_mfma_bs<128>(a, waves, grid, stream);
}

hipError_t launch_decode_stream(const DecodeLaunch& a, int num_waves, hipStream_t stream) {
  const dim3 grid(num_waves / kStreamWaves);
  return (a.prm.head_dim == 64) ? launch_stream_bs<64>(a, grid, stream)
                                : launch_stream_bs<128>(a, grid, stream);
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
