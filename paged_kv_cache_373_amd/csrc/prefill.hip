// prefill.hip - paged prefill (causal multi-query) attention for gfx950.
//
// Sources (by title and section):
//   [PU] Fanyi Pu, "Infra: PagedAttention":
//        section "KV Cache 为什么会浪费显存": prefill processes the prompt and
//        builds the cache; in causal attention a token attends to the tokens
//        before it, whose K,V the cache keeps.
//        section "Continuous Batching": paging and FlashAttention both keep the
//        dense attention semantics; the attention reads the paged layout.
//        section "按 Block 分配": position t lives in logical block t / B at
//        offset t % B, found through the block table.
//
// The new tokens of sequence b are the last q_len_b of its T_b cached tokens
// (their K,V already written, e.g. by reshape_and_cache); new token i sits at
// position ctx_b + i, ctx_b = T_b - q_len_b, and attends positions 0 .. its own.
//
// Work: a wavefront folds tiles of 16 query rows of one (sequence, KV head)
// - row R = i G + g is new token i's query head g of the KV head - over the
// 32-token chunks up to their last position, with the chunk step of the
// decode kernels (scores and P.V on the matrix cores, online softmax) plus a
// per-row causal limit.  It takes three neighbouring tiles at a time at
// head_dim 64 (one at 128, whose operands take twice the registers): each
// chunk loaded serves all of them, and their steps interleave.  The tiles of a (sequence, KV head)
// run latest first and, in batches of up to 64, the sequences longest first,
// so the longest causal ranges start first; neighbouring workgroups take
// neighbouring tiles, which read the same chunks.  A workgroup has two
// wavefronts: the items nearly as long as the batch's longest are split
// between them (two halves of the chunks, merged in LDS); the others are
// folded by one wavefront while the other leaves.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "chunk.h"
#include "internal.h"

namespace pkv {
namespace {

// Wavefronts per workgroup: two, for one item.  An item whose chunk count is
// within kSplitNum / kSplitDen of the batch's longest sequence's (and at
// least kSplitMin) is split: the first wavefront folds its first half of
// the chunks, the second the rest, and the two states are merged in LDS.
// Every other item is folded by the first wavefront alone while the second
// leaves at once, so its slot goes to the next workgroup.  The longest items
// set the launch's time (on the chunked Llama step the longest wavefronts run
// as long as the launch), and splitting them shortens that chain.
constexpr int kNW = 2;
constexpr int kSplitNum = 4, kSplitDen = 5, kSplitMin = 16;
// The second wavefront's running maxima start at this finite value rather
// than -inf: a row that sees none of its half's chunks keeps exp2(-inf) = 0
// for its masked scores (with -inf a masked score would give NaN).
constexpr float kEmptyMax = -1.0e30f;

// 16-row tiles a wavefront takes at a time: three at head_dim 64 (measured
// against one, two and four on the chunked Llama step: 100 us against 180,
// 113 and 111), one at 128, whose operands and states take twice the
// registers.
constexpr int prefill_tiles_per_wave(int head_dim) { return head_dim <= 64 ? 3 : 1; }

// One chunk folded into the states of TPW tiles at once: the arithmetic of
// Mfma<D, BS>::step for each tile, regrouped by phase - every tile's QK^T
// products, then every tile's masks and per-lane maxima, one uniform test for
// a rescale in any tile (rare: the maximum moves past the margin; only then
// are the row maxima formed across lanes), then every
// tile's exponentials and P.V products.  Each phase is one straight run of
// independent instructions over the tiles, which the compiler interleaves;
// per tile the operations and their order are the step's, so the results are
// the same bits (the rescale test, made on each lane's maximum rather than
// its row's, picks the same chunks unless a row holds a NaN score, whose
// output is NaN either way).  With kCausal, lim[t] is how many of the chunk's tokens the
// lane's row of tile t may see.
template <int D, int BS, int TPW, bool kCausal>
__device__ __forceinline__ void step_tiles(const bf16x8_t (&qop)[TPW][D / 32],
                                           typename Mfma<D, BS>::Regs& x, int valid, float sl,
                                           int c, typename Mfma<D, BS>::State (&st)[TPW],
                                           const int (&lim)[TPW]) {
  constexpr int HS = D / 32;
  constexpr int NT = D / 16;
  f32x4_t s0[TPW], s1[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    s0[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    s1[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int hs = 0; hs < HS; ++hs) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      s0[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.k[0][hs], qop[t][hs], s0[t], 0, 0, 0);
      s1[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.k[1][hs], qop[t][hs], s1[t], 0, 0, 0);
    }
  }
  // The masks, maxima and exponentials run at raised wave priority: the
  // other wavefront on the SIMD, which is most likely in its matrix-core
  // products, yields issue slots to this one's vector work, and the two
  // phases overlap more often (about 4 % on the chunked Llama step).
  __builtin_amdgcn_s_setprio(1);
  const bool tail = valid < 32;  // wave-uniform
  const int lv = valid - 8 * c;  // tokens of this lane group still in range
  float xs[TPW][8];
  float cm[TPW];
  bool need = false;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xs[t][i] = s0[t][i];
      xs[t][4 + i] = s1[t][i];
    }
    if constexpr (kCausal) {
      const int lvc = min(valid, lim[t]) - 8 * c;
#pragma unroll
      for (int e = 0; e < 8; ++e) xs[t][e] = (e < lvc) ? xs[t][e] : -INFINITY;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) xs[t][e] = (!tail || e < lv) ? xs[t][e] : -INFINITY;
    }
    cm[t] = maxnan(maxnan(xs[t][0], xs[t][1], xs[t][2]), maxnan(xs[t][3], xs[t][4], xs[t][5]),
                   maxnan(xs[t][6], xs[t][7]));
    // a lane tests its own eight scores against its row's running maximum;
    // the maximum over the row's four lane groups is formed only for a rescale
    need = need || cm[t] * sl > st[t].m2 + kRescaleThreshold;
  }
  if (__ballot(need) != 0) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      if (__ballot(cm[t] * sl > st[t].m2 + kRescaleThreshold) != 0) {
        const float mn = fmaxf(st[t].m2, max_over_rows(cm[t]) * sl);
        const float alpha = fast_exp2(st[t].m2 - mn);  // 0 on the first chunk (m2 = -inf)
        st[t].m2 = mn;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = __shfl(alpha, 4 * c + i);  // factor of row 4 c + i
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) st[t].acc[nt][i] *= a;
          st[t].lsum[i] *= a;
        }
      }
    }
  }
  bf16x8_t pa[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      pa[t][e] = static_cast<__bf16>(fast_exp2(fmaf(xs[t][e], sl, -st[t].m2)));
  if (tail) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int e = 0; e < 8; ++e) x.v[nt][e] = (e < lv) ? x.v[nt][e] : static_cast<__bf16>(0.f);
  }
  __builtin_amdgcn_s_setprio(0);
  const bf16x8_t ones = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      st[t].acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[t], x.v[nt], st[t].acc[nt], 0, 0, 0);
#pragma unroll
  for (int t = 0; t < TPW; ++t)
    st[t].lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[t], ones, st[t].lsum, 0, 0, 0);
}

template <int D, int BS>
__global__ void __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 2 : 1)))
    prefill_mfma(const PrefillLaunch a) {
  using M = Mfma<D, BS>;
  using Regs = typename M::Regs;
  constexpr int NB = M::NB;
  constexpr int HS = M::HS;
  constexpr int NT = M::NT;
  constexpr int DEPTH = kDepth;
  static_assert(DEPTH >= 1 && DEPTH <= 3, "ring depth");
  constexpr int kBatchChunks = 64 / NB;  // chunks whose blocks one batch of lane loads covers
  constexpr int TPW = prefill_tiles_per_wave(D);

  // XCD-aware placement: consecutive workgroups go to the eight XCDs in turn,
  // and each XCD has an L2 of its own.  Workgroup L serves pair
  // p = 8 (L / 8 / W) + L % 8 and its item block (L / 8) % W, so every
  // workgroup of a pair runs on the same XCD and the pair's K/V, which all of
  // its items read, is fetched into that XCD's L2 only.  Pair p is (the
  // sequence of rank p / Hkv, KV head p % Hkv).
  const int W = a.wg_per_pair;
  const int L = blockIdx.x;
  const int t8 = L >> 3;
  const int pair = 8 * (t8 / W) + (L & 7);
  if (pair >= a.num_seqs * a.num_kv_heads) return;
  const int br = pair / a.num_kv_heads;
  const int h = pair - br * a.num_kv_heads;
  // Longest sequences first: for up to 64 sequences, rank r is the r-th
  // longest (ties by index), each wavefront ranking the lengths in its lanes,
  // so the longest causal ranges start in the first round of workgroups and
  // the short sequences' items fill the slots that free up (70.9-72.5 against
  // 74.5-75.2 us on the chunked Llama step, whose batch order puts a long
  // sequence late).  Larger batches keep their order.
  int b = br;
  int t_top = 0;  // the longest sequence's length (0: not ranked, no item is split)
  if (a.num_seqs <= 64) {
    const int ln = threadIdx.x & 63;
    const int Tl = ln < a.num_seqs ? a.seq_lens[ln] : -1;
    int rank = 0;
    for (int i = 0; i < a.num_seqs; ++i) {
      const int Ti = __builtin_amdgcn_readlane(Tl, i);
      rank += (Ti > Tl || (Ti == Tl && i < ln)) ? 1 : 0;
    }
    const unsigned long long hit = __ballot(ln < a.num_seqs && rank == br);
    b = hit != 0 ? static_cast<int>(__builtin_ctzll(hit)) : br;
    const unsigned long long top = __ballot(ln < a.num_seqs && rank == 0);
    t_top = top != 0 ? __builtin_amdgcn_readlane(Tl, static_cast<int>(__builtin_ctzll(top))) : 0;
  }
  const int wblk = t8 - (t8 / W) * W;  // this workgroup's block of items within the pair
  const int lane = threadIdx.x & 63;
  const int c = lane >> 4;
  const int r = lane & 15;
  const int G = a.group;
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;

  // The sequence's rows in q/out and its lengths.  A row range outside
  // [0, num_tokens) is skipped; q_len > T (or T beyond the table) makes the
  // sequence's rows NaN.
  const int q0 = a.cu_q_lens[b];
  const int q1 = a.cu_q_lens[b + 1];
  if (q0 < 0 || q1 < q0 || q1 > a.num_tokens) return;
  const int nq = q1 - q0;
  const int T = a.seq_lens[b];
  const int ntiles = (nq * G + 15) / 16;
  // This wavefront's index in the workgroup.  It is kept per lane: made
  // uniform (readfirstlane), it let the compiler restructure the item loop
  // and spill 25 registers from the chunk loop at two wavefronts per SIMD.
  const int part = threadIdx.x >> 6;
  const int wave0 = wblk * kNW + part;
  const int nwaves = W * kNW;
  if (nq > T || T > a.max_blocks_per_seq * BS) {
    for (int e = wave0 * 64 + lane; e < nq * G * D; e += nwaves * 64) {
      const int row = e / (G * D);
      const int rem = e - row * G * D;
      store_out(a.out, (static_cast<size_t>(q0 + row) * Hq + h * G) * D + rem, NAN, a.out_f32);
    }
    return;
  }
  const int ctx = T - nq;
  const float sl = a.scale_log2;
  const size_t blk_stride = static_cast<size_t>(Hkv) * M::kTile;
  const size_t head_off = static_cast<size_t>(h) * M::kTile;
  const int32_t* row_bt = a.block_tables + static_cast<size_t>(b) * a.max_blocks_per_seq;
  const typename M::Lane ln(c, r);
  struct Slot {
    Regs x;
  };

  // A workgroup takes TPW neighbouring tiles at a time (an item): each chunk
  // a wavefront loads serves all of their rows, and their steps interleave.
  // The second wavefront's states of a split item, for the merge:
  // [TPW][4 NT accumulators + 4 sums + 1 maximum][64 lanes].
  constexpr int kStWords = 4 * NT + 5;
  __shared__ float s_part[TPW * kStWords * 64];
  const int nk_top = (t_top + 31) / 32;
  const int nitems = (ntiles + TPW - 1) / TPW;
  for (int j = wblk; j < nitems; j += W) {
    const int tile0 = (nitems - 1 - j) * TPW;  // latest tiles first
    const int last_i = min(nq - 1, ((tile0 + TPW) * 16 - 1) / G);
    const int pos_max = ctx + last_i;      // the item's last position
    const int pos_min = ctx + (tile0 * 16) / G;  // and its first (every row sees up to here)
    const int nk = pos_max / 32 + 1;       // chunks up to it
    const bool split = nk >= kSplitMin && kSplitDen * nk >= kSplitNum * nk_top && nk_top > 0;
    if (!split && part != 0) continue;
    // This lane's row (r) of tile t: new token i, head g; past nq the row is
    // a zero query whose output is dropped.
    int pos[TPW];
    bf16x8_t qop[TPW][HS];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int R = (tile0 + t) * 16 + r;
      const int i = R / G;
      const int g = R - i * G;
      const bool live = i < nq;
      pos[t] = live ? ctx + i : -1;
      const uint16_t* qrow =
          a.q + (static_cast<size_t>(q0 + (live ? i : 0)) * Hq + h * G + (live ? g : 0)) * D + 8 * c;
#pragma unroll
      for (int hs = 0; hs < HS; ++hs) qop[t][hs] = live ? load_bf16x8(qrow + 32 * hs) : bf16x8_t{};
    }
    const int last_blk = (min(T, 32 * nk) - 1) / BS;
    // a dead row (past nq) sees every chunk the item reads, so its state stays finite
#pragma unroll
    for (int t = 0; t < TPW; ++t) pos[t] = pos[t] < 0 ? pos_max : pos[t];
    typename M::State st[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      st[t].reset();
      if (part != 0) st[t].m2 = kEmptyMax;
    }
    // This wavefront's chunks: all of them, or its half of a split item.
    const int klo = (split && part != 0) ? nk / 2 : 0;
    const int khi = (split && part == 0) ? nk / 2 : nk;

    for (int k0 = klo; k0 < khi; k0 += kBatchChunks) {
      // the batch's blocks, one per lane (clamped to the last one needed)
      const int first_blk = k0 * NB;
      const int bid = row_bt[min(first_blk + lane, last_blk)];
      const int nkb = min(kBatchChunks, khi - k0);
      auto issue = [&](int kb, Slot& sl8) {
        size_t base[NB];
#pragma unroll
        for (int jb = 0; jb < NB; ++jb)
          base[jb] = static_cast<size_t>(__builtin_amdgcn_readlane(
                         bid, min(kb * NB + jb, last_blk - first_blk))) *
                         blk_stride +
                     head_off;
        M::load(a.k_cache, a.v_cache, base, ln, sl8.x);
      };
      auto consume = [&](int kb, Slot& sl8) {
        const int t0 = 32 * (k0 + kb);
        if (pos_min - t0 >= 31) {
          // every row of the item sees the whole chunk: no mask to apply
          step_tiles<D, BS, TPW, false>(qop, sl8.x, 32, sl, c, st, pos);
        } else {
          const int valid = min(32, T - t0);
          int lim[TPW];
#pragma unroll
          for (int t = 0; t < TPW; ++t) lim[t] = pos[t] - t0 + 1;
          step_tiles<D, BS, TPW, true>(qop, sl8.x, valid, sl, c, st, lim);
        }
      };
      // every refill issues its loads (one past the batch re-reads its last
      // chunk, which is not folded again) so the wait counts stay exact
      Slot ring[DEPTH];
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) issue(min(s, nkb - 1), ring[s]);
      for (int kb = 0;;) {
        if (kb >= nkb) break;
        consume(kb, ring[0]);
        issue(min(kb + DEPTH, nkb - 1), ring[0]);
        ++kb;
        if constexpr (DEPTH > 1) {
          if (kb >= nkb) break;
          consume(kb, ring[1]);
          issue(min(kb + DEPTH, nkb - 1), ring[1]);
          ++kb;
        }
        if constexpr (DEPTH > 2) {
          if (kb >= nkb) break;
          consume(kb, ring[2]);
          issue(min(kb + DEPTH, nkb - 1), ring[2]);
          ++kb;
        }
      }
    }

    // A split item's two states: the second wavefront's through LDS into the
    // first's.  Lane (c, r) holds row 4 c + i's accumulator (features
    // 16 nt + r) and sum, and row r's maximum; both are taken to the larger
    // maximum of the two (every row sees chunk 0, so one of them is real).
    if (split) {
      if (part != 0) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          float* sp = s_part + t * kStWords * 64 + lane;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sp[(4 * nt + i) * 64] = st[t].acc[nt][i];
#pragma unroll
          for (int i = 0; i < 4; ++i) sp[(4 * NT + i) * 64] = st[t].lsum[i];
          sp[(4 * NT + 4) * 64] = st[t].m2;
        }
      }
      __syncthreads();
      if (part == 0) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          __builtin_amdgcn_sched_barrier(0);  // one tile's LDS reads at a time
          const float* sp = s_part + t * kStWords * 64 + lane;
          const float mb = sp[(4 * NT + 4) * 64];
          const float mn = fmaxf(st[t].m2, mb);
          const float fa = fast_exp2(st[t].m2 - mn);
          const float fb = fast_exp2(mb - mn);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float fai = __shfl(fa, 4 * c + i);  // factors of row 4 c + i
            const float fbi = __shfl(fb, 4 * c + i);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              st[t].acc[nt][i] = st[t].acc[nt][i] * fai + sp[(4 * nt + i) * 64] * fbi;
            st[t].lsum[i] = st[t].lsum[i] * fai + sp[(4 * NT + i) * 64] * fbi;
          }
        }
      }
      __syncthreads();  // (the next item reuses the LDS)
      if (part != 0) continue;
    }

    // Lane (c, r) holds row 4 c + e of each tile: its accumulator for
    // features 16 nt + r and its sum, whose quotient is the output.
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int Ro = (tile0 + t) * 16 + 4 * c + e;
        const int io = Ro / G;
        if (io < nq) {
          const int go = Ro - io * G;
          const float inv = 1.0f / st[t].lsum[e];
          const size_t orow = (static_cast<size_t>(q0 + io) * Hq + h * G + go) * D;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            store_out(a.out, orow + 16 * nt + r, st[t].acc[nt][e] * inv, a.out_f32);
        }
      }
    }
  }
}

template <int D>
hipError_t launch_d(const PrefillLaunch& a, dim3 grid, hipStream_t stream) {
  const dim3 block(kNW * 64);
  switch (a.block_size) {
    case 8: prefill_mfma<D, 8><<<grid, block, 0, stream>>>(a); break;
    case 16: prefill_mfma<D, 16><<<grid, block, 0, stream>>>(a); break;
    default: prefill_mfma<D, 32><<<grid, block, 0, stream>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace

bool prefill_shape_supported(int head_dim, int block_size, int group) {
  return (head_dim == 64 || head_dim == 128) &&
         (block_size == 8 || block_size == 16 || block_size == 32) && group >= 1 && group <= 16;
}

hipError_t launch_prefill(const PrefillLaunch& a, int max_q_len, hipStream_t stream) {
  // one workgroup per item (tiles of 16 rows, three per item at head_dim 64)
  // of the longest sequence's rows (a longer one is still covered: the
  // workgroups stride over the items)
  const int tiles = (max_q_len * a.group + 15) / 16;
  const int tpw = prefill_tiles_per_wave(a.head_dim);
  const int items = (tiles + tpw - 1) / tpw;
  PrefillLaunch la = a;
  la.wg_per_pair = items;  // one item per workgroup
  if (la.wg_per_pair < 1) la.wg_per_pair = 1;
  // eight workgroups (one per XCD) per group of eight (sequence, KV head)
  // pairs and item block; the ones past the last pair exit at once
  const int64_t pair_groups = (static_cast<int64_t>(a.num_seqs) * a.num_kv_heads + 7) / 8;
  const int64_t wgs = 8 * pair_groups * la.wg_per_pair;
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(wgs));
  return a.head_dim == 64 ? launch_d<64>(la, grid, stream) : launch_d<128>(la, grid, stream);
}

}  // namespace pkv
