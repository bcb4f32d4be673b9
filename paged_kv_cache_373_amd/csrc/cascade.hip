// cascade.hip - shared-prefix ("cascade") decode for gfx950 (CDNA4).
//
// Sources (by title and section):
//   [PU] Fanyi Pu, "Infra: PagedAttention":
//        section "共享前缀，分叉时 Copy-on-write": several samples of one prompt
//        point their block tables at the same physical blocks for the
//        prompt's KV; full prefix blocks stay shared after the fork.
//        section "按 Block 分配": softmax spans every token the query sees;
//        segment results merge by o = (Z1 o1 + Z2 o2) / (Z1 + Z2) after
//        rescaling to a common maximum, and segments need not coincide with
//        physical blocks.
//
// Each sequence's tokens are cut into two segments: its group's shared
// prefix and its own suffix (the tokens past the prefix).  The prefix segment
// of the members of a group is computed together: the group's query rows
// (row R = member * G + head) are cut into blocks of kCascadeRows = 16, one
// matrix-core tile, and a wavefront folds a prefix chunk for one row block.
// The row blocks of one (KV head, prefix segment) are consecutive items, so
// they run in one workgroup and a shared chunk comes from HBM once and from
// the caches for the other row blocks: a shared block is fetched once per
// group rather than once per member.  The segment results then merge by the
// rule above.
//
// Launch 1 (cascade_partials) folds items into partial states (max in base-2
// units, sum, unnormalised accumulator): a prefix item is up to
// kCascadePrefixChunks 32-token chunks of a group's prefix for one row
// block; a suffix item is up to kCascadeSuffixChunks chunks of one
// sequence's suffix for its G rows.
// Launch 2 (cascade_merge) merges, for each (sequence, KV head), its group's
// prefix items and its own suffix items in item order.  No result depends on
// the timing of the wavefronts.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "chunk.h"
#include "internal.h"

namespace pkv {
namespace {

constexpr int kNW = 4;  // wavefronts per workgroup in both launches
constexpr int kNTH = kNW * 64;
constexpr int kCascadeLdsBytes = 160 * 1024;  // the most a workgroup may ask for on gfx950

__device__ __forceinline__ int div_up(int a, int b) { return (a + b - 1) / b; }

// Ints of launch 1's LDS: item prefixes per group and sequence, each
// sequence's group and length, the group starts and prefix lengths, scan
// partials and the error flag.
__host__ __device__ constexpr int cascade_lds_ints(int S, int NG) {
  return (NG + 1) + (S + 1) + S + S + (NG + 1) + NG + kNW + 1;
}

// Exclusive prefix of count(0 .. n-1) into pre[0 .. n], by all NTH threads
// (count(i) is evaluated twice by the thread owning i and must not change in
// between); s_wsum holds NTH / 64 ints.  Ends with a barrier.
template <int NTH = kNTH, typename F>
__device__ void block_scan(int n, F count, int* pre, int* s_wsum, int tid) {
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int per = (n + NTH - 1) / NTH;  // thread tid owns [tid per, tid per + per)
  int mine = 0;
  for (int j = 0; j < per; ++j) {
    const int i = tid * per + j;
    if (i < n) mine += count(i);
  }
  int incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  int run = incl - mine;
  for (int ww = 0; ww < w; ++ww) run += s_wsum[ww];
  for (int j = 0; j < per; ++j) {
    const int i = tid * per + j;
    if (i < n) {
      pre[i] = run;
      run += count(i);
    }
  }
  if (tid == NTH - 1) pre[n] = run;
  __syncthreads();
}

// Items of group g's prefix and of sequence b's suffix (the launches agree on
// these through the same two functions).
__device__ __forceinline__ int prefix_segments(int L) {
  return div_up(div_up(L, 32), kCascadePrefixChunks);
}
__device__ __forceinline__ int suffix_segments(int suf) {
  return suf > 0 ? div_up(div_up(suf, 32), kCascadeSuffixChunks) : 0;
}
__device__ __forceinline__ int row_blocks(int members, int G) {
  return div_up(members * G, kCascadeRows);
}

template <int D, int BS>
__global__ void __launch_bounds__(kNTH) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 2 : 1)))
    cascade_partials(const CascadeLaunch a) {
  using M = Mfma<D, BS>;
  using Regs = typename M::Regs;
  constexpr int NB = M::NB;
  constexpr int HS = M::HS;
  constexpr int NT = M::NT;
  constexpr int kItemChunks = kCascadePrefixChunks;  // chunks of an item, all in flight
  static_assert(kCascadePrefixChunks == kCascadeSuffixChunks, "one ring for both kinds");

  const int S = a.num_seqs;
  const int NG = a.num_groups;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int G = a.group;
  extern __shared__ int lds[];
  int* s_gpre = lds;              // [NG + 1] items before group g's
  int* s_spre = s_gpre + NG + 1;  // [S + 1] suffix items before sequence b's
  int* s_gof = s_spre + S + 1;    // [S] group of sequence b
  int* s_len = s_gof + S;         // [S] seq_lens
  int* s_gs = s_len + S;          // [NG + 1] group_starts
  int* s_pl = s_gs + NG + 1;      // [NG] prefix_lens
  int* s_misc = s_pl + NG;        // [kNW] scan partials, [kNW] error flag

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int c = lane >> 4;
  const int r = lane & 15;

  // 1. Every sequence's group, and the checks of what lives in device memory:
  // the groups partition [0, S) into non-empty runs, prefixes are whole
  // blocks within the host's bound, no member is shorter than its group's
  // prefix or longer than the host's bound (so the items fit the workspace
  // the host sized from those bounds).  A violation makes every output row
  // NaN (launch 2).
  // the per-sequence and per-group arrays, all loads in flight at once
  for (int i = tid; i < S; i += kNTH) s_len[i] = a.seq_lens[i];
  for (int i = tid; i <= NG; i += kNTH) s_gs[i] = a.group_starts[i];
  for (int i = tid; i < NG; i += kNTH) s_pl[i] = a.prefix_lens[i];
  if (tid == 0) s_misc[kNW] = 0;
  __syncthreads();
  for (int g = tid; g < NG; g += kNTH) {
    const int b0 = s_gs[g];
    const int b1 = s_gs[g + 1];
    const int L = s_pl[g];
    const bool bad = b0 < 0 || b1 <= b0 || b1 > S || (g == 0 && b0 != 0) ||
                     (g == NG - 1 && b1 != S) || L < 0 || L % BS != 0 ||
                     L > a.max_prefix_len;
    if (bad) {
      s_misc[kNW] = 1;
    } else {
      for (int b = b0; b < b1; ++b) s_gof[b] = g;
    }
  }
  __syncthreads();
  const bool groups_ok = s_misc[kNW] == 0;
  if (groups_ok) {
    block_scan(
        NG,
        [&](int g) {
          return Hkv * row_blocks(s_gs[g + 1] - s_gs[g], G) * prefix_segments(s_pl[g]);
        },
        s_gpre, s_misc, tid);
    block_scan(
        S,
        [&](int b) {
          const int T = s_len[b];
          const int suf = T - s_pl[s_gof[b]];
          if (suf < 0 || T > a.max_seq_len) s_misc[kNW] = 1;
          return Hkv * suffix_segments(suf);
        },
        s_spre, s_misc, tid);
  }
  const bool ok = groups_ok && s_misc[kNW] == 0 && s_gpre[NG] <= a.max_pre_items &&
                  s_spre[S] <= a.max_suf_items;
  if (blockIdx.x == 0) {  // what launch 2 reads: the status, each sequence's merge descriptor
    if (tid == 0) a.tables[0] = ok ? 0 : 1;
    if (ok) {
      for (int b = tid; b < S; b += kNTH) {
        const int g = s_gof[b];
        const int L = s_pl[g];
        int* d = a.tables + kCascadeTableHead + 8 * b;
        d[0] = s_gpre[g];                                  // the group's first prefix item
        d[1] = row_blocks(s_gs[g + 1] - s_gs[g], G);   // its row blocks
        d[2] = prefix_segments(L);                         // prefix items per (head, row block)
        d[3] = b - s_gs[g];                                // member index
        d[4] = s_spre[b];                                  // the sequence's first suffix item
        d[5] = suffix_segments(s_len[b] - L);              // suffix items per head
        d[6] = 0;
        d[7] = 0;
      }
    }
  }
  if (!ok) return;

  // 2. Items, one per wavefront at a time.
  const int npre = s_gpre[NG];
  const int total = npre + s_spre[S];
  const int wave = blockIdx.x * kNW + (tid >> 6);
  const int nwaves = gridDim.x * kNW;
  const float sl = a.scale_log2;
  const size_t blk_stride = static_cast<size_t>(Hkv) * M::kTile;
  const typename M::Lane ln(c, r);
  struct Slot {
    Regs x;
  };

  for (int item = wave; item < total; item += nwaves) {
    // the item's rows, KV head and tokens
    int seq0, R0, nrows, trow, h, tok0, tok1;
    float* acc_out;
    float* ml_out;
    if (item < npre) {
      int lo = 0, hi = NG;  // the group: largest g with s_gpre[g] <= item
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_gpre[mid] <= item) lo = mid; else hi = mid;
      }
      const int g = lo;
      const int b0 = s_gs[g];
      const int F = s_gs[g + 1] - b0;
      const int L = s_pl[g];
      const int nseg = prefix_segments(L);
      const int rb_n = row_blocks(F, G);
      // item = ((h nseg) + seg) rb_n + rb within the group: the row blocks
      // of one chunk range are neighbours
      const int rem = item - s_gpre[g];
      const int hs_ = rem / rb_n;
      const int rb = rem - hs_ * rb_n;
      h = hs_ / nseg;
      const int seg = hs_ - h * nseg;
      seq0 = b0;
      R0 = rb * kCascadeRows;
      nrows = min(kCascadeRows, F * G - R0);
      trow = b0;  // every member's table holds the shared blocks; the first one's is read
      tok0 = seg * kCascadePrefixChunks * 32;
      tok1 = min(tok0 + kCascadePrefixChunks * 32, L);
      acc_out = a.pre_acc + static_cast<size_t>(item) * kCascadeRows * D;
      ml_out = a.pre_ml + static_cast<size_t>(item) * kCascadeRows * 2;
    } else {
      const int j = item - npre;
      int lo = 0, hi = S;  // the sequence: largest b with s_spre[b] <= j
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_spre[mid] <= j) lo = mid; else hi = mid;
      }
      const int b = lo;
      const int L = s_pl[s_gof[b]];
      const int T = s_len[b];
      const int nseg = suffix_segments(T - L);
      const int rem = j - s_spre[b];
      h = rem / nseg;
      const int seg = rem - h * nseg;
      seq0 = b;
      R0 = 0;
      nrows = G;
      trow = b;
      tok0 = L + seg * kCascadeSuffixChunks * 32;
      tok1 = min(tok0 + kCascadeSuffixChunks * 32, T);
      acc_out = a.suf_acc + static_cast<size_t>(j) * G * D;
      ml_out = a.suf_ml + static_cast<size_t>(j) * G * 2;
    }
    seq0 = __builtin_amdgcn_readfirstlane(seq0);
    R0 = __builtin_amdgcn_readfirstlane(R0);
    nrows = __builtin_amdgcn_readfirstlane(nrows);
    trow = __builtin_amdgcn_readfirstlane(trow);
    h = __builtin_amdgcn_readfirstlane(h);
    tok0 = __builtin_amdgcn_readfirstlane(tok0);
    tok1 = __builtin_amdgcn_readfirstlane(tok1);
    const int nk = div_up(tok1 - tok0, 32);

    // The item's physical blocks, one per lane (at most 4 chunks of at most
    // 4 blocks; tok0 is a multiple of BS, so chunk k starts at block
    // first_blk + k NB), loaded with the query rows below in one round trip,
    // so no table load waits in the ring.
    const int32_t* row = a.block_tables + static_cast<size_t>(trow) * a.max_blocks_per_seq;
    const int first_blk = tok0 / BS;
    const int nblk = (tok1 - 1) / BS - first_blk + 1;
    const int bid = row[first_blk + min(lane, nblk - 1)];

    // Query rows as the QK^T B operand: lane (c, r) holds dims
    // [32 hs + 8 c, +8) of row R0 + r (member R / G, head R % G of KV head h),
    // zero past the item's rows.
    bf16x8_t qop[HS];
    {
      const int R = R0 + r;
      const bool live = r < nrows;
      const int f = R / G;
      const int gh = R - f * G;
      const uint16_t* qrow =
          a.q + (static_cast<size_t>(live ? seq0 + f : seq0) * Hq + h * G + (live ? gh : 0)) * D +
          8 * c;
#pragma unroll
      for (int hs = 0; hs < HS; ++hs) qop[hs] = live ? load_bf16x8(qrow + 32 * hs) : bf16x8_t{};
    }

    const size_t head_off = static_cast<size_t>(h) * M::kTile;
    // Chunk k of the item (k < nk): its blocks, clamped to the item's last one.
    auto issue = [&](int k, Slot& sl8) {
      size_t base[NB];
#pragma unroll
      for (int jb = 0; jb < NB; ++jb)
        base[jb] = static_cast<size_t>(
                       __builtin_amdgcn_readlane(bid, min(k * NB + jb, nblk - 1))) *
                       blk_stride +
                   head_off;
      M::load(a.k_cache, a.v_cache, base, ln, sl8.x);
    };
    typename M::State st;
    st.reset();
    auto consume = [&](int k, Slot& sl8) {
      M::step(qop, sl8.x, min(32, tok1 - (tok0 + 32 * k)), sl, c, st);
    };

    // All of the item's chunks are loaded at once (at most kItemChunks; the
    // loads of the slots past nk re-read its last chunk, which is not folded
    // again, so every slot issues its loads and the wait counts stay exact),
    // then folded in order.
    Slot ring[kItemChunks];
#pragma unroll
    for (int k = 0; k < kItemChunks; ++k) issue(min(k, nk - 1), ring[k]);
    __builtin_amdgcn_sched_barrier(0);  // every load goes out before the first fold
#pragma unroll
    for (int k = 0; k < kItemChunks; ++k) {
      if (k >= nk) break;
      consume(k, ring[k]);
    }

    // 3. The item's partial states: lane (c, r) holds row 4 c + i's
    // accumulator for features 16 nt + r and its sum, and row r's maximum.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = 4 * c + i;
      if (rl < nrows) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc_out[rl * D + 16 * nt + r] = st.acc[nt][i];
        if (r == 0) ml_out[rl * 2 + 1] = st.lsum[i];
      }
    }
    if (c == 0 && r < nrows) ml_out[r * 2] = st.m2;
  }
}

// Launch 2: wavefront u = b Hkv + h merges the partial states of the G rows
// of (sequence b, KV head h) - its group's prefix items, then its own suffix
// items, in item order - by the rescaled segment rule, and writes them out.
template <int D>
__global__ void __launch_bounds__(kNTH) cascade_merge(const CascadeLaunch a) {
  constexpr int E4 = D / 4;  // float4s per row
  const int S = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int G = a.group;
  const int lane = threadIdx.x & 63;
  const int64_t u = static_cast<int64_t>(blockIdx.x) * kNW + (threadIdx.x >> 6);
  if (u >= static_cast<int64_t>(S) * Hkv) return;
  const int b = static_cast<int>(u / Hkv);
  const int h = static_cast<int>(u - static_cast<int64_t>(b) * Hkv);
  const size_t row0 = static_cast<size_t>(b) * Hq + static_cast<size_t>(h) * G;
  // the status and the descriptor in one round trip (the descriptor is
  // only used when the status says launch 1 wrote it)
  const int status = a.tables[0];
  const int* desc = a.tables + kCascadeTableHead + 8 * b;
  const int gpre_g = desc[0];
  const int rb_n = desc[1];
  const int nsp = desc[2];
  const int f = desc[3];
  const int spre_b = desc[4];
  const int nss = desc[5];
  if (status != 0) {  // a device-side precondition failed
    for (int e = lane; e < G * D; e += 64) store_out(a.out, row0 * D + e, NAN, a.out_f32);
    return;
  }
  for (int e = lane; e < G * E4; e += 64) {
    const int gh = e / E4;
    const int d4 = e - gh * E4;
    const int R = f * G + gh;
    const int rb = R / kCascadeRows;
    const int rl = R - rb * kCascadeRows;
    // piece j < nsp: prefix item j of row block rb; then the suffix items
    auto piece = [&](int j, const float*& ml, const float*& acc) {
      if (j < nsp) {
        const size_t it = static_cast<size_t>(gpre_g) + (static_cast<size_t>(h) * nsp + j) * rb_n + rb;
        ml = a.pre_ml + (it * kCascadeRows + rl) * 2;
        acc = a.pre_acc + (it * kCascadeRows + rl) * D + 4 * d4;
      } else {
        const size_t it = static_cast<size_t>(spre_b) + static_cast<size_t>(h) * nss + (j - nsp);
        ml = a.suf_ml + (it * G + gh) * 2;
        acc = a.suf_acc + (it * G + gh) * D + 4 * d4;
      }
    };
    const int np = nsp + nss;
    float mx = -INFINITY, den = 0.f;
    f32x4_t num = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < np; j0 += 8) {  // eight pieces' loads in flight at a time
      float pm[8], pl[8];
      f32x4_t pa[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float* ml;
        const float* acc;
        piece(min(j0 + t, np - 1), ml, acc);
        pm[t] = ml[0];
        pl[t] = ml[1];
        pa[t] = *reinterpret_cast<const f32x4_t*>(acc);
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (j0 + t < np) {
          const float mn = fmaxf(mx, pm[t]);
          const float fo = fast_exp2(mx - mn);  // 0 for the first piece
          const float fj = fast_exp2(pm[t] - mn);
          den = den * fo + pl[t] * fj;
          num = num * fo + pa[t] * fj;
          mx = mn;
        }
      }
    }
    // no pieces: an empty sequence, whose row is zero
    const f32x4_t o = den > 0.f ? num * (1.0f / den) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) store_out(a.out, (row0 + gh) * D + 4 * d4 + t, o[t], a.out_f32);
  }
}

template <int D, int BS>
hipError_t launch_bs(const CascadeLaunch& a, hipStream_t stream) {
  const size_t lds = static_cast<size_t>(cascade_lds_ints(a.num_seqs, a.num_groups)) * 4;
  // more than the default dynamic allowance when S is large (once per process)
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&cascade_partials<D, BS>),
      hipFuncAttributeMaxDynamicSharedMemorySize, kCascadeLdsBytes);
  if (attr != hipSuccess) return attr;
  cascade_partials<D, BS><<<dim3(a.waves / kNW), dim3(kNTH), lds, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t units = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads;
  cascade_merge<D><<<dim3(static_cast<unsigned>((units + kNW - 1) / kNW)), dim3(kNTH), 0, stream>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// One-launch form.  A task is (group g, KV head h, member block): up to
// members_per_task consecutive members of g, whose query rows R = m G + gh
// (m the member within the block) fill at most one 16-row matrix-core tile.
// The task's chunks are the group's prefix chunks (every row of the task
// attends them) followed by each member's suffix chunks (only that member's
// rows attend them; the other rows' scores are masked to -inf), 32 tokens
// each.  One workgroup runs a task: wavefront w folds chunks w, w + NW, ...
// into one running state of the tile's rows, then the NW states are merged in
// LDS in wavefront order and each row is written out.  Nothing crosses
// workgroups, so there is no device-scope hand-off; the static split of the
// chunks and the fixed merge order make the result bit-reproducible.  The
// tasks of one (g, h) are neighbours in task order and run on one XCD, so the
// group's prefix blocks come from that XCD's L2 after the first read.
//
// A row's running maximum starts at kEmptyMax (finite) rather than -inf, so a
// row that has attended nothing yet stays at exp2(-inf) = 0 for masked scores
// and at a rescale factor of 1, without a select in the fold.
constexpr float kEmptyMax = -1.0e30f;
// Wavefronts of a task's workgroup: one per SIMD (on prefix_cow, 15.2 us
// against 16.4 us with two per SIMD: each wavefront then folds twice the
// chunks, and fewer states are merged at the end).
constexpr int cascade_wg_waves(int head_dim) { return head_dim <= 64 ? 4 : 4; }

template <int D, int BS, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 2 : 1)))
    cascade_wg(const CascadeLaunch a, const CascadeWgLayout lay) {
  using M = Mfma<D, BS>;
  using Regs = typename M::Regs;
  constexpr int NB = M::NB;
  constexpr int HS = M::HS;
  constexpr int NT = M::NT;
  constexpr int NTH = NW * 64;
  constexpr int E4 = D / 4;
  constexpr int kRec = 2 + NB;  // member (-1: prefix), valid tokens, physical blocks

  const int S = a.num_seqs;
  const int NG = a.num_groups;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int G = a.group;
  const int MB = a.max_blocks_per_seq;
  const int mpt = a.members_per_task;
  extern __shared__ __align__(16) int lds[];
  int* s_len = lds + lay.off_len;    // [S] seq_lens
  int* s_gs = lds + lay.off_gs;      // [NG + 1] group_starts
  int* s_pl = lds + lay.off_pl;      // [NG] prefix_lens
  int* s_tpre = lds + lay.off_tpre;  // [NG + 1] tasks before group g's
  int* s_misc = lds + lay.off_misc;  // [NW] scan partials, [NW] error flag
  int* s_rec = lds + lay.off_rec;    // [capacity][kRec] the task's chunk records
  float* s_acc = reinterpret_cast<float*>(lds + lay.off_acc);  // [NW][16][D]
  float* s_ml = reinterpret_cast<float*>(lds + lay.off_ml);    // [NW][16][max, sum]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int c = lane >> 4;
  const int r = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // 1. The lengths and groups, and the checks of what lives in device memory
  // (as for the item form: the groups partition [0, S) into non-empty runs,
  // prefixes are whole blocks within the host's bound, no member is shorter
  // than its group's prefix or longer than the host's bound).  Every
  // workgroup reaches the same verdict; a violation makes every row NaN.
  if (S <= NTH && NG < 64) {
    // A batch of at most NTH sequences in at most 63 groups: every wavefront
    // loads the groups' starts, ends and prefixes into its lanes (lane g:
    // group g) and thread b the length of sequence b, all in one round trip;
    // the checks are ballots and the task prefix a scalar loop, with one
    // barrier.  Each wavefront flags a violation in a word of its own.
    const int ls = a.seq_lens[min(tid, S - 1)];
    const int gs0 = a.group_starts[min(lane, NG)];
    const int gs1 = a.group_starts[min(lane + 1, NG)];
    const int pl = a.prefix_lens[min(lane, NG - 1)];
    // group `lane`: a run of members starting where the previous one ends,
    // its prefix whole blocks within the host's bound
    bool bad = false;
    if (lane < NG)
      bad = (gs0 < 0) | (gs1 <= gs0) | (gs1 > S) | ((lane == 0) & (gs0 != 0)) |
            ((lane == NG - 1) & (gs1 != S)) | (pl < 0) | (pl % BS != 0) |
            (pl > a.max_prefix_len);
    // sequence tid: its group (the groups after the first whose start is
    // <= tid), no shorter than that group's prefix, within the host's bound
    int grp = 0;
    for (int g = 1; g < NG; ++g) grp += __builtin_amdgcn_readlane(gs0, g) <= tid ? 1 : 0;
    const int plb = __shfl(pl, grp);
    if (tid < S) {
      s_len[tid] = ls;
      bad = bad | (ls < plb) | (ls > a.max_seq_len);
    }
    const int F = gs1 - gs0;
    const int cnt = (lane < NG && F > 0 && F <= S) ? Hkv * div_up(F, mpt) : 0;
    if (w == 0) {
      if (lane <= NG) s_gs[lane] = gs0;
      if (lane < NG) s_pl[lane] = pl;
      // tasks before group g (lane g), Hkv ceil(F_g / mpt) per group
      int run = 0, mine = 0;
      for (int g = 0; g < NG; ++g) {
        mine = lane == g ? run : mine;
        run += __builtin_amdgcn_readlane(cnt, g);
      }
      if (lane < NG) s_tpre[lane] = mine;
      if (lane == 0) s_tpre[NG] = run;
    }
    const bool any_bad = __ballot(bad) != 0;  // (every lane takes part)
    if (lane == 0) s_misc[NW + w] = any_bad ? 1 : 0;
    __syncthreads();
  } else {
    // The three arrays' first NTH entries are loaded together (clamped
    // indices, no branch around the loads), so the set-up waits for one round
    // trip rather than three.
    {
      const int ls = a.seq_lens[min(tid, S - 1)];
      const int lg = a.group_starts[min(tid, NG)];
      const int lp = a.prefix_lens[min(tid, NG - 1)];
      if (tid < S) s_len[tid] = ls;
      if (tid <= NG) s_gs[tid] = lg;
      if (tid < NG) s_pl[tid] = lp;
      for (int i = tid + NTH; i < S; i += NTH) s_len[i] = a.seq_lens[i];
      for (int i = tid + NTH; i <= NG; i += NTH) s_gs[i] = a.group_starts[i];
      for (int i = tid + NTH; i < NG; i += NTH) s_pl[i] = a.prefix_lens[i];
    }
    if (tid < NW) s_misc[NW + tid] = 0;
    __syncthreads();
    // Group g (thread g): a run of members starting where the previous one
    // ends, its prefix whole blocks within the host's bound.
    for (int g = tid; g < NG; g += NTH) {
      const int b0 = s_gs[g];
      const int b1 = s_gs[g + 1];
      const int L = s_pl[g];
      const bool bad = b0 < 0 || b1 <= b0 || b1 > S || (g == 0 && b0 != 0) ||
                       (g == NG - 1 && b1 != S) || L < 0 || L % BS != 0 ||
                       L > a.max_prefix_len;
      if (bad) s_misc[NW] = 1;
    }
    // Sequence b (thread b): its group (the last whose start is <= b; some
    // group in [0, NG) even when the starts are not a partition, which the
    // group checks flag), no shorter than that group's prefix, within the
    // host's bound.
    for (int b = tid; b < S; b += NTH) {
      int lo = 0, hi = NG;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_gs[mid] <= b) lo = mid; else hi = mid;
      }
      const int T = s_len[b];
      if (T < s_pl[lo] || T > a.max_seq_len) s_misc[NW] = 1;
    }
    // Tasks before each group, Hkv ceil(F_g / mpt) per group (a group of no
    // members or more than S counts none; the checks above flag it).
    auto group_tasks = [&](int g) __attribute__((always_inline)) {
      const int F = s_gs[g + 1] - s_gs[g];
      return F > 0 && F <= S ? Hkv * div_up(F, mpt) : 0;
    };
    if (NG <= 64) {
      // one wavefront's scan, lane g holding group g
      if (tid < 64) {
        const int mine = tid < NG ? group_tasks(tid) : 0;
        int incl = mine;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(incl, off);
          if (tid >= off) incl += y;
        }
        if (tid < NG) s_tpre[tid + 1] = incl;
        if (tid == 0) s_tpre[0] = 0;
      }
      __syncthreads();
    } else {
      block_scan<NTH>(NG, group_tasks, s_tpre, s_misc, tid);
    }
  }
  int flagged = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) flagged |= s_misc[NW + i];
  if (flagged != 0) {
    for (int b = blockIdx.x; b < S; b += gridDim.x)
      for (int e = tid; e < Hq * D; e += NTH)
        store_out(a.out, static_cast<size_t>(b) * Hq * D + e, NAN, a.out_f32);
    return;
  }

  const float sl = a.scale_log2;
  const size_t blk_stride = static_cast<size_t>(Hkv) * M::kTile;
  const typename M::Lane ln(c, r);
  struct Slot {
    Regs x;
    int pos;
  };
  const int ntask = s_tpre[NG];
  // XCD-aware order: workgroup L starts at task (L % 8) (grid / 8) + L / 8,
  // so consecutive tasks run on one XCD (workgroups go to the XCDs in turn)
  const int grid = gridDim.x;
  const int L8 = blockIdx.x;
  const int tau0 = (grid % 8 == 0) ? (L8 & 7) * (grid >> 3) + (L8 >> 3) : L8;
  for (int tau = tau0; tau < ntask; tau += grid) {
    // 2. The task: its group, head and member block.
    int lo = 0, hi = NG;  // the group: largest g with s_tpre[g] <= tau
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_tpre[mid] <= tau) lo = mid; else hi = mid;
    }
    const int g = lo;
    const int b0 = s_gs[g];
    const int F = s_gs[g + 1] - b0;
    const int L = s_pl[g];
    const int nblk = div_up(F, mpt);
    const int rem = tau - s_tpre[g];
    const int h = rem / nblk;
    const int m0 = (rem - h * nblk) * mpt;
    const int mc = min(mpt, F - m0);  // members of this task
    const int nP = div_up(L, 32);     // prefix chunks
    // Suffix chunks of the task's members (every thread reads the mc <= 16
    // lengths itself, so no barrier is needed here).
    int nsuf = 0;
    for (int m = 0; m < mc; ++m) nsuf += div_up(s_len[b0 + m0 + m] - L, 32);
    const int n = nP + nsuf;  // the task's chunks
    if (n > lay.capacity) {
      // (cannot happen for lengths within the host's bounds, which size the
      // launch; a task past them gets NaN rows rather than records past LDS)
      for (int e = tid; e < mc * G * D; e += NTH) {
        const int R = e / D;
        const int m = R / G;
        store_out(a.out, (static_cast<size_t>(b0 + m0 + m) * Hq + h * G + (R - m * G)) * D +
                             (e - R * D), NAN, a.out_f32);
      }
      __syncthreads();
      continue;
    }

    // The tile's query rows as the QK^T B operand: lane (c, r) holds dims
    // [32 hs + 8 c, +8) of row r (member r / G, head r % G).  Rows past the
    // task's members read member 0's row; they attend nothing (always masked)
    // and are not written.  They load now, ahead of the records' table loads,
    // so the first fold does not wait for them (0.1 us on prefix_cow).
    const int rm = r / G;
    const bool live = r < mc * G;
    bf16x8_t qop[HS];
    {
      const uint16_t* qrow =
          a.q + (static_cast<size_t>(b0 + m0 + (live ? rm : 0)) * Hq + h * G + (live ? r - rm * G : 0)) *
                    D + 8 * c;
#pragma unroll
      for (int hs = 0; hs < HS; ++hs) qop[hs] = load_bf16x8(qrow + 32 * hs);
    }
    // 3. The chunk records: member (-1: prefix), valid tokens, physical blocks.
    for (int i = tid; i < n; i += NTH) {
      int member, tok0, last_blk;
      const int32_t* row;
      if (i < nP) {
        member = -1;
        tok0 = 32 * i;
        row = a.block_tables + static_cast<size_t>(b0) * MB;  // every member's row holds the prefix
        last_blk = (L - 1) / BS;
        s_rec[i * kRec + 1] = min(32, L - tok0);
      } else {
        // suffix chunk j: member m's chunk j - (suffix chunks before m)
        int j = i - nP;
        int m = 0;
        int T = s_len[b0 + m0];
        for (int cnt = div_up(T - L, 32); j >= cnt && m + 1 < mc; cnt = div_up(T - L, 32)) {
          j -= cnt;
          ++m;
          T = s_len[b0 + m0 + m];
        }
        member = m;
        tok0 = L + 32 * j;
        row = a.block_tables + static_cast<size_t>(b0 + m0 + m) * MB;
        last_blk = (T - 1) / BS;
        s_rec[i * kRec + 1] = min(32, T - tok0);
      }
      s_rec[i * kRec] = member;
#pragma unroll
      for (int jb = 0; jb < NB; ++jb)
        s_rec[i * kRec + 2 + jb] = row[min(min(tok0 / BS + jb, last_blk), MB - 1)];
    }
    __syncthreads();

    // 4. Loading and folding the task's chunks.
    const size_t head_off = static_cast<size_t>(h) * M::kTile;
    auto issue = [&](int pos, Slot& sl8) __attribute__((always_inline)) {
      const int* rec = s_rec + pos * kRec;
      size_t base[NB];
#pragma unroll
      for (int jb = 0; jb < NB; ++jb)
        base[jb] = static_cast<size_t>(__builtin_amdgcn_readfirstlane(rec[2 + jb])) * blk_stride +
                   head_off;
      M::load(a.k_cache, a.v_cache, base, ln, sl8.x);
      sl8.pos = pos;
    };
    typename M::State st;
    st.reset();
    st.m2 = kEmptyMax;
    // One chunk into the state: Mfma::step with the rows the chunk does not
    // belong to masked out.
    auto consume = [&](Slot& sl8) __attribute__((always_inline)) {
      const int* rec = s_rec + sl8.pos * kRec;
      const int member = __builtin_amdgcn_readfirstlane(rec[0]);
      const int valid = __builtin_amdgcn_readfirstlane(rec[1]);
      const bool active = live && (member < 0 || member == rm);
      f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hs = 0; hs < HS; ++hs) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sl8.x.k[0][hs], qop[hs], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sl8.x.k[1][hs], qop[hs], s1, 0, 0, 0);
      }
      const int lv = active ? valid - 8 * c : 0;  // this lane's tokens its row attends
      float xs[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xs[i] = (i < lv) ? s0[i] : -INFINITY;
        xs[4 + i] = (4 + i < lv) ? s1[i] : -INFINITY;
      }
      float cm = maxnan(maxnan(xs[0], xs[1], xs[2]), maxnan(xs[3], xs[4], xs[5]),
                        maxnan(xs[6], xs[7]));
      cm = max_over_rows(cm) * sl;
      if (__ballot(cm > st.m2 + kRescaleThreshold) != 0) {
        const float mn = fmaxf(st.m2, cm);
        const float alpha = fast_exp2(st.m2 - mn);
        st.m2 = mn;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float f = __shfl(alpha, 4 * c + i);  // factor of row 4 c + i
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) st.acc[nt][i] *= f;
          st.lsum[i] *= f;
        }
      }
      bf16x8_t pa;
#pragma unroll
      for (int e = 0; e < 8; ++e) pa[e] = static_cast<__bf16>(fast_exp2(fmaf(xs[e], sl, -st.m2)));
      if (valid < 32) {
        const int vv = valid - 8 * c;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            sl8.x.v[nt][e] = (e < vv) ? sl8.x.v[nt][e] : static_cast<__bf16>(0.f);
      }
      const bf16x8_t ones = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        st.acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, sl8.x.v[nt], st.acc[nt], 0, 0, 0);
      st.lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, ones, st.lsum, 0, 0, 0);
    };

    // 5. Wavefront w folds chunks w, w + NW, ... through a ring of two (a
    // refill past its last chunk re-reads its first, which is not folded
    // again, so every refill issues its loads and the wait counts stay exact).
    const int nmine = n > w ? (n - w + NW - 1) / NW : 0;
    if (nmine > 0) {
      Slot ring[2];
      issue(w, ring[0]);
      issue(nmine > 1 ? w + NW : w, ring[1]);
      for (int k = 0;;) {
        if (k >= nmine) break;
        consume(ring[0]);
        issue(k + 2 < nmine ? w + (k + 2) * NW : w, ring[0]);
        ++k;
        if (k >= nmine) break;
        consume(ring[1]);
        issue(k + 2 < nmine ? w + (k + 2) * NW : w, ring[1]);
        ++k;
      }
    }

    // 6. The wavefronts' states into LDS (lane (c, r) holds row 4 c + i's
    // accumulator for features 16 nt + r and its sum, and row r's maximum),
    // then merged in wavefront order and written out.
    {
      float* sa = s_acc + static_cast<size_t>(w) * kCascadeRows * D;
      float* sm = s_ml + w * kCascadeRows * 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * c + i;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sa[row * D + 16 * nt + r] = st.acc[nt][i];
        if (r == 0) sm[row * 2 + 1] = st.lsum[i];
      }
      if (c == 0) sm[r * 2] = st.m2;
    }
    __syncthreads();
    for (int e = tid; e < mc * G * E4; e += NTH) {
      const int R = e / E4;
      const int d4 = e - R * E4;
      // every state's values read first (independent LDS reads), then folded
      // in wavefront order; a wavefront that attended none of the row's tokens
      // (sum 0, maximum kEmptyMax) adds nothing
      float pm[NW], pl[NW];
      f32x4_t pa[NW];
#pragma unroll
      for (int wv = 0; wv < NW; ++wv) {
        pm[wv] = s_ml[(wv * kCascadeRows + R) * 2];
        pl[wv] = s_ml[(wv * kCascadeRows + R) * 2 + 1];
        pa[wv] = *reinterpret_cast<const f32x4_t*>(
            s_acc + (static_cast<size_t>(wv) * kCascadeRows + R) * D + 4 * d4);
      }
      float mx = kEmptyMax;
#pragma unroll
      for (int wv = 0; wv < NW; ++wv) mx = fmaxf(mx, pm[wv]);
      float den = 0.f;
      f32x4_t num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int wv = 0; wv < NW; ++wv) {
        const float fj = fast_exp2(pm[wv] - mx);
        den += pl[wv] * fj;
        num += pa[wv] * fj;
      }
      // a member with no tokens (T = 0) has an all-zero row
      const f32x4_t o = den > 0.f ? num * (1.0f / den) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int m = R / G;
      const size_t orow =
          (static_cast<size_t>(b0 + m0 + m) * Hq + h * G + (R - m * G)) * D + 4 * d4;
#pragma unroll
      for (int t = 0; t < 4; ++t) store_out(a.out, orow + t, o[t], a.out_f32);
    }
    __syncthreads();  // the task's records, states and member prefix are done with
  }
}

template <int D, int BS, int NW>
hipError_t launch_wg_bs(const CascadeLaunch& a, const CascadeWgLayout& lay, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&cascade_wg<D, BS, NW>),
      hipFuncAttributeMaxDynamicSharedMemorySize, kCascadeLdsBytes);
  if (attr != hipSuccess) return attr;
  cascade_wg<D, BS, NW><<<dim3(a.wg_grid), dim3(NW * 64), static_cast<size_t>(lay.words) * 4,
                          stream>>>(a, lay);
  return hipGetLastError();
}

template <int D>
hipError_t launch_wg_d(const CascadeLaunch& a, const CascadeWgLayout& lay, hipStream_t stream) {
  constexpr int NW = cascade_wg_waves(D);
  switch (a.block_size) {
    case 8: return launch_wg_bs<D, 8, NW>(a, lay, stream);
    case 16: return launch_wg_bs<D, 16, NW>(a, lay, stream);
    default: return launch_wg_bs<D, 32, NW>(a, lay, stream);
  }
}

template <int D>
hipError_t launch_d(const CascadeLaunch& a, hipStream_t stream) {
  switch (a.block_size) {
    case 8: return launch_bs<D, 8>(a, stream);
    case 16: return launch_bs<D, 16>(a, stream);
    default: return launch_bs<D, 32>(a, stream);
  }
}

}  // namespace

bool cascade_shape_supported(int head_dim, int block_size, int group, int num_seqs) {
  return (head_dim == 64 || head_dim == 128) &&
         (block_size == 8 || block_size == 16 || block_size == 32) && group >= 1 &&
         group <= 16 && num_seqs <= kCascadeMaxSeqs;
}

CascadeWgLayout cascade_wg_layout(int head_dim, int block_size, int num_seqs, int num_groups,
                                  int64_t want_chunks) {
  CascadeWgLayout lay = {};
  const int nw = cascade_wg_waves(head_dim);
  const int nb = block_size >= 32 ? 1 : 32 / block_size;
  auto up4 = [](int64_t x) { return static_cast<int32_t>((x + 3) / 4 * 4); };
  int32_t w = 0;
  lay.off_len = w;
  w = up4(w + num_seqs);
  lay.off_gs = w;
  w = up4(w + num_groups + 1);
  lay.off_pl = w;
  w = up4(w + num_groups);
  lay.off_tpre = w;
  w = up4(w + num_groups + 1);
  lay.off_misc = w;
  w = up4(w + 2 * nw);
  lay.off_acc = w;
  w = up4(w + static_cast<int64_t>(nw) * kCascadeRows * head_dim);
  lay.off_ml = w;
  w = up4(w + nw * kCascadeRows * 2);
  lay.off_rec = w;
  const int64_t left = kCascadeLdsBytes / 4 - w;
  const int rec = 2 + nb;
  int64_t cap = left > 0 ? left / rec : 0;
  if (want_chunks > 0 && want_chunks < cap) cap = want_chunks;
  lay.capacity = static_cast<int32_t>(cap);
  lay.words = lay.capacity > 0 ? up4(w + static_cast<int64_t>(lay.capacity) * rec) : w;
  return lay;
}

hipError_t launch_cascade(const CascadeLaunch& a, hipStream_t stream) {
  if (a.use_wg) {
    if (a.wg_grid < 1 || a.members_per_task < 1 || a.members_per_task * a.group > kCascadeRows)
      return hipErrorInvalidValue;
    // all of the LDS: one workgroup per compute unit
    const CascadeWgLayout lay =
        cascade_wg_layout(a.head_dim, a.block_size, a.num_seqs, a.num_groups, 0);
    if (lay.capacity < a.wg_chunks) return hipErrorInvalidValue;
    return a.head_dim == 64 ? launch_wg_d<64>(a, lay, stream) : launch_wg_d<128>(a, lay, stream);
  }
  if (a.waves < kNW || a.waves % kNW != 0) return hipErrorInvalidValue;
  return a.head_dim == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace pkv
