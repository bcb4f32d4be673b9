// decode_wg.hip - the workgroup stream decode kernel for gfx950 (CDNA4).
//
// Sources (by title and section):
//   [ITH] iThome ithelp article 10405755 on PagedAttention, section
//         "PagedAttention 的核心想法": attention over a sequence's tokens is
//         unchanged; the kernel finds each token's K,V through the block table.
//   [PU]  Fanyi Pu, "Infra: PagedAttention", section "按 Block 分配": softmax
//         spans every visible token; segment results (o, max, Z) merge by
//         o = (Z1 o1 + Z2 o2) / (Z1 + Z2) after rescaling to a common maximum,
//         and segments need not coincide with physical blocks.
//
// The work of a call is the same as the stream kernel's: every (sequence b,
// KV head h) unit u = b Hkv + h cut into n_b = ceil(T_b / 32) chunks of 32
// tokens, C chunks in unit order.  It is dealt out in equal contiguous
// windows, but here a window belongs to a whole workgroup - all the
// wavefronts one compute unit holds - rather than to one wavefront:
//
//   * Inside a window the wavefronts take chunks one at a time from a counter
//     in LDS, so a wavefront that the hardware serves more slowly simply
//     takes fewer; the workgroup's wavefronts finish together.
//   * Each chunk is folded on its own (a fresh online softmax) and leaves its
//     (max, sum, accumulator) in an LDS slot of its own, then counts itself
//     in its batch: eight consecutive slots of its unit.  The wavefront that
//     counts a batch's last chunk merges the batch into the batch's first
//     slot right away, while its other chunk is loading.  The streaming loop
//     touches nothing but LDS besides its loads: a global store or atomic
//     inside it would leave loads and stores pending together on the
//     wavefront's memory counter, and the compiler then waits for every load
//     in flight before each fold.
//   * Once every chunk of the window is in, each unit's batches (at most
//     eight slots) are merged by one wavefront, all in slot order: the order
//     depends on the unit's chunk count alone, so which wavefront folded or
//     merged what never changes a result bit.  The window's first and last
//     units, the only ones a window edge can cut, have wavefronts of their
//     own.  A unit that lies wholly in the window is written to the output.
//     A cut unit is published as a piece (the window's part of it) and
//     counted on a device counter; the last piece to arrive merges all of
//     the unit's pieces in window order.
//
// A window holds at most `capacity` chunks (the LDS slots).  When the call's
// chunks need more, each workgroup walks several windows in turn, with a
// barrier between them.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "chunk.h"
#include "internal.h"

namespace pkv {
namespace {

// Words (4 bytes) of LDS per window chunk besides its state: the chunk
// record (kRecBase + NB words) and a unit-list entry (kUnitWords).
constexpr int kRecBase = 5;    // sequence, KV head, unit's first window position | its chunks
                               // here << 12, valid | last << 8 | entry << 12, batch count
constexpr int kUnitWords = 4;  // first window position | chunks << 12 | whole << 24, sequence,
                               // head, unused
constexpr int kBatch = 8;      // slots merged together (all their reads in flight at once)
constexpr int kMiscWords = 4;  // chunk counter, first and last units' chunks, middle units
// Unit entries pack window positions and chunk counts in 12 bits.
static_assert(kWgMaxCapacity < 4096, "window positions must fit 12 bits");

// LDS-only ordering: the slot writes of a fold are complete before its count
// is, and a merge reads slots only after the count that completed them.
// Vector-memory loads in flight are not waited for.
__device__ __forceinline__ void lds_release() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
}
__device__ __forceinline__ void lds_acquire() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int D, int BS, int NW, bool kStream>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 2 : 1)))
    decode_wg(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
              const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
              const int32_t* __restrict__ seq_lens, const DecodeParams prm, const WgLayout lay) {
  using M = Mfma<D, BS>;
  using Regs = typename M::Regs;
  constexpr int NB = M::NB;
  constexpr int HS = M::HS;
  constexpr int NT = M::NT;
  constexpr int DEPTH = kDepth;
  constexpr int NTH = NW * 64;
  constexpr int kBlocksPerChunk = 32 / BS;
  constexpr int DS = kRecBase + NB;  // words per chunk record
  constexpr int E4 = D / 4;          // float4s per head in a state slot
  constexpr int kMaxIt = (16 * E4 + 63) / 64;  // float4s of a slot per lane at the largest group

  extern __shared__ __align__(16) int lds[];
  int* s_len = lds + lay.off_len;
  int* s_pre = lds + lay.off_pre;
  int* s_wsum = lds + lay.off_wsum;
  int* s_misc = lds + lay.off_misc;
  int* s_rec = lds + lay.off_rec;
  int* s_unit = lds + lay.off_unit;  // unit entries: [0] first unit, [1] last unit, [2 + t] the rest
  int* s_list = lds + lay.off_list;  // entries of the units between the first and the last
  float* s_acc = reinterpret_cast<float*>(lds + lay.off_acc);  // [capacity][G][16][NT]
  float* s_ml = reinterpret_cast<float*>(lds + lay.off_ml);    // [capacity][G][max, sum]

  const int S = prm.num_seqs;
  const int Hkv = prm.num_kv_heads;
  const int Hq = prm.num_q_heads;
  const int G = prm.group;
  const int MB = prm.max_blocks_per_seq;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int c = lane >> 4;
  const int r = lane & 15;

  // 1. Lengths and the chunk prefix; the windows of this workgroup.  (The
  // middle-unit counter starts at zero; the prefix's barriers order this
  // before the first window's records.)
  if (tid == 0) s_misc[3] = 0;
  // A batch of at most 64 sequences keeps them in the lanes of every
  // wavefront (lane b: T_b and the chunks before sequence b), scanned in
  // registers, with one barrier after wavefront 0 has stored them; larger
  // batches take the general prefix.  The lanes also serve the records'
  // search below.
  const bool lanes_hold = S <= 64;
  int lane_len = 0, lane_pre = 0;
  if (lanes_hold) {
    const int T = seq_lens[min(lane, S - 1)];
    lane_len = lane < S ? T : 0;
    const int nbl = (lane_len + 31) >> 5;
    const int incl = wave_incl_scan(nbl);
    lane_pre = incl - nbl;
    if (tid < 64) {
      if (lane < S) {
        s_len[lane] = lane_len;
        s_pre[lane] = lane_pre;
      }
      if (lane == S - 1) s_pre[S] = incl;
    }
    __syncthreads();
  } else {
    chunk_prefix<NTH>(seq_lens, S, s_len, s_pre, s_wsum, tid);
  }
  const int64_t C = static_cast<int64_t>(Hkv) * s_pre[S];
  const int64_t NWG = gridDim.x;
  const int64_t per_group = (C + NWG - 1) / NWG;
  const int64_t wpg = per_group <= lay.capacity ? 1 : (per_group + lay.capacity - 1) / lay.capacity;
  if (wpg > lay.max_windows) {
    // More chunks than the bound the launch was sized for (some T_b above
    // max_seq_len): every output row becomes NaN.
    for (int b = blockIdx.x; b < S; b += gridDim.x)
      for (int e = tid; e < Hq * D; e += NTH)
        store_out(prm.out, static_cast<size_t>(b) * Hq * D + e, NAN, prm.out_f32);
    return;
  }
  zero_empty_rows<D, NTH>(prm, s_len, tid);
  const int64_t NWIN = NWG * wpg;
  const int64_t NWeff = C < NWIN ? C : NWIN;  // windows that hold chunks

  const typename M::Lane ln(c, r);
  const float sl = prm.scale_log2;
  const size_t blk_stride = static_cast<size_t>(Hkv) * M::kTile;
  struct Slot {  // one ring entry: a chunk's K/V operands, its unit's query group, its position
    Regs x;
    bf16x8_t q[HS];
    int pos;
  };

  // Sequence holding global chunk cc: the largest lo with Hkv * s_pre[lo] <= cc.
  auto seq_of = [&](int64_t cc) __attribute__((always_inline)) {
    int lo = 0, hi = S;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (static_cast<int64_t>(Hkv) * s_pre[mid] <= cc)
        lo = mid;
      else
        hi = mid;
    }
    return lo;
  };
  // Unit of global chunk cc and the chunk's index in it.
  auto locate = [&](int64_t cc, int& b, int& h, int& lc) __attribute__((always_inline)) {
    b = seq_of(cc);
    const int nb = (s_len[b] + 31) >> 5;
    const int rem = static_cast<int>(cc - static_cast<int64_t>(Hkv) * s_pre[b]);
    h = rem / nb;
    lc = rem - h * nb;
  };

  // A fused step's cache writes: wavefront gw of the grid writes the new
  // tokens of units gw, gw + (all wavefronts), ...  The memory counter retires
  // a wavefront's stores and loads in issue order, so a store issued among the
  // ring's loads would hold up every load behind it until it is acknowledged
  // (and a store among the first loads of the whole grid is acknowledged
  // slowly).  The first unit's rows are loaded now and written at the end;
  // any further units after that.
  const int fused = prm.k_new != nullptr ? 1 : 0;
  const int units = S * Hkv;
  const int gwave = static_cast<int>(blockIdx.x) * NW + __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gwaves = static_cast<int>(gridDim.x) * NW;
  TokenWrite<D, BS> tw;
  if (fused && gwave < units) tw.load(prm, block_tables, gwave, s_len[gwave / Hkv], lane);
  NewToken<D> nxt;  // the new token of the next chunk to fold, when it holds one

  for (int64_t k = 0; k < wpg; ++k) {
    const int64_t x = static_cast<int64_t>(blockIdx.x) * wpg + k;  // window id
    if (x >= NWeff) break;
    const int64_t ws = x * C / NWeff;
    const int n = static_cast<int>((x + 1) * C / NWeff - ws);
    if (k > 0) {  // the previous window's slots, records and lists are done with
      __syncthreads();
      if (tid == 0) s_misc[3] = 0;
      __syncthreads();
    }

    // 2. The window's chunk records and its unit list.  Unit entry 0 is the
    // window's first unit, 1 its last (unused when the window holds one
    // unit), 2 + t the unit between them whose first chunk sits at window
    // position t: a unit's chunks are consecutive in the window, so each
    // chunk finds its unit's entry, and the unit's chunk count in the window,
    // from its own position and index alone.  The entries of the units
    // between go to a list as well, in any order.
    {
      // With the sequences in the lanes, a chunk's sequence is the last one
      // of the window's span whose prefix (times Hkv) is <= the chunk: the
      // span's ends from two ballots, then a short walk over it per lane.
      int span0 = 0, span1 = 0;
      if (lanes_hold) {
        const int64_t hp = static_cast<int64_t>(Hkv) * lane_pre;
        span0 = __popcll(__ballot(lane < S && hp <= ws)) - 1;
        span1 = __popcll(__ballot(lane < S && hp <= ws + n - 1)) - 1;
      }
      for (int t = tid; t < n; t += NTH) {
        int b, h, lc;
        if (lanes_hold) {
          const int64_t cc = ws + t;
          b = span0;
          int pb = __builtin_amdgcn_readlane(lane_pre, span0);
          int tb = __builtin_amdgcn_readlane(lane_len, span0);
          for (int j = span0 + 1; j <= span1; ++j) {
            const int pj = __builtin_amdgcn_readlane(lane_pre, j);
            if (static_cast<int64_t>(Hkv) * pj <= cc) {
              b = j;
              pb = pj;
              tb = __builtin_amdgcn_readlane(lane_len, j);
            }
          }
          const int nb = (tb + 31) >> 5;
          const int rem = static_cast<int>(cc - static_cast<int64_t>(Hkv) * pb);
          h = rem / nb;
          lc = rem - h * nb;
        } else {
          locate(ws + t, b, h, lc);
        }
        const int T = s_len[b];
        const int nb = (T + 31) >> 5;
        const int valid = min(32, T - 32 * lc);
        const int first = max(t - lc, 0);       // the unit's first chunk in the window
        const int end = min(t - lc + nb, n);     // and one past its last
        const int kk = end - first;
        const int ui = first == 0 ? 0 : (end == n ? 1 : 2 + first);
        int* rec = s_rec + t * DS;
        rec[0] = b;
        rec[1] = h;
        rec[2] = first | (kk << 12);
        rec[3] = valid | ((lc == nb - 1 ? 4 : 0) << 8) | (ui << 12);
        rec[4] = 0;
        const int last_blk = (T + BS - 1) / BS - 1;
        const int32_t* row = block_tables + static_cast<size_t>(b) * MB;
#pragma unroll
        for (int j = 0; j < NB; ++j) rec[kRecBase + j] = row[min(lc * kBlocksPerChunk + j, last_blk)];
        if (t == first) {  // the unit's first chunk in the window writes its entry
          const int whole = (lc == 0 && end - first == nb) ? 1 : 0;
          int* ue = s_unit + ui * kUnitWords;
          ue[0] = first | (kk << 12) | (whole << 24);
          ue[1] = b;
          ue[2] = h;
          ue[3] = 0;
          if (ui >= 2)
            s_list[__hip_atomic_fetch_add(s_misc + 3, 1, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_WORKGROUP)] = ui;
        }
      }
      if (tid == 0) s_misc[0] = 0;  // chunk counter
      __syncthreads();
    }
    // Windows holding the first and the last chunk of unit (b, h).
    auto unit_span = [&](int b, int h, int64_t& gf, int64_t& gl) __attribute__((always_inline)) {
      const int nb = (s_len[b] + 31) >> 5;
      const int64_t cu0 = static_cast<int64_t>(Hkv) * s_pre[b] + static_cast<int64_t>(h) * nb;
      gf = ((cu0 + 1) * NWeff - 1) / C;
      gl = ((cu0 + nb) * NWeff - 1) / C;
    };

    auto grab = [&]() __attribute__((always_inline)) {
      int j = 0;
      if (lane == 0)
        j = __hip_atomic_fetch_add(s_misc, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return __builtin_amdgcn_readfirstlane(j);
    };
    auto issue = [&](int pos, Slot& sl8) __attribute__((always_inline)) {
      const int* rec = s_rec + pos * DS;
      const int b = __builtin_amdgcn_readfirstlane(rec[0]);
      const int hh = __builtin_amdgcn_readfirstlane(rec[1]);
      const size_t head_off = static_cast<size_t>(hh) * M::kTile;
      size_t base[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j)
        base[j] = static_cast<size_t>(__builtin_amdgcn_readfirstlane(rec[kRecBase + j])) *
                      blk_stride + head_off;
      M::template load<kStream>(k_cache, v_cache, base, ln, sl8.x);
      M::load_q(q, Hq, G, b, hh, c, r, sl8.q);
      sl8.pos = pos;
    };

    // The merged state of the kk slots p0, p0 + stride, ... for float4 e of
    // the [G][16][NT] slot layout (head gh).  Slots are read eight at a time (all
    // eight reads in flight) and folded against a running maximum; the
    // batches and the order within them depend on kk alone.
    auto merge_slots = [&](int p0, int kk, int stride, int e, int gh, float& mx, float& den,
                           f32x4_t& num) __attribute__((always_inline)) {
      mx = -INFINITY;
      den = 0.f;
      num = f32x4_t{0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < kk; j0 += 8) {
        float2 ml[8];
        f32x4_t a[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int p = p0 + stride * min(j0 + t, kk - 1);
          ml[t] = *reinterpret_cast<const float2*>(s_ml + (p * G + gh) * 2);
          a[t] = *reinterpret_cast<const f32x4_t*>(s_acc + static_cast<size_t>(p) * G * D + 4 * e);
        }
        float bm = ml[0].x;
#pragma unroll
        for (int t = 1; t < 8; ++t) bm = (j0 + t < kk) ? fmaxf(bm, ml[t].x) : bm;
        const float mn = fmaxf(mx, bm);
        const float fo = fast_exp2(mx - mn);  // 0 before the first batch
        den *= fo;
        num *= fo;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          if (j0 + t < kk) {
            const float f = fast_exp2(ml[t].x - mn);
            den += f * ml[t].y;
            num += f * a[t];
          }
        }
        mx = mn;
      }
    };
    // Output row features of float4 e: d = 16 nt + rr for nt = 4 n4 .. 4 n4 + 3.
    auto store_row4 = [&](size_t row, int e, int gh, const f32x4_t& v) __attribute__((always_inline)) {
      const int rem = e - gh * E4;
      const int rr = rem / (NT / 4);
      const int n4 = rem - rr * (NT / 4);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        store_out(prm.out, row * D + 16 * (4 * n4 + t) + rr, v[t], prm.out_f32);
    };
    // Counts the chunk folded into slot `pos`: in its unit when the unit has
    // at most one batch here, else in its batch, and the wavefront that
    // counts a batch's last chunk merges the batch into its first slot and
    // counts the batch in the unit.  A unit is complete when its count
    // reaches unit_target.
    auto count = [&](int pos) __attribute__((always_inline)) {
      const int* rec = s_rec + pos * DS;
      const int fk = __builtin_amdgcn_readfirstlane(rec[2]);
      const int ui = (__builtin_amdgcn_readfirstlane(rec[3]) >> 12) & 4095;
      const int first = fk & 4095;
      const int kk = fk >> 12;
      if (kk > kBatch) {
        const int bfirst = first + ((pos - first) & ~(kBatch - 1));
        const int bsize = min(kBatch, first + kk - bfirst);
        lds_release();
        int done = 0;
        if (lane == 0)
          done = __hip_atomic_fetch_add(s_rec + bfirst * DS + 4, 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_WORKGROUP) + 1;
        done = __builtin_amdgcn_readfirstlane(done);
        lds_acquire();
        if (done != bsize) return;
        // Straight-line code (no loop with a run-time trip count): inside the
        // streaming loop such a loop costs the compiler its exact count of the
        // loads in flight, and every fold would then wait for all of them.
#pragma unroll
        for (int it = 0; it < kMaxIt; ++it) {
          const int e = lane + 64 * it;
          if (e < G * E4) {
            const int gh = e / E4;
            float2 ml[kBatch];
            f32x4_t a[kBatch];
#pragma unroll
            for (int t = 0; t < kBatch; ++t) {
              const int p = bfirst + min(t, bsize - 1);
              ml[t] = *reinterpret_cast<const float2*>(s_ml + (p * G + gh) * 2);
              a[t] = *reinterpret_cast<const f32x4_t*>(s_acc + static_cast<size_t>(p) * G * D + 4 * e);
            }
            float mx = ml[0].x;
#pragma unroll
            for (int t = 1; t < kBatch; ++t) mx = (t < bsize) ? fmaxf(mx, ml[t].x) : mx;
            float den = 0.f;
            f32x4_t num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < kBatch; ++t) {
              const float f = (t < bsize) ? fast_exp2(ml[t].x - mx) : 0.f;
              den += f * ml[t].y;
              num += f * a[t];
            }
            *reinterpret_cast<f32x4_t*>(s_acc + static_cast<size_t>(bfirst) * G * D + 4 * e) = num;
            if (e == gh * E4)
              *reinterpret_cast<float2*>(s_ml + (bfirst * G + gh) * 2) = make_float2(mx, den);
          }
        }
      }
      lds_release();
      if (lane == 0)
        __hip_atomic_fetch_add(s_unit + ui * kUnitWords + 3, 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    auto unit_target = [&](int ui) __attribute__((always_inline)) {
      const int kk = (__builtin_amdgcn_readfirstlane(s_unit[ui * kUnitWords]) >> 12) & 4095;
      return kk <= kBatch ? kk : (kk + kBatch - 1) / kBatch;
    };
    auto unit_count = [&](int ui) __attribute__((always_inline)) {
      return __builtin_amdgcn_readfirstlane(__hip_atomic_load(
          s_unit + ui * kUnitWords + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    };
    // Waits until every chunk of the unit in entry ui is folded and counted.
    // Only a wavefront that has folded all of its own chunks waits, so the
    // chunks it waits for are in the hands of wavefronts still folding.
    auto wait_unit = [&](int ui) __attribute__((always_inline)) {
      const int target = unit_target(ui);
      while (unit_count(ui) != target) __builtin_amdgcn_s_sleep(1);
      lds_acquire();
    };

    // The window's own state of the unit in entry ui (complete) for float4 e:
    // its batches' merged slots, or its chunks' slots for a one-batch unit.
    auto own_state = [&](int ui, int e, int gh, float& mx, float& den, f32x4_t& num) __attribute__((always_inline)) {
      const int e0 = __builtin_amdgcn_readfirstlane(s_unit[ui * kUnitWords]);
      const int lu = e0 & 4095;
      const int kk = (e0 >> 12) & 4095;
      if (kk > kBatch)
        merge_slots(lu, (kk + kBatch - 1) / kBatch, kBatch, e, gh, mx, den, num);
      else
        merge_slots(lu, kk, 1, e, gh, mx, den, num);
    };
    // Every piece of unit (b, hh) - windows gf .. gl - merged in window order
    // into the output.  Piece own_j, when own_j >= 0, is this window's and is
    // taken from its slots (entry own_ui) instead of the workspace; the others
    // are published and counted.  The arithmetic is the same either way, so
    // the result does not depend on which window merges.
    auto merge_pieces = [&](int b, int hh, int64_t gf, int64_t gl, int own_j, int own_ui) __attribute__((always_inline)) {
      const int64_t u = static_cast<int64_t>(b) * Hkv + hh;
      const size_t row0 = static_cast<size_t>(b) * Hq + static_cast<size_t>(hh) * G;
      const int kp = static_cast<int>(gl - gf + 1);
      const CoherentReader racc(prm.part_out + (u + gf) * G * D,
                                static_cast<uint32_t>(kp * G * D * sizeof(float)));
      const CoherentReader rml(prm.part_ml + (u + gf) * G * 2,
                               static_cast<uint32_t>(kp * G * 2 * sizeof(float)));
      for (int e = lane; e < G * E4; e += 64) {
        const int gh = e / E4;
        float omx = 0.f, oden = 0.f;
        f32x4_t onum = {0.f, 0.f, 0.f, 0.f};
        if (own_j >= 0) own_state(own_ui, e, gh, omx, oden, onum);
        float mx = -INFINITY, den = 0.f;
        f32x4_t num = {0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0; j0 < kp; j0 += 8) {  // eight pieces' loads in flight at a time
          f32x4_t a[8];
          float pm[8], pl[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int j = min(j0 + t, kp - 1);
            a[t] = racc.f32x4(static_cast<uint32_t>((j * G * D + 4 * e) * sizeof(float)));
            pm[t] = rml.f32(static_cast<uint32_t>(((j * G + gh) * 2) * sizeof(float)));
            pl[t] = rml.f32(static_cast<uint32_t>(((j * G + gh) * 2 + 1) * sizeof(float)));
          }
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            if (j0 + t < kp) {
              const bool mine = j0 + t == own_j;
              const float pmt = mine ? omx : pm[t];
              const float plt = mine ? oden : pl[t];
              const f32x4_t at = mine ? onum : a[t];
              const float mn = fmaxf(mx, pmt);
              const float fo = fast_exp2(mx - mn);  // 0 for the first piece
              const float fj = fast_exp2(pmt - mn);
              den = den * fo + plt * fj;
              num = num * fo + at * fj;
              mx = mn;
            }
          }
        }
        store_row4(row0 + gh, e, gh, num * (1.0f / den));
      }
    };
    // A whole unit (entry ui, complete) to the output.
    auto finish_whole = [&](int ui) __attribute__((always_inline)) {
      const int b = __builtin_amdgcn_readfirstlane(s_unit[ui * kUnitWords + 1]);
      const int hh = __builtin_amdgcn_readfirstlane(s_unit[ui * kUnitWords + 2]);
      const size_t row0 = static_cast<size_t>(b) * Hq + static_cast<size_t>(hh) * G;
      for (int e = lane; e < G * E4; e += 64) {
        const int gh = e / E4;
        float mx, den;
        f32x4_t num;
        own_state(ui, e, gh, mx, den, num);
        store_row4(row0 + gh, e, gh, num * (1.0f / den));
      }
    };
    // Publishes this window's piece of the cut unit in entry ui (complete) to
    // workspace slot u + x and counts it; true when it was the last of the
    // unit's pieces to be counted.
    auto publish = [&](int ui) __attribute__((always_inline)) {
      const int b = __builtin_amdgcn_readfirstlane(s_unit[ui * kUnitWords + 1]);
      const int hh = __builtin_amdgcn_readfirstlane(s_unit[ui * kUnitWords + 2]);
      const int64_t u = static_cast<int64_t>(b) * Hkv + hh;
      int64_t gf, gl;
      unit_span(b, hh, gf, gl);
      float* pacc = prm.part_out + (u + x) * G * D;  // [G][16][NT]
      float* pml = prm.part_ml + (u + x) * G * 2;    // [G][max, sum]
      for (int e = lane; e < G * E4; e += 64) {
        const int gh = e / E4;
        float mx, den;
        f32x4_t num;
        own_state(ui, e, gh, mx, den, num);
#pragma unroll
        for (int t = 0; t < 4; ++t) store_coherent(pacc + 4 * e + t, num[t]);
        if (e == gh * E4) {
          store_coherent(pml + gh * 2, mx);
          store_coherent(pml + gh * 2 + 1, den);
        }
      }
      // The piece's device-coherent stores have completed before it is
      // counted (this waits for the wavefront's loads in flight as well).
      __builtin_amdgcn_s_waitcnt(0);
      uint32_t prev = 0;
      if (lane == 0)
        prev = __hip_atomic_fetch_add(prm.counters + u, 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      prev = __builtin_amdgcn_readfirstlane(prev);
      return prev == static_cast<uint32_t>(gl - gf);
    };
    // After the last piece of the cut unit in entry ui was counted here: all
    // pieces merged into the output, and the counter left at zero for the
    // next call.
    auto merge_all = [&](int ui) __attribute__((always_inline)) {
      const int b = __builtin_amdgcn_readfirstlane(s_unit[ui * kUnitWords + 1]);
      const int hh = __builtin_amdgcn_readfirstlane(s_unit[ui * kUnitWords + 2]);
      const int64_t u = static_cast<int64_t>(b) * Hkv + hh;
      int64_t gf, gl;
      unit_span(b, hh, gf, gl);
      __asm__ __volatile__("" ::: "memory");
      merge_pieces(b, hh, gf, gl, -1, ui);
      if (lane == 0)
        __hip_atomic_store(prm.counters + u, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // A cut unit (entry ui, waited for here): this window's piece is published to
    // workspace slot u + x and counted; when it is the last of the unit's
    // pieces to be counted, all of them are merged into the output.  With
    // `fast`, the counter is read first: when every other piece is counted
    // already, they are merged with this window's state straight away and
    // nothing is published (the counter is then left at zero for the next
    // call; no other window touches it again).
    auto finish_cut = [&](int ui, bool fast) __attribute__((always_inline)) {
      const int b = __builtin_amdgcn_readfirstlane(s_unit[ui * kUnitWords + 1]);
      const int hh = __builtin_amdgcn_readfirstlane(s_unit[ui * kUnitWords + 2]);
      const int64_t u = static_cast<int64_t>(b) * Hkv + hh;
      int64_t gf, gl;
      unit_span(b, hh, gf, gl);
      const uint32_t others = static_cast<uint32_t>(gl - gf);
      uint32_t seen = 0;
      if (fast && lane == 0)
        seen = __hip_atomic_load(prm.counters + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      wait_unit(ui);
      if (fast) {
        seen = __builtin_amdgcn_readfirstlane(seen);
        if (seen == others) {
          // The other pieces were stored and acknowledged before they were
          // counted, and their loads are issued after the count was seen.
          __asm__ __volatile__("" ::: "memory");
          merge_pieces(b, hh, gf, gl, static_cast<int>(x - gf), ui);
          if (lane == 0)
            __hip_atomic_store(prm.counters + u, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          return;
        }
      }
      if (publish(ui)) merge_all(ui);
    };
    // A fused step's new token of the chunk in `sl8`, if it holds one, into
    // `nxt` (the chunk is the next one this wavefront folds).
    auto load_new = [&](const Slot& sl8) __attribute__((always_inline)) {
      const int* rec = s_rec + sl8.pos * DS;
      const int vf = __builtin_amdgcn_readfirstlane(rec[3]);
      if (((vf >> 8) & 4) && prm.k_new != nullptr) {
        const int hh = __builtin_amdgcn_readfirstlane(rec[1]);
        const size_t row =
            (static_cast<size_t>(__builtin_amdgcn_readfirstlane(rec[0])) * Hkv + hh) * D;
        nxt.load(prm.k_new + row, prm.v_new + row, true, c, r);
      }
    };
    // Folds the chunk in `sl8` into its LDS slot.
    auto consume = [&](Slot& sl8) __attribute__((always_inline)) {
      const int pos = sl8.pos;
      const int* rec = s_rec + pos * DS;
      const int vf = __builtin_amdgcn_readfirstlane(rec[3]);
      const int valid = vf & 255;
      if (((vf >> 8) & 4) && prm.k_new != nullptr) {
        // The unit's last chunk holds the new token of a fused decode step
        // (position valid - 1), whose rows (in `nxt`) replace the operands.
        patch_new_operands<D, BS>(sl8.x, nxt, valid, lane);
      }
      typename M::State st;
      st.reset();
      M::step(sl8.q, sl8.x, valid, sl, c, st);
      float* sa = s_acc + static_cast<size_t>(pos) * G * D;
      float* sm = s_ml + static_cast<size_t>(pos) * G * 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int gh = 4 * c + i;
        if (gh < G) {
#pragma unroll
          for (int n4 = 0; n4 < NT / 4; ++n4)
            *reinterpret_cast<f32x4_t*>(sa + gh * D + r * NT + 4 * n4) =
                f32x4_t{st.acc[4 * n4][i], st.acc[4 * n4 + 1][i], st.acc[4 * n4 + 2][i],
                        st.acc[4 * n4 + 3][i]};
          if (r == 0) sm[gh * 2 + 1] = st.lsum[i];
        }
      }
      if (c == 0 && r < G) sm[r * 2] = st.m2;
    };
    // 3. The wavefronts take chunks until the window's are gone.  Every ring
    // refill issues its loads (a chunk past the window re-reads the window's
    // first chunk, which nobody folds) so the wait counts stay exact.
    static_assert(DEPTH == 2, "ring depth");
    Slot ring[2];
    int jr[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      jr[s] = grab();
      issue(jr[s] < n ? jr[s] : 0, ring[s]);
      if (s == 0) load_new(ring[0]);
    }
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // A wavefront's grabs rise, and it folds its chunks in grab order: once
    // one lies past the window, so do all the ring's later entries.  (The
    // ring is walked with constant indices so its registers stay put.)
    // After each fold the chunk is counted (and a batch it completes
    // merged), then the next chunk's new token (if it holds one) is loaded
    // before the refill, so the fold that needs it waits for nothing else.
    // The refill's loads are the last thing in the loop body: code after
    // them, or a global store or atomic anywhere in the loop, leaves the
    // compiler unable to count the loads in flight at the next fold, which
    // then waits for all of them.
    // Wavefront 0, which finishes the window's first unit, stops taking
    // chunks once that unit is cut by the window's edge, complete, and at
    // most 2 NW chunks are left: its piece is then published while the
    // window's last chunks are folded, and the previous window's last-unit
    // owner more often finds it counted and merges without publishing its own
    // (a threshold of NW / 2, NW, 2 NW, 3 NW chunks: 31.77, 31.56, 31.51,
    // 31.88 us against 31.99 us on the Llama-shaped step).
    auto first_unit_done = [&]() __attribute__((always_inline)) {
      const int taken = __builtin_amdgcn_readfirstlane(
          __hip_atomic_load(s_misc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
      if (n - taken > 2 * NW) return false;
      if ((__builtin_amdgcn_readfirstlane(s_unit[0]) >> 24) != 0) return false;
      return unit_count(0) == unit_target(0);
    };
    auto advance = [&](Slot& sl8, int& j, const Slot& next) __attribute__((always_inline)) {
      const int pos = sl8.pos;
      consume(sl8);
      count(pos);
      load_new(next);
      j = (NW > 1 && w == 0 && first_unit_done()) ? n : grab();  // (others remain to fold the rest)
      issue(j < n ? j : 0, sl8);
    };
    for (;;) {
      if (jr[0] >= n) break;
      advance(ring[0], jr[0], ring[1]);
      if (jr[1] >= n) break;
      advance(ring[1], jr[1], ring[0]);
    }

    // 4. Each unit is finished by one wavefront as soon as it is complete
    // (the others may still be folding; no barrier): the first unit by
    // wavefront 0, the last by wavefront NW - 1, the others round robin over
    // the rest.  The first unit's chunks come first in the window, and
    // wavefront 0 leaves the stream early for it (above), so it usually
    // publishes its piece while the window's last chunks are still being
    // folded.  A cut unit's owner reads the unit's counter
    // while it waits for the unit's last chunks, and when every other piece
    // is counted already, merges them without publishing its own.
    auto finish = [&](int ui) __attribute__((always_inline)) {
      if ((__builtin_amdgcn_readfirstlane(s_unit[ui * kUnitWords]) >> 24) != 0) {
        wait_unit(ui);
        finish_whole(ui);
      } else {
        finish_cut(ui, true);
      }
    };
    if (w == 0) {
      finish(0);
    } else if (w == NW - 1) {
      // (a window holding one unit has no entry 1: its last chunk is unit 0's)
      if ((__builtin_amdgcn_readfirstlane(s_rec[(n - 1) * DS + 3]) >> 12) == 1) finish(1);
    } else {
      const int nlist = __builtin_amdgcn_readfirstlane(s_misc[3]);
      for (int i = w - 1; i < nlist; i += NW - 2)
        finish(__builtin_amdgcn_readfirstlane(s_list[i]));
    }
  }
  if (fused && gwave < units) tw.store(prm, lane);
  if (fused)
    for (int u = gwave + gwaves; u < units; u += gwaves) {
      TokenWrite<D, BS> more;
      more.load(prm, block_tables, u, s_len[u / Hkv], lane);
      more.store(prm, lane);
    }
}

// Allows an instantiation the LDS a workgroup may use beyond the default
// dynamic allowance (once per process; repeated calls set the same value).
template <int D, int BS, int NW, bool kStream>
hipError_t allow_lds() {
  static const hipError_t e = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&decode_wg<D, BS, NW, kStream>),
      hipFuncAttributeMaxDynamicSharedMemorySize, kWgLdsBytes);
  return e;
}

template <int D, int BS, int NW, bool kStream>
hipError_t launch_wg(const DecodeLaunch& a, int groups, const WgLayout& lay, size_t lds,
                     hipStream_t stream) {
  const hipError_t e = allow_lds<D, BS, NW, kStream>();
  if (e != hipSuccess) return e;
  decode_wg<D, BS, NW, kStream><<<dim3(groups), dim3(NW * 64), lds, stream>>>(
      a.q, a.k_cache, a.v_cache, a.block_tables, a.seq_lens, a.prm, lay);
  return hipGetLastError();
}

template <int D, int NWS, int NWC>
hipError_t launch_wg_bs(const DecodeLaunch& a, int groups, const WgLayout& lay, size_t lds,
                        hipStream_t stream) {
  const bool st = a.prm.stream_kv != 0;
  switch (a.prm.block_size) {
    case 8:
      return st ? launch_wg<D, 8, NWS, true>(a, groups, lay, lds, stream)
                : launch_wg<D, 8, NWC, false>(a, groups, lay, lds, stream);
    case 16:
      return st ? launch_wg<D, 16, NWS, true>(a, groups, lay, lds, stream)
                : launch_wg<D, 16, NWC, false>(a, groups, lay, lds, stream);
    default:
      return st ? launch_wg<D, 32, NWS, true>(a, groups, lay, lds, stream)
                : launch_wg<D, 32, NWC, false>(a, groups, lay, lds, stream);
  }
}

}  // namespace

// Wavefronts per workgroup.  At head_dim 64 with streaming K/V loads (no
// block shared in the call), five (one SIMD with two, three with one):
// measured against four to eight on the Llama-shaped batch of 64 with the
// lane-held set-up (30.50-30.56 us against 30.61-30.67 for six, 30.82 for
// seven, 31.22 for eight, 31.91 for four); more bytes in flight per compute
// unit only lengthen the queues at the end of a window.  With cached loads
// (blocks shared across the call, many hits in L2), six: on the copy-on-write
// batch five ran 28.35 us against 26.96 for six.  At head_dim 128, four.
int wg_waves_per_group(int head_dim, bool stream_kv) {
  return head_dim <= 64 ? (stream_kv ? 5 : 6) : 4;
}
// The most either choice uses (the LDS layout has room for it).
static int wg_max_waves(int head_dim) { return head_dim <= 64 ? 6 : 4; }

WgLayout wg_layout(int head_dim, int block_size, int group, int num_seqs, int max_windows) {
  WgLayout lay = {};
  const int nb = block_size >= 32 ? 1 : 32 / block_size;
  const int nw = wg_max_waves(head_dim);
  auto up4 = [](int w) { return (w + 3) / 4 * 4; };
  int w = 0;
  lay.off_len = w;
  w = up4(w + num_seqs);
  lay.off_pre = w;
  w = up4(w + num_seqs + 1);
  lay.off_wsum = w;
  w = up4(w + nw);
  lay.off_misc = w;
  w = up4(w + kMiscWords);
  const int fixed = w;
  const int per_chunk = kRecBase + nb + kUnitWords + 1 + group * head_dim + 2 * group;
  int cap = (kWgLdsBytes / 4 - fixed - 2 * kUnitWords - 4 * 4) / per_chunk;
  if (cap > kWgMaxCapacity) cap = kWgMaxCapacity;
  lay.capacity = cap;
  lay.off_rec = w;
  w = up4(w + cap * (kRecBase + nb));
  lay.off_unit = w;
  w = up4(w + (cap + 2) * kUnitWords);
  lay.off_list = w;
  w = up4(w + cap);
  lay.off_acc = w;
  w = up4(w + cap * group * head_dim);
  lay.off_ml = w;
  w = up4(w + cap * group * 2);
  lay.words = w;
  lay.max_windows = max_windows;
  return lay;
}

hipError_t launch_decode_wg(const DecodeLaunch& a, int num_groups, int max_windows,
                            hipStream_t stream) {
  const WgLayout lay = wg_layout(a.prm.head_dim, a.prm.block_size, a.prm.group, a.num_seqs,
                                 max_windows);
  if (lay.capacity < 1) return hipErrorInvalidValue;
  const size_t lds = static_cast<size_t>(lay.words) * 4;
  return a.prm.head_dim == 64 ? launch_wg_bs<64, 5, 6>(a, num_groups, lay, lds, stream)
                              : launch_wg_bs<128, 4, 4>(a, num_groups, lay, lds, stream);
}

}  // namespace pkv
