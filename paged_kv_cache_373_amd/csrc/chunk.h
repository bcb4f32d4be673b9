// chunk.h - device code shared by the matrix-core decode kernels: element
// types, device-coherent partial-result access, the 32-token chunk step on
// the matrix cores, and the new-token patch of the fused decode step.
// Included by the kernel translation units only (HIP device code).
#pragma once

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

// 32-token chunks each wavefront of the matrix-core kernels keeps in flight.
#ifndef PKV_PIPELINE_DEPTH
#define PKV_PIPELINE_DEPTH 2
#endif
constexpr int kDepth = PKV_PIPELINE_DEPTH;

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
}

// A K/V tile load: an ordinary load, or (kStream) a non-temporal one, which
// tells the caches the line will not be read again soon.  Streaming loads pay
// off only when no other sequence of the call reads the same physical block
// (no shared prefix): a block several sequences share is served from the
// caches for all but its first reader only with ordinary loads.
template <bool kStream>
__device__ __forceinline__ bf16x8_t load_kv(const uint16_t* p) {
  const u32x4_t* a = reinterpret_cast<const u32x4_t*>(p);
  if constexpr (kStream)
    return __builtin_bit_cast(bf16x8_t, __builtin_nontemporal_load(a));
  else
    return __builtin_bit_cast(bf16x8_t, *a);
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  // v_cvt_pk_bf16_f32 rounds to nearest even
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// NaN-propagating maximum (IEEE 754-2019 maximum): one v_maximum3_f32 for up
// to three operands on gfx950.  Unlike fmaxf it needs no canonicalising of
// operands the compiler cannot prove canonical (matrix-core results, values
// moved between lanes), which would cost an instruction per operand.  A NaN
// operand gives NaN, as it would through the exponential that follows.
__device__ __forceinline__ float maxnan(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float maxnan(float a, float b, float c) {
  return maxnan(maxnan(a, b), c);
}

// Inclusive sum over lanes 0 .. lane of the wavefront, in registers: a
// Hillis-Steele scan inside each 16-lane row (row shifts by 1, 2, 4, 8 with
// zeros shifted in), then row 0's total added to row 1 and row 2's to row 3
// (broadcast of lane 15 of the row before), then lane 31's running total to
// rows 2 and 3.  Six data-parallel-primitive adds, no trip through the LDS
// crossbar as a shuffle takes.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return x;
}

// Maximum over the four 16-lane rows of the wavefront at each lane's column
// (lanes r, 16 + r, 32 + r and 48 + r), on every lane.  The two row-swap
// instructions of gfx950 pair rows (0,1) and (2,3), then halves (0,1) and
// (2,3), in registers: no trip through the LDS crossbar as a shuffle takes.
__device__ __forceinline__ float max_over_rows(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto p16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float t = maxnan(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
  const uint32_t w = __float_as_uint(t);
  const auto p32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return maxnan(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
}

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

// Reads of partials through a buffer resource with the device-coherence cache
// policy (the same bit an agent-scope atomic load carries).  Unlike atomic
// loads the compiler keeps many of these in flight at once, which is what a
// merge over many partials needs.  Offsets are in bytes and stay below
// `bytes`; the resource's fourth word is the raw 32-bit data format of gfx9.
struct CoherentReader {
  static constexpr int kRsrcWord3 = 0x00020000;
  static constexpr int kDeviceCoherent = 16;  // SC1
  __amdgpu_buffer_rsrc_t rsrc;
  __device__ CoherentReader(const void* base, uint32_t bytes)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                               kRsrcWord3)) {}
  __device__ float f32(uint32_t off) const {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_raw_buffer_load_b32(rsrc, off, 0, kDeviceCoherent));
  }
  __device__ f32x4_t f32x4(uint32_t off) const {
    return __builtin_bit_cast(f32x4_t,
                              __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, kDeviceCoherent));
  }
};

__device__ __forceinline__ void store_out(void* out, size_t idx, float v, int out_f32) {
  if (out_f32)
    static_cast<float*>(out)[idx] = v;
  else
    static_cast<uint16_t*>(out)[idx] = float_to_bf16_bits(v);
}

// ---------------------------------------------------------------------------
// The matrix-core chunk step shared by decode_stream and decode_mfma.
//
// A wavefront consumes a KV head's tokens 32 at a time (a "chunk": 1, 2 or 4
// physical blocks at B = 32, 16, 8).  Lane roles (lane = 16 c + r, c in 0..3,
// r in 0..15):
//   QK^T   S^T[t][g] = sum_d K[t][d] Q[g][d] as two 16x16x32 MFMAs per 16-token
//          half u of the chunk and per 32-wide slice of d.
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
template <int D, int BS>
struct Mfma {
  static_assert(D % 32 == 0 && D <= 128, "head_dim");
  static_assert(BS == 8 || BS == 16 || BS == 32, "block_size");
  static constexpr int HS = D / 32;                  // 32-wide slices of d (QK^T k-steps)
  static constexpr int NT = D / 16;                  // 16-wide slices of d (P.V n-tiles)
  static constexpr int NB = BS >= 32 ? 1 : 32 / BS;  // physical blocks per chunk
  static constexpr size_t kTile = static_cast<size_t>(BS) * D;  // elements per (block, head)

  struct Regs {  // one chunk's operands
    bf16x8_t k[2][HS];
    bf16x8_t v[NT];
  };
  struct State {  // online softmax of the G query heads of one KV head
    float m2;        // running max of head g = r, base-2 units
    f32x4_t acc[NT];
    f32x4_t lsum;
    __device__ void reset() {
      m2 = -INFINITY;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      lsum = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  struct Lane {  // lane-constant address parts
    int kj[2], koff[2], vj, voff;
    __device__ explicit Lane(int c, int r) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tok = 8 * (r >> 2) + 4 * u + (r & 3);
        kj[u] = tok / BS;
        koff[u] = (tok % BS) * D + 8 * c;
      }
      vj = (8 * c) / BS;
      voff = r * BS + (8 * c) % BS;
    }
  };

  // Query group of KV head `kvh` of sequence b as the QK^T B operand.  The
  // loads go through a buffer resource that spans the group's G rows: lanes
  // of rows r >= G address past its end and read zeros, so no instruction
  // touches the operand between its load and the matrix-core op that uses it
  // (a select there would make the wavefront wait for the load early).
  static __device__ void load_q(const uint16_t* q, int Hq, int G, int b, int kvh, int c, int r,
                                bf16x8_t (&qop)[HS]) {
    constexpr int kRsrcWord3 = 0x00020000;
    const uint16_t* grp = q + (static_cast<size_t>(b) * Hq + static_cast<size_t>(kvh) * G) * D;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(grp), 0, G * D * 2, kRsrcWord3);
    const int off = (r * D + 8 * c) * 2;
#pragma unroll
    for (int hs = 0; hs < HS; ++hs)
      qop[hs] = __builtin_bit_cast(bf16x8_t,
                                   __builtin_amdgcn_raw_buffer_load_b128(rq, off + 64 * hs, 0, 0));
  }

  // Issues the loads of one chunk whose NB (block, head) tiles start at the
  // element offsets `base` (wave-uniform); kStream selects non-temporal loads.
  template <bool kStream = false>
  static __device__ void load(const uint16_t* k_cache, const uint16_t* v_cache,
                              const size_t (&base)[NB], const Lane& ln, Regs& x) {
    // base[j] for this lane's block j (a lane constant): two levels of
    // selects on the bits of j, so the choice stays in registers
    auto pick = [&](int j) {
      if constexpr (NB == 1) {
        return base[0];
      } else if constexpr (NB == 2) {
        return (j == 1) ? base[1] : base[0];
      } else {
        const size_t lo = (j & 1) ? base[1] : base[0];
        const size_t hi = (j & 1) ? base[3] : base[2];
        return (j & 2) ? hi : lo;
      }
    };
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint16_t* kp = k_cache + pick(ln.kj[u]) + ln.koff[u];
#pragma unroll
      for (int hs = 0; hs < HS; ++hs) x.k[u][hs] = load_kv<kStream>(kp + 32 * hs);
    }
    const uint16_t* vp = v_cache + pick(ln.vj) + ln.voff;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) x.v[nt] = load_kv<kStream>(vp + 16 * nt * BS);
  }

  // Folds one chunk into the state.  Tokens valid .. 31 of the chunk
  // (valid in 1..32, wave-uniform) lie past the sequence: their scores are
  // selected to -inf and their V rows to 0, so whatever those slots hold
  // (NaN included) never reaches the result.
  //
  // With kCausal, `lim` (per lane) is how many of the chunk's tokens the
  // lane's row r may see (causal attention: a row sees the positions up to its
  // own); the later ones get -inf scores as well.  The V rows are masked by
  // `valid` alone.
  template <bool kCausal = false>
  static __device__ void step(const bf16x8_t (&qop)[HS], Regs& x, int valid, float sl, int c,
                              State& st, int lim = 32) {
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.k[0][hs], qop[hs], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.k[1][hs], qop[hs], s1, 0, 0, 0);
    }
    // xs[e]: raw score q.k of token 8 c + e, e = 4 u + i (sl > 0 scales it
    // to base-2 units inside the exponent below, and keeps the order)
    float xs[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xs[i] = s0[i];
      xs[4 + i] = s1[i];
    }
    const bool tail = valid < 32;   // wave-uniform
    const int lv = valid - 8 * c;   // tokens of this lane group still in range
    if constexpr (kCausal) {
      const int lvc = min(valid, lim) - 8 * c;  // and visible to this lane's row
#pragma unroll
      for (int e = 0; e < 8; ++e) xs[e] = (e < lvc) ? xs[e] : -INFINITY;
    } else if (tail) {
#pragma unroll
      for (int e = 0; e < 8; ++e) xs[e] = (e < lv) ? xs[e] : -INFINITY;
    }
    float cm = maxnan(maxnan(xs[0], xs[1], xs[2]), maxnan(xs[3], xs[4], xs[5]), maxnan(xs[6], xs[7]));
    cm = max_over_rows(cm) * sl;
    // every lane of head g now holds the chunk maximum of head g, base-2 units
    if (__ballot(cm > st.m2 + kRescaleThreshold) != 0) {
      const float mn = fmaxf(st.m2, cm);
      const float alpha = fast_exp2(st.m2 - mn);  // 0 on the first chunk (m2 = -inf)
      st.m2 = mn;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = __shfl(alpha, 4 * c + i);  // factor of head 4 c + i
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) st.acc[nt][i] *= a;
        st.lsum[i] *= a;
      }
    }
    bf16x8_t pa;
#pragma unroll
    for (int e = 0; e < 8; ++e) pa[e] = static_cast<__bf16>(fast_exp2(fmaf(xs[e], sl, -st.m2)));
    if (tail) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          x.v[nt][e] = (e < lv) ? x.v[nt][e] : static_cast<__bf16>(0.f);
    }
    const bf16x8_t ones = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      st.acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, x.v[nt], st.acc[nt], 0, 0, 0);
    st.lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, ones, st.lsum, 0, 0, 0);
  }
};


// The new token of a fused decode step: its K and V rows (bf16 [D] each) in
// the layout the patch below needs - lane (c, r) holds dims [32 hs + 8 c, +8)
// of K for each hs, and feature 16 nt + r of V for each nt.  Loaded together
// with a chunk, through buffer resources whose size is the row's for the
// chunk holding a unit's last position and 0 for every other chunk: the
// loads are issued for every chunk, which keeps the ring's wait counts exact,
// but only the needed ones touch memory (a size-0 resource reads nothing and
// returns zeros).
template <int D>
struct NewToken {
  static constexpr int HS = D / 32;
  static constexpr int NT = D / 16;
  bf16x8_t k[HS];
  uint16_t v[NT];
  __device__ void load(const uint16_t* k_row, const uint16_t* v_row, bool needed, int c, int r) {
    constexpr int kRsrcWord3 = 0x00020000;
    const int bytes = needed ? D * 2 : 0;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(k_row), 0, bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(v_row), 0, bytes, kRsrcWord3);
#pragma unroll
    for (int hs = 0; hs < HS; ++hs)
      k[hs] = __builtin_bit_cast(bf16x8_t,
                                 __builtin_amdgcn_raw_buffer_load_b128(rk, (32 * hs + 8 * c) * 2, 0, 0));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      v[nt] = __builtin_amdgcn_raw_buffer_load_b16(rv, (16 * nt + r) * 2, 0, 0);
  }
};

// The new token of a fused decode step sits at position tn = valid - 1 of its
// unit's last chunk.  Its K and V rows (`nt`, loaded with the chunk) replace
// that position's operands in `x`; the cache slot is read, whatever it holds,
// before or after it is written.  Lane roles as in Mfma.
template <int D, int BS>
__device__ __forceinline__ void patch_new_operands(typename Mfma<D, BS>::Regs& x,
                                                   const NewToken<D>& nt, int valid, int lane) {
  using M = Mfma<D, BS>;
  constexpr int HS = M::HS;
  constexpr int NT = M::NT;
  const int c = lane >> 4;
  const int r = lane & 15;
  const int tn = valid - 1;
  const int un = (tn & 7) >> 2;             // K operand half holding the token
  const int rn = 4 * (tn >> 3) + (tn & 3);  // and its lane row
  const int cn = tn >> 3;                   // V operand lane group holding the token
  const int en = tn & 7;                    // and its element
  const bool in0 = (r == rn) && (un == 0);
  const bool in1 = (r == rn) && (un == 1);
#pragma unroll
  for (int hs = 0; hs < HS; ++hs) {
    const u32x4_t nk = __builtin_bit_cast(u32x4_t, nt.k[hs]);
    const u32x4_t o0 = __builtin_bit_cast(u32x4_t, x.k[0][hs]);
    const u32x4_t o1 = __builtin_bit_cast(u32x4_t, x.k[1][hs]);
    u32x4_t r0, r1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r0[e] = in0 ? nk[e] : o0[e];
      r1[e] = in1 ? nk[e] : o1[e];
    }
    x.k[0][hs] = __builtin_bit_cast(bf16x8_t, r0);
    x.k[1][hs] = __builtin_bit_cast(bf16x8_t, r1);
  }
  if (c == cn) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        x.v[n][e] = (e == en) ? __builtin_bit_cast(__bf16, nt.v[n]) : x.v[n][e];
  }
}

// One unit's new token of a fused decode step, written to its cache slot by
// any one wavefront (the one that reads the unit's last chunk patches its
// operands instead, so the slot may be read before or after this write).
// Unit u is sequence u / Hkv, KV head u % Hkv; its token is position T - 1 of
// a sequence of T >= 1 tokens: block table entry (T - 1) / BS, offset
// (T - 1) % BS.  load() issues the unit's loads (table entry, K row, V row)
// as vector loads; store() writes them once they have arrived.
template <int D, int BS>
struct TokenWrite {
  static constexpr int NV = D / 64;  // V features per lane
  u32x4_t k;                         // lanes l < D / 8: K dims [8 l, 8 l + 8)
  uint16_t v[NV];                    // lanes l: V features l + 64 j
  int blk;
  int on, hh, off;
  __device__ void load(const DecodeParams& prm, const int32_t* block_tables, int u, int T,
                       int lane) {
    constexpr int kRsrcWord3 = 0x00020000;
    const int Hkv = prm.num_kv_heads;
    const int b = u / Hkv;
    hh = u - b * Hkv;
    on = T >= 1 ? 1 : 0;
    off = on ? (T - 1) % BS : 0;
    const int32_t* ent = block_tables + static_cast<size_t>(b) * prm.max_blocks_per_seq +
                         (on ? (T - 1) / BS : 0);
    const size_t row = static_cast<size_t>(u) * D;
    const int bytes = on ? D * 2 : 0;
    const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(ent), 0, on ? 4 : 0, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(prm.k_new + row), 0, bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(prm.v_new + row), 0, bytes, kRsrcWord3);
    blk = __builtin_amdgcn_raw_buffer_load_b32(rt, 0, 0, 0);
    k = __builtin_amdgcn_raw_buffer_load_b128(rk, (lane < D / 8 ? 16 * lane : 0), 0, 0);
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] = __builtin_amdgcn_raw_buffer_load_b16(rv, 2 * (lane + 64 * j), 0, 0);
  }
  __device__ void store(const DecodeParams& prm, int lane) const {
    if (!on) return;
    const size_t tile =
        (static_cast<size_t>(__builtin_amdgcn_readfirstlane(blk)) * prm.num_kv_heads + hh) *
        Mfma<D, BS>::kTile;
    // Non-temporal: nothing in this launch reads the slot back from the cache.
    if (lane < D / 8)
      __builtin_nontemporal_store(
          k, reinterpret_cast<u32x4_t*>(prm.k_cache_w + tile + off * D + 8 * lane));
#pragma unroll
    for (int j = 0; j < NV; ++j)
      __builtin_nontemporal_store(
          v[j], &prm.v_cache_w[tile + static_cast<size_t>(lane + 64 * j) * BS + off]);
  }
};

// Sequence lengths into s_len[0, S) and the exclusive prefix of per-sequence
// 32-token chunk counts into s_pre[0, S], by all NTH threads of the workgroup
// (s_wsum holds one int per wavefront).  Ends with a barrier.
template <int NTH>
__device__ __forceinline__ void chunk_prefix(const int32_t* seq_lens, int S, int* s_len,
                                             int* s_pre, int* s_wsum, int tid) {
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int b = tid; b < S; b += NTH) s_len[b] = seq_lens[b];
  __syncthreads();
  const int per = (S + NTH - 1) / NTH;  // thread tid sums sequences [tid per, tid per + per)
  int mine = 0;
  for (int j = 0; j < per; ++j) {
    const int b = tid * per + j;
    if (b < S) mine += (s_len[b] + 31) >> 5;
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
    const int b = tid * per + j;
    if (b < S) {
      s_pre[b] = run;
      run += (s_len[b] + 31) >> 5;
    }
  }
  if (tid == NTH - 1) s_pre[S] = run;
  __syncthreads();
}

// Sequences with no tokens get an all-zero output row (workgroups share them
// round robin).
template <int D, int NTH>
__device__ __forceinline__ void zero_empty_rows(const DecodeParams& prm, const int* s_len,
                                                int tid) {
  const int Hq = prm.num_q_heads;
  for (int b = blockIdx.x; b < prm.num_seqs; b += gridDim.x)
    if (s_len[b] == 0)
      for (int e = tid; e < Hq * D; e += NTH)
        store_out(prm.out, static_cast<size_t>(b) * Hq * D + e, 0.f, prm.out_f32);
}

}  // namespace
}  // namespace pkv
