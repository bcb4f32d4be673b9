// check.hip - checkers of the device-resident inputs that the attention and
// cache calls take on trust: the block tables and lengths of a decode call,
// the slot mapping of a cache write, and the (src, dst) pairs of a block copy.
//
// Sources (by title and section):
//   [ITH] iThome ithelp article 10405755 on PagedAttention, section
//         "手動畫一次 block table": a sequence of T tokens uses logical blocks
//         0 .. ceil(T/B)-1, each mapped by its table row to a physical block.
//   [PU]  Fanyi Pu, "Infra: PagedAttention", section "按 Block 分配": position
//         t lives in logical block t/B at offset t%B (its slot), and section
//         "共享前缀，分叉时 Copy-on-write": a shared block is copied to a fresh
//         block before a diverging write.
//
// Each checker only compares the values it is given; it never uses a table
// entry, slot or block id to address memory, so any values are safe to check.
// Violations are ORed into one int32 word as a bit mask; the word is cleared by
// the call itself (a one-thread kernel), so a call can be captured in a graph.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace pkv {
namespace {

constexpr int kCheckThreads = 256;

__global__ void clear_flags(int32_t* flags) { *flags = 0; }

// One workgroup per sequence (grid-stride).  Bit 0: a table entry that the
// sequence uses (logical blocks 0 .. ceil(T/B)-1) lies outside [0, P).
// Bit 1: a length outside [0, max_len]; that row's entries are not read.
__global__ void __launch_bounds__(kCheckThreads)
    check_tables_kernel(const int32_t* __restrict__ bt, const int32_t* __restrict__ lens,
                        int32_t S, int32_t MB, int32_t P, int32_t B, int32_t max_len,
                        int32_t* flags) {
  for (int b = blockIdx.x; b < S; b += gridDim.x) {
    const int T = lens[b];
    int f = (T < 0 || T > max_len) ? 2 : 0;
    const int nb = f == 0 ? (T + B - 1) / B : 0;  // <= MB, since max_len <= MB * B
    for (int j = threadIdx.x; j < nb; j += blockDim.x) {
      const int v = bt[static_cast<size_t>(b) * MB + j];
      if (v < 0 || v >= P) f |= 1;
    }
    if (f != 0) atomicOr(flags, f);
  }
}

// Thread i checks element i against every later one, a tile of kCheckThreads
// at a time through LDS.  Bit 0: a slot >= num_slots.  Bit 1: a non-negative
// slot that appears twice.  (Negative slots are padding and skipped.)
__global__ void __launch_bounds__(kCheckThreads)
    check_slots_kernel(const int64_t* __restrict__ slots, int32_t n, int64_t num_slots,
                       int32_t* flags) {
  __shared__ int64_t tile[kCheckThreads];
  const int i = blockIdx.x * kCheckThreads + threadIdx.x;
  const int64_t si = i < n ? slots[i] : -1;
  int f = si >= num_slots ? 1 : 0;
  for (int j0 = blockIdx.x * kCheckThreads; j0 < n; j0 += kCheckThreads) {
    __syncthreads();
    tile[threadIdx.x] = j0 + threadIdx.x < n ? slots[j0 + threadIdx.x] : -1;
    __syncthreads();
    if (si >= 0)
      for (int t = 0; t < kCheckThreads; ++t)
        if (j0 + t > i && j0 + t < n && tile[t] == si) f |= 2;
  }
  if (f != 0) atomicOr(flags, f);
}

// Thread i checks pair i against every pair.  Bit 0: a src or dst outside
// [0, P).  Bit 1: a dst that appears twice.  Bit 2: a dst that is also some
// pair's src (the copies would then depend on their order).
__global__ void __launch_bounds__(kCheckThreads)
    check_pairs_kernel(const int32_t* __restrict__ pairs, int32_t n, int32_t P, int32_t* flags) {
  __shared__ int32_t tsrc[kCheckThreads], tdst[kCheckThreads];
  const int i = blockIdx.x * kCheckThreads + threadIdx.x;
  const int32_t src = i < n ? pairs[2 * i] : 0;
  const int32_t dst = i < n ? pairs[2 * i + 1] : 0;
  int f = (i < n && (src < 0 || src >= P || dst < 0 || dst >= P)) ? 1 : 0;
  for (int j0 = 0; j0 < n; j0 += kCheckThreads) {
    __syncthreads();
    const int jl = j0 + threadIdx.x;
    tsrc[threadIdx.x] = jl < n ? pairs[2 * jl] : -1;
    tdst[threadIdx.x] = jl < n ? pairs[2 * jl + 1] : -1;
    __syncthreads();
    if (i < n)
      for (int t = 0; t < kCheckThreads; ++t) {
        const int j = j0 + t;
        if (j >= n) break;
        if (j != i && tdst[t] == dst) f |= 2;
        if (tsrc[t] == dst) f |= 4;
      }
  }
  if (f != 0) atomicOr(flags, f);
}

int groups_for(int64_t n) {
  const int64_t g = (n + kCheckThreads - 1) / kCheckThreads;
  return static_cast<int>(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_check_tables(const int32_t* block_tables, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                               int32_t block_size, int32_t max_len, int32_t* flags,
                               hipStream_t stream) {
  clear_flags<<<1, 1, 0, stream>>>(flags);
  if (num_seqs > 0) {
    const int grid = num_seqs < 4096 ? num_seqs : 4096;
    check_tables_kernel<<<grid, kCheckThreads, 0, stream>>>(
        block_tables, seq_lens, num_seqs, max_blocks_per_seq, num_blocks, block_size, max_len,
        flags);
  }
  return hipGetLastError();
}

hipError_t launch_check_slots(const int64_t* slot_mapping, int32_t num_tokens, int64_t num_slots,
                              int32_t* flags, hipStream_t stream) {
  clear_flags<<<1, 1, 0, stream>>>(flags);
  if (num_tokens > 0)
    check_slots_kernel<<<groups_for(num_tokens), kCheckThreads, 0, stream>>>(
        slot_mapping, num_tokens, num_slots, flags);
  return hipGetLastError();
}

hipError_t launch_check_pairs(const int32_t* block_pairs, int32_t num_pairs, int32_t num_blocks,
                              int32_t* flags, hipStream_t stream) {
  clear_flags<<<1, 1, 0, stream>>>(flags);
  if (num_pairs > 0)
    check_pairs_kernel<<<groups_for(num_pairs), kCheckThreads, 0, stream>>>(
        block_pairs, num_pairs, num_blocks, flags);
  return hipGetLastError();
}

}  // namespace pkv
