// cache_ops.hip - the two cache writers of the paged KV cache, for gfx950.
//
//   reshape_and_cache  puts token n's K and V rows into slot_mapping[n]
//                      (iThome ithelp article 10405755 on PagedAttention,
//                      section "手動畫一次 block table": a new token goes into
//                      the next free slot of the tail block; Fanyi Pu,
//                      "Infra: PagedAttention", section "按 Block 分配": the
//                      slot is physical block t/B's offset t%B).
//   append_tokens      the same write for a decode step's one new token per
//                      sequence, at position T_b - 1 of its block table (the
//                      non-fused half of pkv_paged_attention_decode_append).
//   copy_blocks        copies whole blocks src -> dst in every layer (Fanyi Pu,
//                      "Infra: PagedAttention", section "共享前缀，分叉时
//                      Copy-on-write": a shared tail block is duplicated before
//                      the first diverging write).
// Both are bit copies: no value is rounded or converted.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// One thread moves 8 features (16 bytes) of one (token, KV head) row.
// K: one 16-byte store into the token's row of the [B, D] tile.
// V: the tile is [D, B], so the 8 features go to 8 rows at stride B.
__global__ void __launch_bounds__(256)
    reshape_and_cache_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                             const int64_t* __restrict__ slot_mapping, int64_t num_items,
                             int32_t num_kv_heads, int32_t head_dim, uint16_t* __restrict__ k_cache,
                             uint16_t* __restrict__ v_cache, int32_t block_size) {
  const int64_t item = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (item >= num_items) return;
  const int32_t chunks = head_dim / 8;
  const int64_t row = item / chunks;  // (token, head)
  const int32_t c8 = static_cast<int32_t>(item - row * chunks);
  const int64_t n = row / num_kv_heads;
  const int32_t h = static_cast<int32_t>(row - n * num_kv_heads);
  const int64_t slot = slot_mapping[n];
  if (slot < 0) return;
  const int64_t blk = slot / block_size;
  const int32_t off = static_cast<int32_t>(slot - blk * block_size);
  const size_t src = static_cast<size_t>(row) * head_dim + 8 * c8;
  const size_t tile = (static_cast<size_t>(blk) * num_kv_heads + h) * block_size * head_dim;

  const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(k + src);
  *reinterpret_cast<u32x4_t*>(k_cache + tile + static_cast<size_t>(off) * head_dim + 8 * c8) = kv;

  const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(v + src);
  uint16_t* vdst = v_cache + tile + static_cast<size_t>(8 * c8) * block_size + off;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    vdst[static_cast<size_t>(2 * e) * block_size] = static_cast<uint16_t>(vv[e] & 0xFFFFu);
    vdst[static_cast<size_t>(2 * e + 1) * block_size] = static_cast<uint16_t>(vv[e] >> 16);
  }
}

// One thread per 8 features of one (sequence, KV head): the new token of
// sequence b sits at position T_b - 1, in block table[b][(T_b - 1) / B] at
// offset (T_b - 1) % B.
__global__ void __launch_bounds__(256)
    append_tokens_kernel(const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                         const int32_t* __restrict__ block_tables,
                         const int32_t* __restrict__ seq_lens, int64_t num_items,
                         int32_t max_blocks_per_seq, int32_t num_kv_heads, int32_t head_dim,
                         uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                         int32_t block_size) {
  const int64_t item = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (item >= num_items) return;
  const int32_t chunks = head_dim / 8;
  const int64_t row = item / chunks;  // (sequence, head)
  const int32_t c8 = static_cast<int32_t>(item - row * chunks);
  const int64_t b = row / num_kv_heads;
  const int32_t h = static_cast<int32_t>(row - b * num_kv_heads);
  const int32_t T = seq_lens[b];
  if (T <= 0) return;
  const int32_t t = T - 1;
  const int64_t blk = block_tables[b * max_blocks_per_seq + t / block_size];
  const int32_t off = t % block_size;
  const size_t src = static_cast<size_t>(row) * head_dim + 8 * c8;
  const size_t tile = (static_cast<size_t>(blk) * num_kv_heads + h) * block_size * head_dim;
  *reinterpret_cast<u32x4_t*>(k_cache + tile + static_cast<size_t>(off) * head_dim + 8 * c8) =
      *reinterpret_cast<const u32x4_t*>(k_new + src);
  const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(v_new + src);
  uint16_t* vdst = v_cache + tile + static_cast<size_t>(8 * c8) * block_size + off;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    vdst[static_cast<size_t>(2 * e) * block_size] = static_cast<uint16_t>(vv[e] & 0xFFFFu);
    vdst[static_cast<size_t>(2 * e + 1) * block_size] = static_cast<uint16_t>(vv[e] >> 16);
  }
}

struct LayerPtrs {
  u32x4_t* k[kMaxCopyLayers];
  u32x4_t* v[kMaxCopyLayers];
};

// grid (pair, layer, K|V); the workgroup streams one block in 16-byte units,
// four per thread in flight at a time (a 16 KiB block is one round trip).
__global__ void __launch_bounds__(256)
    copy_blocks_kernel(const LayerPtrs ptrs, const int32_t* __restrict__ block_pairs,
                       int64_t units_per_block) {
  const int pair = blockIdx.x;
  const int layer = blockIdx.y;
  u32x4_t* base = blockIdx.z == 0 ? ptrs.k[layer] : ptrs.v[layer];
  const int64_t src = block_pairs[2 * pair];
  const int64_t dst = block_pairs[2 * pair + 1];
  const u32x4_t* s = base + src * units_per_block;
  u32x4_t* d = base + dst * units_per_block;
  for (int64_t i0 = threadIdx.x; i0 < units_per_block; i0 += 4 * 256) {
    u32x4_t v[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int64_t i = i0 + m * 256;
      if (i < units_per_block) v[m] = s[i];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int64_t i = i0 + m * 256;
      if (i < units_per_block) d[i] = v[m];
    }
  }
}

// grid (block i, layer, K|V); the workgroup streams one block between the
// cache and the host buffer (pinned host memory the device reads and writes
// directly), four 16-byte units per thread in flight at a time.  The host
// buffer holds [layer][K|V][i] blocks back to back.
__global__ void __launch_bounds__(256)
    swap_blocks_kernel(const LayerPtrs ptrs, const int32_t* __restrict__ block_ids, int32_t n,
                       u32x4_t* host, int64_t units_per_block, int to_host) {
  const int64_t i = blockIdx.x;
  const int layer = blockIdx.y;
  const int z = blockIdx.z;
  u32x4_t* cache = (z == 0 ? ptrs.k[layer] : ptrs.v[layer]) +
                   static_cast<int64_t>(block_ids[i]) * units_per_block;
  u32x4_t* h = host + ((static_cast<int64_t>(layer) * 2 + z) * n + i) * units_per_block;
  const u32x4_t* src = to_host ? cache : h;
  u32x4_t* dst = to_host ? h : cache;
  for (int64_t j0 = threadIdx.x; j0 < units_per_block; j0 += 4 * 256) {
    u32x4_t v[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int64_t j = j0 + m * 256;
      if (j < units_per_block) v[m] = src[j];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int64_t j = j0 + m * 256;
      if (j < units_per_block) dst[j] = v[m];
    }
  }
}

}  // namespace

hipError_t launch_reshape_and_cache(const uint16_t* k, const uint16_t* v,
                                    const int64_t* slot_mapping, int32_t num_tokens,
                                    int32_t num_kv_heads, int32_t head_dim, uint16_t* k_cache,
                                    uint16_t* v_cache, int32_t block_size, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(num_tokens) * num_kv_heads * (head_dim / 8);
  if (items == 0) return hipSuccess;
  const int64_t blocks = (items + 255) / 256;
  reshape_and_cache_kernel<<<dim3(static_cast<uint32_t>(blocks)), 256, 0, stream>>>(
      k, v, slot_mapping, items, num_kv_heads, head_dim, k_cache, v_cache, block_size);
  return hipGetLastError();
}

hipError_t launch_append_tokens(const uint16_t* k_new, const uint16_t* v_new,
                                const int32_t* block_tables, const int32_t* seq_lens,
                                int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_kv_heads,
                                int32_t head_dim, uint16_t* k_cache, uint16_t* v_cache,
                                int32_t block_size, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(num_seqs) * num_kv_heads * (head_dim / 8);
  if (items == 0) return hipSuccess;
  const int64_t blocks = (items + 255) / 256;
  append_tokens_kernel<<<dim3(static_cast<uint32_t>(blocks)), 256, 0, stream>>>(
      k_new, v_new, block_tables, seq_lens, items, max_blocks_per_seq, num_kv_heads, head_dim,
      k_cache, v_cache, block_size);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                              const int32_t* block_pairs, int32_t num_pairs,
                              int64_t block_bytes, hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  LayerPtrs ptrs = {};
  for (int l = 0; l < num_layers; ++l) {
    ptrs.k[l] = static_cast<u32x4_t*>(k_caches[l]);
    ptrs.v[l] = static_cast<u32x4_t*>(v_caches[l]);
  }
  const dim3 grid(num_pairs, num_layers, 2);
  copy_blocks_kernel<<<grid, 256, 0, stream>>>(ptrs, block_pairs, block_bytes / 16);
  return hipGetLastError();
}

hipError_t launch_swap_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                              const int32_t* block_ids, int32_t n, int64_t block_bytes,
                              void* host_dev, int to_host, hipStream_t stream) {
  LayerPtrs ptrs = {};
  for (int l = 0; l < num_layers; ++l) {
    ptrs.k[l] = static_cast<u32x4_t*>(k_caches[l]);
    ptrs.v[l] = static_cast<u32x4_t*>(v_caches[l]);
  }
  const dim3 grid(static_cast<unsigned>(n), num_layers, 2);
  swap_blocks_kernel<<<grid, 256, 0, stream>>>(ptrs, block_ids, n, static_cast<u32x4_t*>(host_dev),
                                                block_bytes / 16, to_host);
  return hipGetLastError();
}

}  // namespace pkv
