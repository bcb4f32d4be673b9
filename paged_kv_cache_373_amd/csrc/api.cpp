// api.cpp - the extern "C" boundary declared in include/pagedkv.h.
//
// Every entry point validates what the host can see (pointers, sizes,
// alignment, workspace) before it touches the HIP runtime; a failed check
// returns an error status and enqueues nothing.  Then it fills a launch
// description and calls the launcher of the chosen kernel.
#include "pagedkv.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <cstddef>

#include "internal.h"

namespace {

constexpr int32_t kAbiMajor = 2;
constexpr int32_t kAbiMinor = 0;
constexpr size_t kAlign = 256;
constexpr int32_t kMaxGridYZ = 65535;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Partition length of the partitioned kernels when the caller leaves the
// choice to the library (the stream kernel has no partitions): long enough
// that the split-KV merge costs a few percent of the KV traffic, short enough
// that a batch of moderate sequences yields thousands of workgroups.
int32_t default_partition(const pkv_decode_dims* d, int32_t block_size) {
  int32_t ps = d->max_seq_len >= 8192 ? 512 : 256;
  if (ps % block_size != 0) ps = block_size;  // generic kernel with an odd block size
  return ps;
}

enum Family { kGeneric, kMfma, kStream, kStreamWg };

// Wavefronts the stream kernel launches by default: one per SIMD of an MI355X
// (256 CUs x 4), every one resident from the start; fewer when the problem is
// small.  At head_dim 64 two per SIMD were measured too: the longer streams of
// one per SIMD publish half the pieces and keep enough bytes in flight (8
// sequences of 16-32 K tokens: 82.3 -> 75.7 us; the 16-layer pool step at
// B = 8 / 16 / 32 within -2 .. +3.5 % per layer).
int32_t stream_wave_target(int32_t /*head_dim*/) { return 1024; }
constexpr int32_t kMinChunksPerWave = 4;
// The workgroup stream kernel launches one workgroup per compute unit of an
// MI355X, fewer when a workgroup would get under this many chunks.
constexpr int32_t kWgGroupTarget = 256;
constexpr int32_t kMinChunksPerGroup = 32;

struct Plan {
  bool ok;
  pkv_status status;
  int32_t group, partition, num_partitions;
  Family family;
  bool balanced;
  int waves;         // partitioned kernel: waves per workgroup
  int stream_waves;  // stream kernel: wavefronts launched
  int wg_groups;     // workgroup stream kernel: workgroups launched
  int wg_windows;    // and windows per workgroup the workspace has slots for
  // workspace: [counters | partition outputs | (max, sum) pairs]
  size_t counter_bytes, part_out_offset, part_ml_offset, workspace_bytes;
};

Plan plan_decode(const pkv_decode_dims* d, int32_t block_size) {
  Plan p = {};
  p.status = PKV_ERR_INVALID;
  if (d == nullptr) return p;
  if (d->num_seqs < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->head_dim < 1 ||
      block_size < 1 || d->num_blocks < 1 || d->max_blocks_per_seq < 1 || d->max_seq_len < 0 ||
      d->partition_size < 0)
    return p;
  if (d->num_q_heads % d->num_kv_heads != 0) return p;
  if (static_cast<int64_t>(d->max_seq_len) >
      static_cast<int64_t>(d->max_blocks_per_seq) * block_size)
    return p;
  if (d->out_dtype != PKV_DTYPE_BF16 && d->out_dtype != PKV_DTYPE_F32) return p;
  if (d->kernel != PKV_KERNEL_AUTO && d->kernel != PKV_KERNEL_MFMA &&
      d->kernel != PKV_KERNEL_GENERIC && d->kernel != PKV_KERNEL_STREAM &&
      d->kernel != PKV_KERNEL_STREAM_WG)
    return p;
  if (d->waves_per_group != 0 && d->waves_per_group != 1 && d->waves_per_group != 2 &&
      d->waves_per_group != 4)
    return p;
  if (d->balance_partitions != 0 && d->balance_partitions != 1) return p;
  if (d->stream_waves < 0 || d->stream_waves % 4 != 0) return p;
  if (d->no_shared_blocks != 0 && d->no_shared_blocks != 1) return p;
  if (d->num_seqs > kMaxGridYZ || d->num_kv_heads > kMaxGridYZ || d->num_q_heads > kMaxGridYZ)
    return (p.status = PKV_ERR_UNSUPPORTED, p);
  p.group = d->num_q_heads / d->num_kv_heads;
  p.partition = d->partition_size > 0 ? d->partition_size : default_partition(d, block_size);
  if (p.partition % block_size != 0) return p;
  const bool stream_ok =
      pkv::stream_shape_supported(d->head_dim, block_size, p.group, d->num_seqs);
  const bool mfma_ok =
      pkv::mfma_shape_supported(d->head_dim, block_size, p.group, p.partition);
  const bool generic_ok = pkv::generic_shape_supported(d->head_dim, block_size, p.group);
  const size_t units = static_cast<size_t>(d->num_seqs) * d->num_kv_heads;
  // chunks the call can hold at most
  const int64_t chunk_bound =
      static_cast<int64_t>(units) * ((static_cast<int64_t>(d->max_seq_len) + 31) / 32);
  // The workgroup stream kernel's launch: workgroups, and the windows each
  // walks when the chunk bound exceeds what its LDS holds at once.
  if (stream_ok) {
    const int nw = pkv::wg_waves_per_group(d->head_dim, d->no_shared_blocks != 0);
    int64_t groups = d->stream_waves > 0 ? (d->stream_waves + nw - 1) / nw : 0;
    if (groups == 0) {
      groups = (chunk_bound + kMinChunksPerGroup - 1) / kMinChunksPerGroup;
      if (groups > kWgGroupTarget) groups = kWgGroupTarget;
      if (groups < 1) groups = 1;
    }
    const pkv::WgLayout lay = pkv::wg_layout(d->head_dim, block_size, p.group, d->num_seqs, 1);
    if (lay.capacity >= 1) {
      const int64_t per_group = (chunk_bound + groups - 1) / groups;
      const int64_t windows = per_group <= lay.capacity ? 1 : (per_group + lay.capacity - 1) / lay.capacity;
      p.wg_groups = static_cast<int>(groups);
      p.wg_windows = static_cast<int>(windows);
    }
  }
  const bool wg_ok = stream_ok && p.wg_groups > 0;
  switch (d->kernel) {
    case PKV_KERNEL_STREAM:
      if (!stream_ok) return (p.status = PKV_ERR_UNSUPPORTED, p);
      p.family = kStream;
      break;
    case PKV_KERNEL_STREAM_WG:
      if (!wg_ok) return (p.status = PKV_ERR_UNSUPPORTED, p);
      p.family = kStreamWg;
      break;
    case PKV_KERNEL_MFMA:
      if (!mfma_ok) return (p.status = PKV_ERR_UNSUPPORTED, p);
      p.family = kMfma;
      break;
    case PKV_KERNEL_GENERIC:
      if (!generic_ok) return (p.status = PKV_ERR_UNSUPPORTED, p);
      p.family = kGeneric;
      break;
    default:
      // the workgroup kernel when one window per workgroup holds the call
      if (d->partition_size == 0 && wg_ok && p.wg_windows == 1)
        p.family = kStreamWg;
      else if (d->partition_size == 0 && stream_ok)
        p.family = kStream;
      else if (mfma_ok)
        p.family = kMfma;
      else if (generic_ok)
        p.family = kGeneric;
      else
        return (p.status = PKV_ERR_UNSUPPORTED, p);
  }
  const size_t counter_bytes = round_up(units * sizeof(uint32_t), kAlign);
  if (p.family == kStream || p.family == kStreamWg) {
    // wavefronts (stream kernel) or windows (workgroup kernel) that share the
    // chunks: each can publish one piece more than there are units
    int64_t wv = d->stream_waves;
    if (wv == 0) {
      wv = (chunk_bound + kMinChunksPerWave - 1) / kMinChunksPerWave;
      wv = wv < stream_wave_target(d->head_dim) ? wv : stream_wave_target(d->head_dim);
      wv = (wv + 3) / 4 * 4;
      if (wv < 4) wv = 4;
    }
    p.stream_waves = static_cast<int>(wv);
    p.num_partitions = 1;
    // [counters | per-piece (acc) slots | per-piece (max, sum) slots]
    const size_t slots =
        units + (p.family == kStream ? static_cast<size_t>(p.stream_waves)
                                     : static_cast<size_t>(p.wg_groups) * p.wg_windows);
    p.counter_bytes = counter_bytes;
    p.part_out_offset = p.counter_bytes;
    p.part_ml_offset = p.part_out_offset +
                       round_up(slots * p.group * d->head_dim * sizeof(float), kAlign);
    p.workspace_bytes = p.part_ml_offset + round_up(slots * p.group * 2 * sizeof(float), kAlign);
  } else {
    // waves per workgroup: each wave should own at least two 32-token chunks
    if (p.family == kMfma) {
      const int chunks = p.partition / 32;
      p.waves = d->waves_per_group != 0 ? d->waves_per_group
                                        : (chunks >= 8 ? 4 : (chunks >= 4 ? 2 : 1));
    }
    // the matrix-core kernel balances partitions when asked to
    p.balanced = p.family == kMfma && d->balance_partitions == 1;
    const int64_t np = (static_cast<int64_t>(d->max_seq_len) + p.partition - 1) / p.partition;
    p.num_partitions = static_cast<int32_t>(np < 1 ? 1 : np);
    if (p.num_partitions > 1) {
      // [counters | partition outputs | (max, sum) pairs]
      const size_t rows = static_cast<size_t>(d->num_seqs) * d->num_q_heads * p.num_partitions;
      p.counter_bytes = counter_bytes;
      p.part_out_offset = p.counter_bytes;
      p.part_ml_offset = p.part_out_offset + round_up(rows * d->head_dim * sizeof(float), kAlign);
      p.workspace_bytes = p.part_ml_offset + round_up(rows * 2 * sizeof(float), kAlign);
    }
  }
  p.ok = true;
  p.status = PKV_OK;
  return p;
}

pkv_status hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

}  // namespace

extern "C" {

int32_t pkv_abi_version(void) { return (kAbiMajor << 16) | kAbiMinor; }

const char* pkv_status_string(int32_t status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID: return "PKV_ERR_INVALID: invalid argument";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED: shape or option not implemented";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE: workspace missing or too small";
    case PKV_ERR_HIP: return "PKV_ERR_HIP: HIP runtime or launch error";
    default: return "unknown pkv_status";
  }
}

size_t pkv_decode_workspace_size(const pkv_decode_dims* dims, int32_t block_size) {
  const Plan p = plan_decode(dims, block_size);
  if (!p.ok) return static_cast<size_t>(-1);
  return p.workspace_bytes;
}

size_t pkv_decode_workspace_zeroed_bytes(const pkv_decode_dims* dims, int32_t block_size) {
  const Plan p = plan_decode(dims, block_size);
  if (!p.ok) return static_cast<size_t>(-1);
  return p.counter_bytes;
}

int32_t pkv_decode_plan_kernel(const pkv_decode_dims* dims, int32_t block_size) {
  const Plan p = plan_decode(dims, block_size);
  if (!p.ok) return -1;
  switch (p.family) {
    case kStreamWg: return PKV_KERNEL_STREAM_WG;
    case kStream: return PKV_KERNEL_STREAM;
    case kMfma: return PKV_KERNEL_MFMA;
    default: return PKV_KERNEL_GENERIC;
  }
}

}  // extern "C"

namespace pkv {

// Shared by the decode entry points; k_new / v_new are null for a plain decode.
pkv_status decode_entry(const void* q, const void* k_new, const void* v_new, const void* k_cache,
                       const void* v_cache, const int32_t* block_tables, const int32_t* seq_lens,
                       int32_t block_size, float scale, void* out, const pkv_decode_dims* dims,
                       void* workspace, size_t workspace_bytes, void* stream) {
  const Plan p = plan_decode(dims, block_size);
  if (!p.ok) return p.status;
  if (dims->num_seqs == 0) return PKV_OK;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || block_tables == nullptr ||
      seq_lens == nullptr || out == nullptr)
    return PKV_ERR_INVALID;
  const bool append = k_new != nullptr || v_new != nullptr;
  if (append && (k_new == nullptr || v_new == nullptr || dims->head_dim % 8 != 0 ||
                 !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
                 !aligned16(v_cache)))
    return PKV_ERR_INVALID;
  if (!std::isfinite(scale) || !(scale > 0.f)) return PKV_ERR_INVALID;  // the kernels need scale > 0
  if (p.family != kGeneric && (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)))
    return PKV_ERR_INVALID;
  if (p.workspace_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < p.workspace_bytes) return PKV_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return PKV_ERR_WORKSPACE;
  }
  pkv::DecodeLaunch a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.num_seqs = dims->num_seqs;
  a.prm.num_seqs = dims->num_seqs;
  a.prm.num_q_heads = dims->num_q_heads;
  a.prm.num_kv_heads = dims->num_kv_heads;
  a.prm.group = p.group;
  a.prm.head_dim = dims->head_dim;
  a.prm.block_size = block_size;
  a.prm.max_blocks_per_seq = dims->max_blocks_per_seq;
  a.prm.partition_size = p.partition;
  a.prm.balanced = p.balanced ? 1 : 0;
  a.prm.num_partitions = p.num_partitions;
  a.prm.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634074);
  a.prm.out_f32 = dims->out_dtype == PKV_DTYPE_F32 ? 1 : 0;
  a.prm.stream_kv = dims->no_shared_blocks;
  a.prm.out = out;
  if (p.workspace_bytes > 0) {
    char* ws = static_cast<char*>(workspace);
    a.prm.counters = reinterpret_cast<uint32_t*>(ws);
    a.prm.part_out = reinterpret_cast<float*>(ws + p.part_out_offset);
    a.prm.part_lse = reinterpret_cast<float*>(ws + p.part_ml_offset);
    a.prm.part_ml = reinterpret_cast<float*>(ws + p.part_ml_offset);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* kc_w = static_cast<uint16_t*>(const_cast<void*>(k_cache));
  uint16_t* vc_w = static_cast<uint16_t*>(const_cast<void*>(v_cache));
  if (append && (p.family == kStream || p.family == kStreamWg)) {
    // one launch: the wavefront that folds a unit's last chunk writes the new
    // token and uses it in place of the slot's old contents
    a.prm.k_new = static_cast<const uint16_t*>(k_new);
    a.prm.v_new = static_cast<const uint16_t*>(v_new);
    a.prm.k_cache_w = kc_w;
    a.prm.v_cache_w = vc_w;
  } else if (append) {
    const hipError_t e = pkv::launch_append_tokens(
        static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), block_tables,
        seq_lens, dims->num_seqs, dims->max_blocks_per_seq, dims->num_kv_heads, dims->head_dim,
        kc_w, vc_w, block_size, s);
    if (e != hipSuccess) return PKV_ERR_HIP;
  }
  switch (p.family) {
    case kStream: return hip_status(pkv::launch_decode_stream(a, p.stream_waves, s));
    case kStreamWg:
      return hip_status(pkv::launch_decode_wg(a, p.wg_groups, p.wg_windows, s));
    case kMfma: return hip_status(pkv::launch_decode_mfma(a, p.waves, s));
    default: return hip_status(pkv::launch_decode_generic(a, s));
  }
}

}  // namespace pkv

extern "C" {

pkv_status pkv_paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* seq_lens,
                                      int32_t block_size, float scale, void* out,
                                      const pkv_decode_dims* dims, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return pkv::decode_entry(q, nullptr, nullptr, k_cache, v_cache, block_tables, seq_lens, block_size,
                     scale, out, dims, workspace, workspace_bytes, stream);
}

pkv_status pkv_paged_attention_decode_append(const void* q, const void* k_new, const void* v_new,
                                             void* k_cache, void* v_cache,
                                             const int32_t* block_tables,
                                             const int32_t* seq_lens, int32_t block_size,
                                             float scale, void* out, const pkv_decode_dims* dims,
                                             void* workspace, size_t workspace_bytes,
                                             void* stream) {
  if (k_new == nullptr || v_new == nullptr) {
    const Plan p = plan_decode(dims, block_size);
    if (!p.ok) return p.status;
    return dims->num_seqs == 0 ? PKV_OK : PKV_ERR_INVALID;
  }
  return pkv::decode_entry(q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens, block_size, scale,
                     out, dims, workspace, workspace_bytes, stream);
}

pkv_status pkv_reshape_and_cache(const void* k, const void* v, const int64_t* slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                 void* k_cache, void* v_cache, int32_t num_blocks,
                                 int32_t block_size, void* stream) {
  if (num_tokens < 0 || num_kv_heads < 1 || head_dim < 8 || head_dim % 8 != 0 ||
      num_blocks < 1 || block_size < 1)
    return PKV_ERR_INVALID;
  if (num_tokens == 0) return PKV_OK;
  if (k == nullptr || v == nullptr || slot_mapping == nullptr || k_cache == nullptr ||
      v_cache == nullptr)
    return PKV_ERR_INVALID;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_ERR_INVALID;
  return hip_status(pkv::launch_reshape_and_cache(
      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), slot_mapping, num_tokens,
      num_kv_heads, head_dim, static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
      block_size, static_cast<hipStream_t>(stream)));
}

pkv_status pkv_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                           const int32_t* block_pairs, int32_t num_pairs, int64_t block_bytes,
                           void* stream) {
  if (num_pairs < 0 || num_layers < 1 || num_layers > pkv::kMaxCopyLayers || block_bytes <= 0 ||
      block_bytes % 16 != 0)
    return PKV_ERR_INVALID;
  if (num_pairs == 0) return PKV_OK;
  if (num_pairs > 0x7FFFFFFF / 2 || k_caches == nullptr || v_caches == nullptr ||
      block_pairs == nullptr)
    return PKV_ERR_INVALID;
  for (int32_t l = 0; l < num_layers; ++l)
    if (k_caches[l] == nullptr || v_caches[l] == nullptr || !aligned16(k_caches[l]) ||
        !aligned16(v_caches[l]))
      return PKV_ERR_INVALID;
  return hip_status(pkv::launch_copy_blocks(k_caches, v_caches, num_layers, block_pairs,
                                            num_pairs, block_bytes,
                                            static_cast<hipStream_t>(stream)));
}

pkv_status pkv_check_decode_inputs(const int32_t* block_tables, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t max_blocks_per_seq,
                                   int32_t num_blocks, int32_t block_size, int32_t max_seq_len,
                                   int32_t* flags, void* stream) {
  if (flags == nullptr || num_seqs < 0 || max_blocks_per_seq < 1 || num_blocks < 1 ||
      block_size < 1 || max_seq_len < 0)
    return PKV_ERR_INVALID;
  if (num_seqs > 0 && (block_tables == nullptr || seq_lens == nullptr)) return PKV_ERR_INVALID;
  const int64_t cap = static_cast<int64_t>(max_blocks_per_seq) * block_size;
  const int32_t max_len = static_cast<int32_t>(max_seq_len < cap ? max_seq_len : cap);
  return hip_status(pkv::launch_check_tables(block_tables, seq_lens, num_seqs, max_blocks_per_seq,
                                             num_blocks, block_size, max_len, flags,
                                             static_cast<hipStream_t>(stream)));
}

pkv_status pkv_check_slot_mapping(const int64_t* slot_mapping, int32_t num_tokens,
                                  int32_t num_blocks, int32_t block_size, int32_t* flags,
                                  void* stream) {
  if (flags == nullptr || num_tokens < 0 || num_blocks < 1 || block_size < 1)
    return PKV_ERR_INVALID;
  if (num_tokens > 0 && slot_mapping == nullptr) return PKV_ERR_INVALID;
  return hip_status(pkv::launch_check_slots(slot_mapping, num_tokens,
                                            static_cast<int64_t>(num_blocks) * block_size, flags,
                                            static_cast<hipStream_t>(stream)));
}

pkv_status pkv_check_block_pairs(const int32_t* block_pairs, int32_t num_pairs,
                                 int32_t num_blocks, int32_t* flags, void* stream) {
  if (flags == nullptr || num_pairs < 0 || num_pairs > 0x7FFFFFFF / 2 || num_blocks < 1)
    return PKV_ERR_INVALID;
  if (num_pairs > 0 && block_pairs == nullptr) return PKV_ERR_INVALID;
  return hip_status(pkv::launch_check_pairs(block_pairs, num_pairs, num_blocks, flags,
                                            static_cast<hipStream_t>(stream)));
}

pkv_status pkv_merge_attention_states(const float* part_out, const float* part_lse,
                                      int32_t num_rows, int32_t num_parts, int32_t head_dim,
                                      void* out, pkv_dtype out_dtype, void* stream) {
  if (num_rows < 0 || num_parts < 1 || head_dim < 1 || head_dim > 256) return PKV_ERR_INVALID;
  if (out_dtype != PKV_DTYPE_BF16 && out_dtype != PKV_DTYPE_F32) return PKV_ERR_INVALID;
  if (num_rows == 0) return PKV_OK;
  if (part_out == nullptr || part_lse == nullptr || out == nullptr) return PKV_ERR_INVALID;
  return hip_status(pkv::launch_merge(part_out, part_lse, num_rows, num_parts, num_parts,
                                      head_dim, nullptr, 1, 1, out,
                                      out_dtype == PKV_DTYPE_F32 ? 1 : 0,
                                      static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Shared-prefix decode: items and workspace regions for the host bounds.
struct CascadePlan {
  bool ok;
  pkv_status status;
  int32_t group;
  int64_t max_pre_items, max_suf_items;
  int32_t waves;
  int32_t use_wg, members_per_task, wg_grid, wg_chunks;  // the one-launch workgroup form
  // workspace: [pre_acc | pre_ml | suf_acc | suf_ml | tables]
  size_t pre_ml_offset, suf_acc_offset, suf_ml_offset, tables_offset, workspace_bytes;
};

CascadePlan plan_cascade(const pkv_decode_dims* d, int32_t num_groups, int32_t max_prefix_len,
                         int32_t block_size) {
  CascadePlan p = {};
  p.status = PKV_ERR_INVALID;
  if (d == nullptr) return p;
  if (d->num_seqs < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->head_dim < 1 ||
      block_size < 1 || d->num_blocks < 1 || d->max_blocks_per_seq < 1 || d->max_seq_len < 0)
    return p;
  if (d->num_q_heads % d->num_kv_heads != 0) return p;
  if (static_cast<int64_t>(d->max_seq_len) >
      static_cast<int64_t>(d->max_blocks_per_seq) * block_size)
    return p;
  if (d->out_dtype != PKV_DTYPE_BF16 && d->out_dtype != PKV_DTYPE_F32) return p;
  if (num_groups < 0 || (d->num_seqs > 0 && (num_groups < 1 || num_groups > d->num_seqs)))
    return p;
  if (max_prefix_len < 0 || max_prefix_len > d->max_seq_len) return p;
  if (d->kernel < PKV_KERNEL_AUTO || d->kernel > PKV_KERNEL_STREAM_WG) return p;
  p.group = d->num_q_heads / d->num_kv_heads;
  if (!pkv::cascade_shape_supported(d->head_dim, block_size, p.group, d->num_seqs))
    return (p.status = PKV_ERR_UNSUPPORTED, p);
  const int64_t S = d->num_seqs, NG = num_groups, Hkv = d->num_kv_heads, G = p.group;
  const int64_t D = d->head_dim;
  auto div_up = [](int64_t a, int64_t b) { return (a + b - 1) / b; };
  const int64_t seg_p = div_up(div_up(max_prefix_len, 32), pkv::kCascadePrefixChunks);
  const int64_t seg_s = div_up(div_up(d->max_seq_len, 32), pkv::kCascadeSuffixChunks);
  // row blocks over all groups: sum_g ceil(F_g G / rows) <= NG + ceil(S G / rows)
  const int64_t rows = pkv::kCascadeRows;
  p.max_pre_items = Hkv * seg_p * (NG + div_up(S * G, rows));
  p.max_suf_items = S * Hkv * seg_s;
  if (p.max_pre_items + p.max_suf_items > 0x7FFFFFFF) return (p.status = PKV_ERR_UNSUPPORTED, p);
  // launch 1: every wavefront resident on an MI355X (2 per SIMD at head_dim 64,
  // 1 at 128), fewer when there are fewer items
  const int64_t target = D <= 64 ? 2048 : 1024;
  int64_t waves = p.max_pre_items + p.max_suf_items;
  waves = waves < target ? waves : target;
  waves = (waves + 3) / 4 * 4;
  p.waves = static_cast<int32_t>(waves < 4 ? 4 : waves);
  const size_t pre_acc = round_up(static_cast<size_t>(p.max_pre_items) * rows * D * 4, kAlign);
  const size_t pre_ml = round_up(static_cast<size_t>(p.max_pre_items) * rows * 2 * 4, kAlign);
  const size_t suf_acc = round_up(static_cast<size_t>(p.max_suf_items) * G * D * 4, kAlign);
  const size_t suf_ml = round_up(static_cast<size_t>(p.max_suf_items) * G * 2 * 4, kAlign);
  const size_t tables = round_up(static_cast<size_t>(pkv::kCascadeTableHead + 8 * S) * 4, kAlign);
  p.pre_ml_offset = pre_acc;
  p.suf_acc_offset = p.pre_ml_offset + pre_ml;
  p.suf_ml_offset = p.suf_acc_offset + suf_acc;
  p.tables_offset = p.suf_ml_offset + suf_ml;
  p.workspace_bytes = p.tables_offset + tables;
  // The one-launch workgroup form: a task is (group, KV head, block of
  // members); members per task as many as one 16-row tile holds, halved
  // while the tasks would not give every compute unit a workgroup.  It runs
  // when a task's chunks (the longest prefix plus its members' longest
  // suffixes) fit the records in LDS.
  {
    const int64_t kUnits = 256;  // compute units of an MI355X
    int64_t mpt = pkv::kCascadeRows / G;
    while (mpt > 1 && Hkv * div_up(S, mpt) < kUnits) mpt /= 2;
    const int64_t bound = div_up(max_prefix_len, 32) + mpt * div_up(d->max_seq_len, 32);
    const pkv::CascadeWgLayout lay = pkv::cascade_wg_layout(
        d->head_dim, block_size, static_cast<int>(S), static_cast<int>(NG), 0);
    const bool fits = bound >= 1 && bound <= lay.capacity;
    p.wg_chunks = static_cast<int32_t>(fits ? bound : 0);
    if (d->kernel == PKV_KERNEL_STREAM_WG && !fits) return (p.status = PKV_ERR_UNSUPPORTED, p);
    p.use_wg = (d->kernel != PKV_KERNEL_MFMA && fits) ? 1 : 0;
    p.members_per_task = static_cast<int32_t>(mpt);
    // at least the tasks of any grouping, one workgroup per compute unit at
    // most (each asks for the whole LDS, so the dispatcher spreads them over
    // all units; stacking two on a unit while others idle measured slower)
    const int64_t tasks = Hkv * (NG + div_up(S, mpt));
    int64_t grid = tasks < kUnits ? tasks : kUnits;
    grid = (grid + 7) / 8 * 8;
    p.wg_grid = static_cast<int32_t>(grid < 8 ? 8 : grid);
  }
  p.ok = true;
  p.status = PKV_OK;
  return p;
}

}  // namespace

extern "C" {

int32_t pkv_cascade_plan_kernel(const pkv_decode_dims* dims, int32_t num_groups,
                                int32_t max_prefix_len, int32_t block_size) {
  const CascadePlan p = plan_cascade(dims, num_groups, max_prefix_len, block_size);
  if (!p.ok) return -1;
  return p.use_wg ? PKV_KERNEL_STREAM_WG : PKV_KERNEL_MFMA;
}

size_t pkv_cascade_workspace_size(const pkv_decode_dims* dims, int32_t num_groups,
                                  int32_t max_prefix_len, int32_t block_size) {
  const CascadePlan p = plan_cascade(dims, num_groups, max_prefix_len, block_size);
  if (!p.ok) return static_cast<size_t>(-1);
  return p.workspace_bytes;
}

pkv_status pkv_cascade_decode(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* seq_lens,
                              const int32_t* group_starts, const int32_t* prefix_lens,
                              int32_t num_groups, int32_t max_prefix_len, int32_t block_size,
                              float scale, void* out, const pkv_decode_dims* dims,
                              void* workspace, size_t workspace_bytes, void* stream) {
  const CascadePlan p = plan_cascade(dims, num_groups, max_prefix_len, block_size);
  if (!p.ok) return p.status;
  if (dims->num_seqs == 0) return PKV_OK;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || block_tables == nullptr ||
      seq_lens == nullptr || group_starts == nullptr || prefix_lens == nullptr || out == nullptr)
    return PKV_ERR_INVALID;
  if (!std::isfinite(scale) || !(scale > 0.f)) return PKV_ERR_INVALID;  // the kernels need scale > 0
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID;
  if (workspace == nullptr || workspace_bytes < p.workspace_bytes) return PKV_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return PKV_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  pkv::CascadeLaunch a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.group_starts = group_starts;
  a.prefix_lens = prefix_lens;
  a.num_seqs = dims->num_seqs;
  a.num_groups = num_groups;
  a.num_q_heads = dims->num_q_heads;
  a.num_kv_heads = dims->num_kv_heads;
  a.group = p.group;
  a.head_dim = dims->head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = dims->max_blocks_per_seq;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634074);
  a.out_f32 = dims->out_dtype == PKV_DTYPE_F32 ? 1 : 0;
  a.out = out;
  a.pre_acc = reinterpret_cast<float*>(ws);
  a.pre_ml = reinterpret_cast<float*>(ws + p.pre_ml_offset);
  a.suf_acc = reinterpret_cast<float*>(ws + p.suf_acc_offset);
  a.suf_ml = reinterpret_cast<float*>(ws + p.suf_ml_offset);
  a.tables = reinterpret_cast<int32_t*>(ws + p.tables_offset);
  a.max_prefix_len = max_prefix_len;
  a.max_seq_len = dims->max_seq_len;
  a.max_pre_items = p.max_pre_items;
  a.max_suf_items = p.max_suf_items;
  a.waves = p.waves;
  a.use_wg = p.use_wg;
  a.members_per_task = p.members_per_task;
  a.wg_grid = p.wg_grid;
  a.wg_chunks = p.wg_chunks;
  return hip_status(pkv::launch_cascade(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

extern "C" {

pkv_status pkv_paged_prefill(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* seq_lens,
                             const int32_t* cu_q_lens, int32_t num_tokens, int32_t max_q_len,
                             int32_t block_size, float scale, void* out,
                             const pkv_decode_dims* d, void* stream) {
  if (d == nullptr) return PKV_ERR_INVALID;
  if (d->num_seqs < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->head_dim < 1 ||
      block_size < 1 || d->num_blocks < 1 || d->max_blocks_per_seq < 1 || d->max_seq_len < 0 ||
      num_tokens < 0 || max_q_len < 0 || max_q_len > d->max_seq_len)
    return PKV_ERR_INVALID;
  if (d->num_q_heads % d->num_kv_heads != 0) return PKV_ERR_INVALID;
  if (static_cast<int64_t>(d->max_seq_len) >
      static_cast<int64_t>(d->max_blocks_per_seq) * block_size)
    return PKV_ERR_INVALID;
  if (d->out_dtype != PKV_DTYPE_BF16 && d->out_dtype != PKV_DTYPE_F32) return PKV_ERR_INVALID;
  const int32_t group = d->num_q_heads / d->num_kv_heads;
  if (!pkv::prefill_shape_supported(d->head_dim, block_size, group) ||
      d->num_seqs > kMaxGridYZ || d->num_kv_heads > kMaxGridYZ)
    return PKV_ERR_UNSUPPORTED;
  if (d->num_seqs == 0 || num_tokens == 0 || max_q_len == 0) return PKV_OK;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || block_tables == nullptr ||
      seq_lens == nullptr || cu_q_lens == nullptr || out == nullptr)
    return PKV_ERR_INVALID;
  if (!std::isfinite(scale) || !(scale > 0.f)) return PKV_ERR_INVALID;  // the kernels need scale > 0
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID;
  pkv::PrefillLaunch a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.cu_q_lens = cu_q_lens;
  a.num_seqs = d->num_seqs;
  a.num_tokens = num_tokens;
  a.num_q_heads = d->num_q_heads;
  a.num_kv_heads = d->num_kv_heads;
  a.group = group;
  a.head_dim = d->head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = d->max_blocks_per_seq;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634074);
  a.out_f32 = d->out_dtype == PKV_DTYPE_F32 ? 1 : 0;
  a.out = out;
  return hip_status(pkv::launch_prefill(a, max_q_len, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// The swap entry points' checks: the same as copy_blocks for the caches, and
// the host buffer must be pinned host memory the device can address.
pkv_status swap_impl(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                     const int32_t* block_ids, int32_t n, int64_t block_bytes, void* host,
                     int to_host, void* stream) {
  if (n < 0 || num_layers < 1 || num_layers > pkv::kMaxCopyLayers || block_bytes <= 0 ||
      block_bytes % 16 != 0)
    return PKV_ERR_INVALID;
  if (n == 0) return PKV_OK;
  if (n > 0x7FFFFFFF / 2 || k_caches == nullptr || v_caches == nullptr || block_ids == nullptr ||
      host == nullptr || !aligned16(host))
    return PKV_ERR_INVALID;
  for (int32_t l = 0; l < num_layers; ++l)
    if (k_caches[l] == nullptr || v_caches[l] == nullptr || !aligned16(k_caches[l]) ||
        !aligned16(v_caches[l]))
      return PKV_ERR_INVALID;
  hipPointerAttribute_t attr = {};
  if (hipPointerGetAttributes(&attr, host) != hipSuccess) {
    (void)hipGetLastError();  // leave no error behind for the caller's next call
    return PKV_ERR_INVALID;
  }
  if (attr.type != hipMemoryTypeHost || attr.devicePointer == nullptr) return PKV_ERR_INVALID;
  return hip_status(pkv::launch_swap_blocks(k_caches, v_caches, num_layers, block_ids, n,
                                            block_bytes, attr.devicePointer, to_host,
                                            static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

pkv_status pkv_swap_out(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                        const int32_t* block_ids, int32_t num_ids, int64_t block_bytes,
                        void* host_buffer, void* stream) {
  return swap_impl(k_caches, v_caches, num_layers, block_ids, num_ids, block_bytes, host_buffer,
                   1, stream);
}

pkv_status pkv_swap_in(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                       const int32_t* block_ids, int32_t num_ids, int64_t block_bytes,
                       const void* host_buffer, void* stream) {
  return swap_impl(k_caches, v_caches, num_layers, block_ids, num_ids, block_bytes,
                   const_cast<void*>(host_buffer), 0, stream);
}

}  // extern "C"
