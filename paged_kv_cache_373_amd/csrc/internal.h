// internal.h - launchers shared by the kernel translation units and the C ABI
// layer.  Not part of the public interface (see include/pagedkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

// Everything a decode kernel needs besides the tensor pointers.
struct DecodeParams {
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;              // num_q_heads / num_kv_heads
  int32_t head_dim;
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int32_t partition_size;     // tokens per split-KV partition (the longest one when balanced)
  int32_t balanced;           // 1: a sequence's partitions share its 32-token chunks evenly
  int32_t num_partitions;     // grid extent over partitions = ceil(max_seq_len / partition_size)
  float scale_log2;           // scale * log2(e): scores live in base-2 units inside the kernels
  int32_t out_f32;            // 1: out is fp32, 0: out is bf16
  int32_t stream_kv;          // 1: no physical block is read by two sequences of the
                              // call, so the stream kernels read K/V non-temporally
  void* out;                  // [S, Hq, D]
  // Split-KV workspace.  Partitioned kernels (only when num_partitions > 1):
  // partition results per (sequence, q head, partition).  Stream kernels: one
  // slot of G heads per piece, [S * Hkv + waves] slots (per-wavefront ranges)
  // or [S * Hkv + windows] slots (workgroup windows).
  float* part_out;            // [S, Hq, num_partitions, D] partition outputs
  float* part_lse;            // [S, Hq, num_partitions] ln Z_r (vector kernel)
  float* part_ml;             // [S, Hq, num_partitions, 2] (max in base-2 units, sum)
                              // (matrix-core kernel; shares memory with part_lse)
  uint32_t* counters;         // [S, Hkv] finished partitions per (sequence, KV head);
                              // zero before and after every call
  // Decode step with append (stream kernel): each sequence's new token, at
  // position T_b - 1, is written to the slot its table gives and attended.
  const uint16_t* k_new;      // bf16 [S, Hkv, D], or null
  const uint16_t* v_new;      // bf16 [S, Hkv, D]
  uint16_t* k_cache_w;        // the caches, for the new tokens' writes
  uint16_t* v_cache_w;
};

struct DecodeLaunch {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  int32_t num_seqs;
  DecodeParams prm;
};

// The decode entry points' common body (in api.cpp): host checks, the plan,
// then the launch.  k_new / v_new are null for a plain decode.  `workspace`
// must satisfy the workspace contract of pkv_paged_attention_decode.
pkv_status decode_entry(const void* q, const void* k_new, const void* v_new, const void* k_cache,
                        const void* v_cache, const int32_t* block_tables,
                        const int32_t* seq_lens, int32_t block_size, float scale, void* out,
                        const pkv_decode_dims* dims, void* workspace, size_t workspace_bytes,
                        void* stream);

// Shapes the kernels are instantiated for.
bool mfma_shape_supported(int head_dim, int block_size, int group, int partition_size);
bool stream_shape_supported(int head_dim, int block_size, int group, int num_seqs);
bool generic_shape_supported(int head_dim, int block_size, int group);
int stream_waves_per_group();  // the stream kernel's wavefronts per workgroup

// Each launcher enqueues its kernel(s) on `stream` and returns the launch error.
hipError_t launch_decode_stream(const DecodeLaunch& a, int num_waves, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeLaunch& a, int waves, hipStream_t stream);
hipError_t launch_decode_generic(const DecodeLaunch& a, hipStream_t stream);

// Workgroup stream kernel.  One workgroup per compute unit holds
// wg_waves_per_group(head_dim, stream_kv) wavefronts; its LDS (dynamic shared memory) is
// carved as below, in 4-byte words, with room for `capacity` chunks a window.
constexpr int kWgLdsBytes = 160 * 1024;  // LDS a workgroup may use on gfx950
constexpr int kWgMaxCapacity = 1024;     // chunks a window holds at most
struct WgLayout {
  int32_t capacity;     // chunks per window
  int32_t max_windows;  // windows per workgroup the workspace has slots for
  int32_t off_len, off_pre, off_wsum, off_misc, off_rec, off_unit, off_list, off_acc, off_ml;
  int32_t words;        // total LDS words
};
int wg_waves_per_group(int head_dim, bool stream_kv);
WgLayout wg_layout(int head_dim, int block_size, int group, int num_seqs, int max_windows);
hipError_t launch_decode_wg(const DecodeLaunch& a, int num_groups, int max_windows,
                            hipStream_t stream);

// Split-KV merge.  With seq_lens != nullptr, row r = b * rows_per_seq + h
// merges ceil(seq_lens[b] / partition_size) partitions and rows that have at
// most one partition are skipped (their output was written directly);
// otherwise every row merges `num_parts` partitions.
hipError_t launch_merge(const float* part_out, const float* part_lse, int32_t num_rows,
                        int32_t part_stride, int32_t num_parts, int32_t head_dim,
                        const int32_t* seq_lens, int32_t rows_per_seq,
                        int32_t partition_size, void* out, int out_f32, hipStream_t stream);

// Writes k_new/v_new of sequence b (T_b >= 1) to the slot of position T_b - 1
// given by its block table; sequences with T_b == 0 are skipped.
hipError_t launch_append_tokens(const uint16_t* k_new, const uint16_t* v_new,
                                const int32_t* block_tables, const int32_t* seq_lens,
                                int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_kv_heads,
                                int32_t head_dim, uint16_t* k_cache, uint16_t* v_cache,
                                int32_t block_size, hipStream_t stream);

hipError_t launch_reshape_and_cache(const uint16_t* k, const uint16_t* v,
                                    const int64_t* slot_mapping, int32_t num_tokens,
                                    int32_t num_kv_heads, int32_t head_dim, uint16_t* k_cache,
                                    uint16_t* v_cache, int32_t block_size, hipStream_t stream);

constexpr int kMaxCopyLayers = 64;
// Swap: blocks block_ids[0..n) of every layer's K and V cache to (to_host = 1)
// or from (0) the host buffer, [layer][K|V][i] blocks back to back; host_dev
// is the buffer's device address.
hipError_t launch_swap_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                              const int32_t* block_ids, int32_t n, int64_t block_bytes,
                              void* host_dev, int to_host, hipStream_t stream);
hipError_t launch_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                              const int32_t* block_pairs, int32_t num_pairs,
                              int64_t block_bytes, hipStream_t stream);

// Shared-prefix (cascade) decode.  Groups are contiguous runs of sequences,
// group g = [group_starts[g], group_starts[g+1]), sharing their first
// prefix_lens[g] tokens (whole blocks).  Launch 1 folds items into partial
// states: a prefix item is kCascadePrefixChunks 32-token chunks of a group's
// prefix for one block of kCascadeRows query rows (member-major, G heads
// each), a suffix item is kCascadeSuffixChunks chunks of one sequence's tokens
// past the prefix.  Launch 2 merges, per (sequence, KV head), the partials of
// its group's prefix items and of its own suffix items.
constexpr int kCascadeRows = 16;           // query rows of a prefix item: one matrix-core tile
constexpr int kCascadePrefixChunks = 4;    // chunks per prefix item
constexpr int kCascadeSuffixChunks = 4;    // chunks per suffix item
constexpr int kCascadeMaxSeqs = 4096;      // sequences (and groups) per call
constexpr int kCascadeTableHead = 4;       // status word and padding before the item tables
struct CascadeLaunch {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* group_starts;  // [NG + 1]
  const int32_t* prefix_lens;   // [NG]
  int32_t num_seqs, num_groups, num_q_heads, num_kv_heads, group, head_dim, block_size;
  int32_t max_blocks_per_seq;
  float scale_log2;
  int32_t out_f32;
  void* out;
  float* pre_acc;   // [max_pre_items][kCascadeRows][D]
  float* pre_ml;    // [max_pre_items][kCascadeRows][max, sum]
  float* suf_acc;   // [max_suf_items][G][D]
  float* suf_ml;    // [max_suf_items][G][max, sum]
  int32_t* tables;  // [kCascadeTableHead + 8 S]: status, then per sequence its merge
                    // descriptor (first prefix item of its group, row blocks, prefix
                    // items per row block, member index, first suffix item, suffix
                    // items per head, 2 spare)
  int32_t max_prefix_len, max_seq_len;  // host bounds the device lengths are checked against
  int64_t max_pre_items, max_suf_items;
  int32_t waves;    // launch 1 wavefronts (a multiple of 4)
  // the one-launch workgroup form (used when use_wg): members per task and
  // the workgroups launched
  int32_t use_wg, members_per_task, wg_grid, wg_chunks;  // wg_chunks: records a task may need
};
// LDS of the workgroup form, in 4-byte words; capacity = chunk records a task
// may hold.
struct CascadeWgLayout {
  int32_t off_len, off_gs, off_pl, off_tpre, off_misc, off_rec, off_acc, off_ml;
  int32_t words, capacity;
};
bool cascade_shape_supported(int head_dim, int block_size, int group, int num_seqs);
// want_chunks (> 0) caps the records at what a task can need (0: as many as
// the LDS holds).
CascadeWgLayout cascade_wg_layout(int head_dim, int block_size, int num_seqs, int num_groups,
                                  int64_t want_chunks);
hipError_t launch_cascade(const CascadeLaunch& a, hipStream_t stream);

// Paged prefill (causal multi-query attention).  The new tokens of sequence
// b are rows cu_q_lens[b] .. cu_q_lens[b+1]-1 of q and out, the last q_len_b
// of its seq_lens[b] cached tokens.
struct PrefillLaunch {
  const uint16_t* q;           // bf16 [num_tokens, Hq, D]
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;     // [S]
  const int32_t* cu_q_lens;    // [S + 1]
  int32_t num_seqs, num_tokens, num_q_heads, num_kv_heads, group, head_dim, block_size;
  int32_t max_blocks_per_seq;
  float scale_log2;
  int32_t out_f32;
  void* out;                   // [num_tokens, Hq, D]
  int32_t wg_per_pair;         // workgroups per (sequence, KV head) (set by the launcher)
};
bool prefill_shape_supported(int head_dim, int block_size, int group);

// Checkers of device-resident inputs (check.hip); each clears *flags, then ORs
// the violations it finds into it.
hipError_t launch_check_tables(const int32_t* block_tables, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                               int32_t block_size, int32_t max_len, int32_t* flags,
                               hipStream_t stream);
hipError_t launch_check_slots(const int64_t* slot_mapping, int32_t num_tokens, int64_t num_slots,
                              int32_t* flags, hipStream_t stream);
hipError_t launch_check_pairs(const int32_t* block_pairs, int32_t num_pairs, int32_t num_blocks,
                              int32_t* flags, hipStream_t stream);
hipError_t launch_prefill(const PrefillLaunch& a, int max_q_len, hipStream_t stream);

}  // namespace pkv
