/*
 * pagedkv.h - C ABI of the MI355X (gfx950) paged decode-attention library.
 *
 * Sources this interface follows (cited by short key throughout):
 *   [ITH] iThome ithelp article 10405755 on PagedAttention
 *         (ithelp.ithome.com.tw/articles/10405755).
 *   [PU]  Fanyi Pu, "Infra: PagedAttention" (pufanyi.com, ml-revisit/infra).
 *   [AK]  "Paged attention story" (akira.ipas-ai.com, stand-up-comedy series).
 *
 * The library implements the decode-time hot path those pages describe: a KV
 * cache cut into fixed-size physical blocks, reached through a per-sequence
 * block table, read in place by the attention kernel; a slot-mapped writer
 * that puts a new token's K/V into its tail slot; and a whole-block copier for
 * copy-on-write of a shared, partly filled tail block.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers unless an argument says HOST.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only enqueues work on that stream and returns; nothing
 *    synchronises.  Results are visible after the stream is synchronised.
 *  - The library allocates no memory, keeps no pointer after a call returns
 *    and has no mutable global state: calls on different streams with
 *    disjoint outputs and workspaces may run concurrently.
 *  - bf16 is IEEE bfloat16 (1 sign, 8 exponent, 7 fraction bits) stored as
 *    16-bit words; fp32 is IEEE binary32.  Rounding to bf16 is
 *    round-to-nearest-even.
 *  - Host-checkable preconditions are verified before any HIP call; a
 *    violation returns an error status and enqueues nothing.  Values that
 *    live in device memory (table entries, lengths, slots) are the caller's
 *    contract: out-of-range values there are undefined behaviour, exactly
 *    like an out-of-range index into any device array.
 *
 * Cache layout (one layer; a multi-layer model holds one pair per layer)
 * ----------------------------------------------------------------------
 *   P   = num_blocks      physical blocks in the pool      [PU §按 Block 分配]
 *   B   = block_size      tokens per block
 *   Hkv = num_kv_heads,  D = head_dim
 *
 *   k_cache : bf16 [P, Hkv, B, D]  element (p,h,o,d) at ((p*Hkv + h)*B + o)*D + d
 *   v_cache : bf16 [P, Hkv, D, B]  element (p,h,o,d) at ((p*Hkv + h)*D + d)*B + o
 *
 * K keeps each token's head vector contiguous; V is stored transposed inside
 * a block so that a run of consecutive tokens of one feature is contiguous
 * (the operand order of the P.V contraction over tokens).  A (block, head)
 * tile of either tensor is one contiguous B*D*2-byte range.
 *
 * Slots [PU §KV Cache 为什么会浪费显存 defines a slot as the room for one
 * token's KV; §按 Block 分配 reads position t through logical block t/B and
 * in-block offset t%B]:  the token at position t of a sequence whose block
 * table row is bt lives in slot  s = bt[t / B] * B + t % B,  i.e. physical
 * block s / B, offset s % B.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID = -1,     /* null pointer, negative count, inconsistent sizes     */
  PKV_ERR_UNSUPPORTED = -2, /* a shape or option the kernels do not implement       */
  PKV_ERR_WORKSPACE = -3,   /* workspace pointer null or smaller than required      */
  PKV_ERR_HIP = -4          /* a HIP launch or runtime call reported an error       */
} pkv_status;

typedef enum { PKV_DTYPE_BF16 = 0, PKV_DTYPE_F32 = 1 } pkv_dtype;

/* Which decode kernel family runs.
 *   STREAM   matrix-core kernel that deals the call's (sequence, KV head,
 *            32-token chunk) work out evenly to a fixed set of wavefronts;
 *            head_dim 64 or 128, block_size 8/16/32, group <= 16,
 *            num_seqs <= 2048.  Ignores partition_size.
 *   STREAM_WG  the same work dealt out in equal windows to whole workgroups
 *            (one per compute unit; at head_dim 64, 5 wavefronts when the call
 *            declares no_shared_blocks, else 6; 4 at 128)
 *            whose wavefronts take the window's chunks one at a time, so they
 *            finish together; same shape limits.  A window holds as many
 *            chunks as the workgroup's LDS has slots for; when the chunk bound
 *            (from max_seq_len) needs more, each workgroup walks several
 *            windows.  Results do not depend on the timing of the wavefronts.
 *   MFMA     matrix-core kernel over split-KV partitions of partition_size
 *            tokens (a multiple of 32, at most 128 blocks); same head_dim,
 *            block_size and group limits.
 *   GENERIC  vector kernel: any head_dim <= 256, block_size >= 1, group.
 * AUTO picks STREAM_WG when partition_size is 0, the shape allows it and
 * one window per workgroup holds the chunk bound, else STREAM when
 * partition_size is 0 and the shape allows it, then MFMA, then GENERIC.  An explicit family whose limits the shape exceeds
 * gives PKV_ERR_UNSUPPORTED. */
typedef enum {
  PKV_KERNEL_AUTO = 0,
  PKV_KERNEL_MFMA = 1,
  PKV_KERNEL_GENERIC = 2,
  PKV_KERNEL_STREAM = 3,
  PKV_KERNEL_STREAM_WG = 4
} pkv_kernel;

/* Problem description for pkv_paged_attention_decode. */
typedef struct {
  int32_t num_seqs;           /* S  >= 0                                             */
  int32_t num_q_heads;        /* Hq >= 1                                             */
  int32_t num_kv_heads;       /* Hkv >= 1, Hq % Hkv == 0; group G = Hq / Hkv         */
  int32_t head_dim;           /* D                                                   */
  int32_t num_blocks;         /* P, blocks in the pool (bounds contract)             */
  int32_t max_blocks_per_seq; /* row stride (in entries) of block_tables, >= 1       */
  int32_t max_seq_len;        /* host-known bound on every seq_lens[b]; sizes the
                                 split-KV grid; <= max_blocks_per_seq * block_size   */
  int32_t partition_size;     /* tokens per split-KV partition, a multiple of
                                 block_size (and of 32 for the MFMA kernel);
                                 0 = library choice (balanced, see below)            */
  pkv_dtype out_dtype;        /* element type of `out`                               */
  pkv_kernel kernel;          /* kernel family, normally PKV_KERNEL_AUTO              */
  int32_t waves_per_group;    /* matrix-core kernel: wavefronts sharing a partition
                                 (1, 2 or 4); 0 = library choice; ignored otherwise  */
  int32_t balance_partitions; /* matrix-core kernel: 0 = every partition but a
                                 sequence's last holds exactly partition_size
                                 tokens; 1 = a sequence of T tokens is cut into
                                 ceil(T / partition_size) partitions that share
                                 its 32-token chunks evenly.  A library-chosen
                                 partition_size always balances.                     */
  int32_t stream_waves;       /* stream kernels: wavefronts launched, a multiple of 4
                                 (STREAM: each takes an equal share of the work;
                                 STREAM_WG: rounded up to whole workgroups, each
                                 taking an equal share); 0 = library choice          */
  int32_t no_shared_blocks;   /* 0 or 1.  1 declares that no physical block is read
                                 by two sequences of this call (no shared prefix, no
                                 fork sharing a block): the STREAM and STREAM_WG
                                 kernels then read K/V with non-temporal loads,
                                 which do not keep the lines in the caches [PU
                                 §共享前缀，分叉时 Copy-on-write: forks of one
                                 prompt point at the same blocks, which caching
                                 serves for every fork after the first].  Only a
                                 speed hint: results are identical either way.
                                 0 (ordinary loads) is always correct.  Ignored by
                                 the MFMA and GENERIC kernels.  (ABI 2.0; callers
                                 zero-initialise the whole struct.)                  */
} pkv_decode_dims;

/* Bytes of scratch that pkv_paged_attention_decode needs for `dims` and
 * `block_size`; 0 when no split-KV merge can be needed, (size_t)-1 when the
 * arguments are invalid.  The caller allocates it (device memory, 256-byte
 * aligned).  Layout: first a counter region of
 * pkv_decode_workspace_zeroed_bytes bytes (one 32-bit counter per
 * (sequence, KV head), padded), then per-partition results.  The counter
 * region must hold zero bytes when a call starts, and every call leaves it
 * zero when it completes; the rest of the workspace needs no initialisation
 * and holds garbage after a call.  So a workspace zero-filled once serves any
 * number of calls of one shape; before a call whose counter region is larger
 * than the last call's, zero the bytes up to the new size (the last call may
 * have left partial results there).  One workspace serves one call at a
 * time: calls that may overlap (on different streams) need different
 * workspaces. */
size_t pkv_decode_workspace_size(const pkv_decode_dims* dims, int32_t block_size);

/* The form pkv_cascade_decode runs for these arguments: PKV_KERNEL_STREAM_WG
 * (one launch) or PKV_KERNEL_MFMA (two launches); -1 when they are invalid
 * or unsupported. */
int32_t pkv_cascade_plan_kernel(const pkv_decode_dims* dims, int32_t num_groups,
                                int32_t max_prefix_len, int32_t block_size);
/* Leading bytes of the workspace that must be zero when
 * pkv_paged_attention_decode starts (and are zero again when it completes);
 * (size_t)-1 when the arguments are invalid. */
size_t pkv_decode_workspace_zeroed_bytes(const pkv_decode_dims* dims, int32_t block_size);

/* The kernel family pkv_paged_attention_decode runs for `dims` and
 * `block_size`: a pkv_kernel value other than PKV_KERNEL_AUTO (the family
 * AUTO resolves to, or the explicit one), or -1 when the arguments are invalid
 * or the requested family does not support the shape.  Touches no device. */
int32_t pkv_decode_plan_kernel(const pkv_decode_dims* dims, int32_t block_size);

/* Single-query paged decode attention with GQA [ITH §PagedAttention 的核心想法:
 * the attention formula is unchanged, the kernel looks the block table up and
 * reads K,V where the physical blocks are; PU §按 Block 分配: softmax
 * normalises over every token the query can see, s_i = q.k_i / sqrt(d) (the
 * scale is an argument here), and per-segment results merge by
 * o = (Z1 o1 + Z2 o2) / (Z1 + Z2) after rescaling to a common maximum].
 *
 *   q            bf16 [S, Hq, D] contiguous; the query of the one position
 *                being decoded per sequence.
 *   k_cache      bf16, layout above.     v_cache  bf16, layout above.
 *   block_tables int32 [S, max_blocks_per_seq]; row b holds physical block ids
 *                for logical blocks 0 .. ceil(T_b/B)-1, each in [0, P).  Later
 *                entries are never read.
 *   seq_lens     int32 [S]; T_b = number of cached tokens of sequence b,
 *                including the token being decoded (whose K/V must already be
 *                in the cache).  0 <= T_b <= dims->max_seq_len.
 *   block_size   B >= 1.   scale  multiplier of q.k (normally 1/sqrt(D)), finite and > 0
 *                (PKV_ERR_INVALID otherwise; every call taking a scale).
 *   out          [S, Hq, D] contiguous, dims->out_dtype.  Query head h reads
 *                KV head h / G (consecutive query heads share a KV head).
 *                A sequence with T_b == 0 gets an all-zero row.
 *   workspace    device scratch of at least pkv_decode_workspace_size bytes
 *                whose counter region is zero (see above); may be NULL when
 *                that size is 0.
 * Slots of positions >= T_b in a sequence's last block, and blocks no table
 * row references, may hold any bits, NaN included: they never reach `out`
 * (the kernels select them away; they never multiply them by zero).
 * q, k_cache and v_cache must be 16-byte aligned (PKV_ERR_INVALID otherwise,
 * for the matrix-core kernel).
 * Returns PKV_OK, or an error status with nothing enqueued. */
pkv_status pkv_paged_attention_decode(const void* q, const void* k_cache,
                                      const void* v_cache,
                                      const int32_t* block_tables,
                                      const int32_t* seq_lens, int32_t block_size,
                                      float scale, void* out,
                                      const pkv_decode_dims* dims, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* One decode step in one call: the cache write of each sequence's new token
 * followed by paged decode attention over its T_b tokens [ITH §手動畫一次
 * block table: a new token fills the tail block's next slot; PU §按 Block
 * 分配: position t lives at offset t % B of the block its table gives for
 * logical block t / B].  Equivalent to pkv_reshape_and_cache with
 * slot_mapping[b] = bt[b][(T_b - 1) / B] * B + (T_b - 1) % B, followed by
 * pkv_paged_attention_decode with the same arguments; the stream kernel does
 * both in one launch (the wavefront that folds a sequence's last chunk writes
 * the token and uses it), the other kernel families run a small write kernel
 * first.
 *   k_new, v_new  bf16 [S, Hkv, D] contiguous, 16-byte aligned; the K and V of
 *                 position T_b - 1 of every sequence.  Sequences with T_b == 0
 *                 are left alone (nothing is written; their output row is 0).
 *   k_cache, v_cache  written (one slot per sequence and KV head) and read.
 * The block holding position T_b - 1 must belong to sequence b alone (copy a
 * shared tail with pkv_copy_blocks first).  Other arguments, the workspace
 * and the return codes as for pkv_paged_attention_decode. */
pkv_status pkv_paged_attention_decode_append(const void* q, const void* k_new, const void* v_new,
                                             void* k_cache, void* v_cache,
                                             const int32_t* block_tables,
                                             const int32_t* seq_lens, int32_t block_size,
                                             float scale, void* out, const pkv_decode_dims* dims,
                                             void* workspace, size_t workspace_bytes,
                                             void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * call as pkv_paged_attention_decode, same arguments and results, except that
 * its split-KV scratch is a fixed array inside the library instead of a
 * caller workspace.  It allocates nothing (no hipMalloc, no allocating
 * library routine) and enqueues only kernels on `stream`.
 *   Limit: a call whose workspace (pkv_decode_workspace_size for the same
 *   dims and block_size) exceeds PKV_NOALLOC_SCRATCH_BYTES is rejected with
 *   PKV_ERR_WORKSPACE, nothing enqueued.
 *   The array: one per device (the device of `stream`; the current device for
 *   the null stream), PKV_NOALLOC_SCRATCH_BYTES bytes, held until the process
 *   ends.  Every call on a device shares it and leaves its partial results in
 *   it; the library clears what must start at zero (with a small kernel on
 *   `stream`, ordered before the call's own kernels).  Calls that may overlap
 *   on one device (different streams, or host threads, without ordering
 *   between them) race on it: order them, or use pkv_paged_attention_decode
 *   with one workspace each.
 * Returns PKV_OK, PKV_ERR_INVALID / PKV_ERR_UNSUPPORTED as the workspace
 * variant, PKV_ERR_WORKSPACE when the scratch would not fit, PKV_ERR_HIP when
 * the device or the array's address cannot be obtained or a launch fails. */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
pkv_status pkv_paged_attention_decode_noalloc(const void* q, const void* k_cache,
                                              const void* v_cache,
                                              const int32_t* block_tables,
                                              const int32_t* seq_lens, int32_t block_size,
                                              float scale, void* out,
                                              const pkv_decode_dims* dims, void* stream);

/* Slot-mapped cache write [ITH §手動畫一次 block table: the next token goes
 * into the tail block's next free slot; PU §按 Block 分配: new tokens fill the
 * tail block first].  For n in [0, num_tokens) with s = slot_mapping[n] >= 0:
 *   K of token n, head h  -> k_cache block s/B, head h, offset s%B
 *   V of token n, head h  -> v_cache block s/B, head h, offset s%B
 * Negative slots are skipped (padding tokens).  A bit copy: no rounding.
 *   k, v          bf16 [num_tokens, num_kv_heads, head_dim] contiguous.
 *   slot_mapping  int64 [num_tokens]; each s in [-inf, num_blocks*block_size);
 *                 non-negative slots must be distinct within one call.
 * head_dim must be a multiple of 8 (16-byte rows). */
pkv_status pkv_reshape_and_cache(const void* k, const void* v,
                                 const int64_t* slot_mapping, int32_t num_tokens,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 void* k_cache, void* v_cache, int32_t num_blocks,
                                 int32_t block_size, void* stream);

/* Whole-block copy for copy-on-write of a shared tail block [PU §共享前缀，
 * 分叉时 Copy-on-write: before a sequence writes into a block whose reference
 * count is above one, the block is copied and the writer's table entry is
 * pointed at the copy].  For every layer l and pair i, in both caches:
 *   cache_l[dst_i] = cache_l[src_i]     (block_bytes bytes each)
 *   k_caches, v_caches  HOST arrays of num_layers device pointers
 *                       (1 <= num_layers <= 64), 16-byte aligned.
 *   block_pairs         device int32 [num_pairs, 2] = (src, dst) block ids.
 *                       dst ids must be distinct and no dst may also be a src.
 *   block_bytes         bytes per block per cache, a multiple of 16
 *                       (Hkv * B * D * 2 for the layout above).
 * num_pairs == 0 enqueues nothing and returns PKV_OK. */
pkv_status pkv_copy_blocks(void* const* k_caches, void* const* v_caches,
                           int32_t num_layers, const int32_t* block_pairs,
                           int32_t num_pairs, int64_t block_bytes, void* stream);

/* Block swap-out and swap-in [AK §故事沒有說完的部分: when memory runs short,
 * some requests' pages are swapped out and later swapped back in; this rests
 * on pages living anywhere and being found through the table, so a block may
 * come back into a different physical block whose id the table then takes].
 *   k_caches, v_caches  HOST arrays of num_layers device pointers
 *                       (1 <= num_layers <= 64), 16-byte aligned.
 *   block_ids           device int32 [num_ids]: swap-out reads these blocks,
 *                       swap-in writes them (distinct ids for swap-in).
 *   block_bytes         bytes per block per cache, a multiple of 16
 *                       (Hkv * B * D * 2 for the layout above).
 *   host_buffer         PINNED host memory the device can address (allocated
 *                       with hipHostMalloc, or torch's pin_memory), 16-byte
 *                       aligned, holding num_layers * 2 * num_ids * block_bytes
 *                       bytes laid out [layer][K, V][i]: K block block_ids[i]
 *                       of layer l at ((2 l) num_ids + i) block_bytes, its V
 *                       block at ((2 l + 1) num_ids + i) block_bytes.  Pageable
 *                       memory is refused (PKV_ERR_INVALID).
 * One launch: the device copies the blocks over the host link itself.
 * num_ids == 0 enqueues nothing and returns PKV_OK. */
pkv_status pkv_swap_out(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                        const int32_t* block_ids, int32_t num_ids, int64_t block_bytes,
                        void* host_buffer, void* stream);
pkv_status pkv_swap_in(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                       const int32_t* block_ids, int32_t num_ids, int64_t block_bytes,
                       const void* host_buffer, void* stream);

/* Merge of per-segment attention results [PU §按 Block 分配: with Z_r the sum
 * of e^{s_i} over segment r and o_r that segment's own softmax output,
 * o = sum_r Z_r o_r / sum_r Z_r, evaluated after rescaling every Z_r to the
 * common maximum so nothing overflows].
 *   part_out  fp32 [num_rows, num_parts, head_dim]: o_r per row and segment.
 *   part_lse  fp32 [num_rows, num_parts]: ln Z_r; -inf marks an empty segment
 *             (its part_out entry is then ignored).
 *   out       [num_rows, head_dim] in out_dtype; a row whose segments are all
 *             empty becomes 0.
 * head_dim <= 256. */
pkv_status pkv_merge_attention_states(const float* part_out, const float* part_lse,
                                      int32_t num_rows, int32_t num_parts,
                                      int32_t head_dim, void* out,
                                      pkv_dtype out_dtype, void* stream);

/* Shared-prefix ("cascade") decode [PU §共享前缀，分叉时 Copy-on-write: the
 * samples of one prompt point their block tables at the same physical blocks
 * for the prompt, and full prefix blocks stay shared; PU §按 Block 分配:
 * per-segment results merge by o = (Z1 o1 + Z2 o2) / (Z1 + Z2) after
 * rescaling to a common maximum, segments need not follow physical blocks].
 * Computes exactly what pkv_paged_attention_decode computes for the same q,
 * caches, tables and lengths, but reads the blocks a group shares once for
 * the whole group: each sequence's tokens are cut into its group's shared
 * prefix and its own suffix, the prefix is attended by all members' queries
 * together, and the two segment results are merged.
 *
 *   group_starts  device int32 [num_groups + 1]: group g is the sequences
 *                 [group_starts[g], group_starts[g+1]); group_starts[0] = 0,
 *                 strictly increasing, group_starts[num_groups] = S.  A
 *                 sequence that shares nothing is a group of one.
 *   prefix_lens   device int32 [num_groups]: L_g, the tokens every member of
 *                 group g shares; a multiple of block_size, 0 <= L_g <=
 *                 max_prefix_len, L_g <= T_b for every member b, and the first
 *                 L_g / block_size entries of every member's table row are the
 *                 same physical blocks (the first member's row is read).
 *   num_groups    1 <= num_groups <= S (when S > 0).
 *   max_prefix_len  host bound on every L_g, <= dims->max_seq_len.
 *   dims          as for pkv_paged_attention_decode; `partition_size`,
 *                 `waves_per_group`, `balance_partitions` and `stream_waves`
 *                 are ignored.  head_dim 64 or 128, block_size 8, 16 or 32,
 *                 group <= 16, S <= 4096 (PKV_ERR_UNSUPPORTED otherwise).
 *                 `kernel` picks the form: PKV_KERNEL_STREAM_WG one launch, a
 *                 workgroup per (group, KV head, block of members) folding the
 *                 group's prefix and those members' suffixes and merging in
 *                 LDS (PKV_ERR_UNSUPPORTED when a task's chunks - the longest
 *                 prefix plus its members' longest suffixes, from the host
 *                 bounds - exceed its LDS records); PKV_KERNEL_MFMA two
 *                 launches, segments' partial states then their merge; any
 *                 other value the first when it fits, else the second.
 *   workspace     device scratch of at least pkv_cascade_workspace_size bytes,
 *                 256-byte aligned; needs no initialisation and holds garbage
 *                 after the call.
 * If a device-side condition above fails (groups not a partition of the
 * sequences, L_g not a multiple of block_size or above max_prefix_len, a
 * member shorter than L_g, some T_b above dims->max_seq_len), every output row
 * is NaN.  q, k_cache and v_cache 16-byte aligned.  Results do not depend on
 * timing (each form merges in a fixed order).
 * Returns PKV_OK, or an error status with nothing enqueued. */
size_t pkv_cascade_workspace_size(const pkv_decode_dims* dims, int32_t num_groups,
                                  int32_t max_prefix_len, int32_t block_size);
pkv_status pkv_cascade_decode(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* seq_lens,
                              const int32_t* group_starts, const int32_t* prefix_lens,
                              int32_t num_groups, int32_t max_prefix_len, int32_t block_size,
                              float scale, void* out, const pkv_decode_dims* dims,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Paged prefill: causal multi-query attention of each sequence's new tokens
 * over its cached tokens, read through the block table [PU §KV Cache 为什么会
 * 浪费显存: prefill processes the prompt and builds the cache, and in causal
 * attention a token attends to the tokens before it; PU §Continuous Batching:
 * paging (and FlashAttention) keep the dense attention semantics; PU §按 Block
 * 分配: position t is read through logical block t / B, offset t % B].
 *   q           bf16 [num_tokens, Hq, D]: the new tokens' queries, sequence by
 *               sequence.
 *   cu_q_lens   device int32 [S + 1]: sequence b's new tokens are rows
 *               cu_q_lens[b] .. cu_q_lens[b+1]-1 of q and out; 0 = cu_q_lens[0]
 *               <= ... <= cu_q_lens[S] = num_tokens.
 *   seq_lens    T_b: every cached token of sequence b, its q_len_b new ones
 *               included (their K,V written first, e.g. by
 *               pkv_reshape_and_cache); q_len_b <= T_b.
 *   max_q_len   host bound on q_len_b (sizes the grid; a longer chunk is still
 *               computed, only more slowly); <= dims->max_seq_len.
 *   out         [num_tokens, Hq, D] in dims->out_dtype.
 * New token i of sequence b sits at position T_b - q_len_b + i and attends the
 * positions 0 .. its own; query head h reads KV head h / G.  dims as for
 * pkv_paged_attention_decode (kernel, partition and stream fields ignored);
 * head_dim 64 or 128, block_size 8, 16 or 32, group <= 16.  No workspace.
 * A sequence whose row range is not inside [0, num_tokens) is skipped; one
 * with q_len_b > T_b or T_b above the table's capacity gets NaN rows.
 * q, k_cache and v_cache 16-byte aligned.
 * Returns PKV_OK, or an error status with nothing enqueued. */
pkv_status pkv_paged_prefill(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* seq_lens,
                             const int32_t* cu_q_lens, int32_t num_tokens, int32_t max_q_len,
                             int32_t block_size, float scale, void* out,
                             const pkv_decode_dims* dims, void* stream);

/* Checkers of the device-resident inputs the calls above take on trust (for
 * callers that cannot vouch for their tables, e.g. while debugging a block
 * manager).  Each one clears *flags (device int32, caller-owned), then ORs in
 * a bit for every kind of violation it finds; the word is final once the
 * stream reaches the call.  They only compare values: no table entry, slot or
 * block id is used to address memory, so any values may be checked.  They
 * enqueue kernels only (no allocation, copy or memset).  Return PKV_OK, or
 * PKV_ERR_INVALID for a NULL pointer or a negative size, with nothing enqueued.
 *
 * Decode inputs [ITH §手動畫一次 block table: a sequence of T tokens uses
 * logical blocks 0 .. ceil(T/B)-1, each mapped to a physical block]:
 *   bit 0  an entry of row b in 0 .. ceil(T_b/B)-1 outside [0, num_blocks);
 *   bit 1  a length outside [0, min(max_seq_len, max_blocks_per_seq*B)]
 *          (that row's entries are then not examined). */
pkv_status pkv_check_decode_inputs(const int32_t* block_tables, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t max_blocks_per_seq,
                                   int32_t num_blocks, int32_t block_size, int32_t max_seq_len,
                                   int32_t* flags, void* stream);
/* Slot mapping of pkv_reshape_and_cache [PU §按 Block 分配: slot =
 * physical_block * B + offset]: bit 0 a slot >= num_blocks * block_size;
 * bit 1 a non-negative slot that appears twice (negative slots are padding). */
pkv_status pkv_check_slot_mapping(const int64_t* slot_mapping, int32_t num_tokens,
                                  int32_t num_blocks, int32_t block_size, int32_t* flags,
                                  void* stream);
/* Pairs of pkv_copy_blocks [PU §共享前缀，分叉时 Copy-on-write]: bit 0 a src
 * or dst outside [0, num_blocks); bit 1 a dst that appears twice; bit 2 a dst
 * that is also some pair's src. */
pkv_status pkv_check_block_pairs(const int32_t* block_pairs, int32_t num_pairs,
                                 int32_t num_blocks, int32_t* flags, void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* pkv_status_string(int32_t status);

/* Version of this ABI: (major << 16) | minor. */
int32_t pkv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
