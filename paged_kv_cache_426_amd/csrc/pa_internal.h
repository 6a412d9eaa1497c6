// Host-side launch interface between the C ABI (pa_api.cpp) and the gfx950
// kernels. Plain C++: no HIP types, so the validation unit stays host-only.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pa {

// How a decode cuts each sequence's context into the ranges one workgroup
// reads.
enum SplitMode : int {
  kSplitSingle = 0,    // one range per sequence
  kSplitFixed = 1,     // fixed partitions of partition_size tokens
  kSplitBalanced = 2,  // all sequences' blocks end to end, cut into num_splits equal shares
};

// Decode kernel variants: ranges (fixed partitions), balanced shares dealt
// to all waves of a workgroup, balanced shares with one wave per head row,
// whole sequences (single pass; ranges over wider workgroups).
enum KernelKind : int { kKindRanges = 0, kKindShares = 1, kKindRowWaves = 2, kKindSingle = 3 };

// Balanced split: at most this many sequences per call (the per-sequence
// start blocks live in LDS), and at most this many shares.
constexpr int kMaxBalancedSeqs = 1024;
constexpr int kMaxAutoSplits = 2048;

struct DecodeLaunch {
  // outputs: `out`, and/or the three partial arrays
  void *out;
  float *tmp_out;
  float *max_logits;
  float *exp_sums;
  // partial-array stride: fixed split, per (sequence, head) -- index
  // ((b * Hq + h) * max_partitions + partition); balanced split, per head --
  // index (h * max_partitions + share + b), max_partitions = num_splits + B
  int max_partitions;
  // inputs
  const void *q;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  int num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq;
  float scale, k_scale, v_scale;
  int q_dtype, kv_dtype;
  int mode;            // SplitMode
  int partition_size;  // fixed split: tokens per partition
  int num_splits;      // balanced split: shares
  int direct;          // a range covering a whole sequence writes `out` directly
  // decode with append: the new token of every sequence (position n - 1),
  // [num_seqs, Hkv, d] in q's type, written to its slot and attended from
  // these rows; null for a plain decode
  const void *new_k;
  const void *new_v;
  // 8-bit caches with scale tables (pa_decode_scaled): the scale of
  // (physical block e, KV head g) is k_scales[e * scale_block_stride +
  // g * scale_head_stride] (likewise v_scales); null for per-tensor scales
  const float *k_scales;
  const float *v_scales;
  int scale_block_stride, scale_head_stride;
};

// Strides of a scale table of the given layout (a pa.h PA_SCALE_* value)
// over (physical block, KV head); false for an unknown layout.
inline bool scale_strides(int layout, int num_kv_heads, int *block_stride, int *head_stride) {
  switch (layout) {
    case 1: *block_stride = 0; *head_stride = 1; return true;             // [Hkv]
    case 2: *block_stride = 1; *head_stride = 0; return true;             // [num_blocks]
    case 3: *block_stride = num_kv_heads; *head_stride = 1; return true;  // [num_blocks, Hkv]
  }
  return false;
}

struct ReduceLaunch {
  void *out;
  const float *tmp_out;
  const float *max_logits;
  const float *exp_sums;
  const int32_t *context_lens;
  int num_seqs, num_q_heads, head_dim, block_size;
  int max_partitions;
  int mode;            // kSplitFixed or kSplitBalanced
  int partition_size;  // fixed
  int num_splits;      // balanced
  int skip_single;     // sequences held in one piece were already written
  int out_dtype;
};

// A decode kernel's host-side handle and the workgroup size it is built for.
struct KernelRef {
  const void *fn;
  int threads;
};

// Each returns 0 on success or the runtime's error code.
int launch_decode(const DecodeLaunch &a, void *stream);
int launch_reduce(const ReduceLaunch &a, void *stream);
// Scale tables of the slot write and the block copy: null for per-tensor
// scales (slot write) or none to move (copy); strides as in DecodeLaunch.
struct ScaleTables {
  float *k, *v;
  int block_stride, head_stride;
  int block_size;  // tokens per physical block (slot write: slot / block_size)
};

int launch_reshape_and_cache(const void *key, const void *value, void *k_cache, void *v_cache,
                             const int64_t *slot_mapping, int num_tokens, int num_kv_heads,
                             int head_dim, int src_dtype, int cache_dtype, float k_scale,
                             float v_scale, const ScaleTables &tables, void *stream);
// entries: scale entries per block to copy (0: none; 1 or Hkv)
int launch_copy_blocks(void *k_cache, void *v_cache, const int64_t *block_mapping,
                       int num_pairs, size_t block_bytes, float *k_scales, float *v_scales,
                       int entries, void *stream);

// Device scratch of a shared-prefix decode, carved from the caller's workspace.
struct SharedPrefixWorkspace {
  void *q_stack;            // [G, Hq * M, d], q's type
  int32_t *prefix_tables;   // [G, MBS]
  int32_t *prefix_ctx;      // [G]
  int32_t *suffix_tables;   // [B, MBS]
  int32_t *suffix_lens;     // [B]
  int32_t *seq_slot;        // [B]
  float *a_out, *a_max, *a_sum;  // prefix pass partials, balanced layout
  float *b_out, *b_max, *b_sum;  // suffix pass partials, balanced layout
};

struct SharedPrefixLaunch {
  void *out;
  const void *q, *k_cache, *v_cache;
  const int32_t *block_tables, *context_lens;
  const int32_t *group_members;  // [G, M] sequence ids (-1: empty slot)
  const int32_t *prefix_lens;    // [G] shared prefix tokens
  int num_seqs, num_groups, group_size;
  int num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq;
  float scale, k_scale, v_scale;
  int q_dtype, kv_dtype, q_elem_bytes;
  int prefix_splits;  // balanced-split shares of the prefix pass
  int suffix_splits;  // 0: the suffix pass runs single-pass, one partial per (sequence, head)
  SharedPrefixWorkspace ws;
};

// Prep, prefix pass, suffix pass and merge, in stream order.
int launch_shared_prefix(const SharedPrefixLaunch &a, void *stream);

struct PrefillLaunch {
  void *out;
  const void *q, *k_cache, *v_cache;
  const int32_t *block_tables, *context_lens, *query_start;
  int num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq;
  int max_query_len;
  float scale, k_scale, v_scale;
  int q_dtype, kv_dtype;
};

// Causal attention of each sequence's chunk of query tokens over its paged
// context (pa_prefill).
int launch_prefill(const PrefillLaunch &a, void *stream);
// Chunk tokens one prefill workgroup takes for a GQA group size.
int prefill_tokens_per_tile(int group);

// Shares a balanced split uses on the current device: enough workgroups to
// fill every compute unit once at the decode kernel's occupancy.
int balanced_num_splits(const DecodeLaunch &a);

// Size of the fixed device scratch that pa_decode_noalloc uses for split
// partials, and its address on the current device (looked up with
// hipGetSymbolAddress on the first call per device). Returns 0 or the
// runtime's error code.
constexpr size_t kNoallocScratchBytes = (size_t)16 << 20;
int noalloc_scratch(void **ptr);

// Block sizes the decode kernels take: 16 << k tokens, k = 0 .. kMaxSubLog2
// (16 to 256). Returns k, or -1 for any other size.
constexpr int kMaxSubLog2 = 4;
inline int sub_block_log2(int block_size) {
  for (int k = 0; k <= kMaxSubLog2; ++k)
    if (block_size == (16 << k)) return k;
  return -1;
}
// 8-token blocks, which the decode kernels (pa_decode, pa_decode_partials,
// pa_decode_noalloc) also take: a 16-token unit is then two physical blocks.
// The decode parameters carry this value in place of log2(block_size / 16).
constexpr int kHalfBlocks = -1;
constexpr int kHalfBlockSize = 8;
inline bool decode_block_size_ok(int block_size) {
  return block_size == kHalfBlockSize || sub_block_log2(block_size) >= 0;
}

// heads of one KV group that one workgroup serves (a divisor of the group, <= 16)
inline int heads_per_workgroup(int group) {
  return group % 16 == 0 ? 16 : group % 8 == 0 ? 8 : group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
}

}  // namespace pa
