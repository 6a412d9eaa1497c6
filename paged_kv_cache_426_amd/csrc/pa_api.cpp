// C ABI of libpa: argument validation and dispatch to the gfx950 kernels.
// Every check that can be made on the host happens here, before anything is
// enqueued; a failed check returns a status and has no side effects.

#include <limits.h>
#include <math.h>

#include "pa.h"
#include "pa_internal.h"

namespace {

bool supported_head_dim(int d) { return d == 64 || d == 128; }

bool known_dtype(int t) {
  return t == PA_F32 || t == PA_F16 || t == PA_BF16 || t == PA_FP8_E4M3FN || t == PA_INT8;
}

int elem_bytes(int t) { return t == PA_F32 ? 4 : (t == PA_FP8_E4M3FN || t == PA_INT8) ? 1 : 2; }

// 8-bit cache types: codes scaled by k_scale / v_scale
bool quantised(int t) { return t == PA_FP8_E4M3FN || t == PA_INT8; }

bool supported_decode_pair(int q, int kv) {
  if (q == kv) return q == PA_F32 || q == PA_F16 || q == PA_BF16;
  return quantised(kv) && (q == PA_F16 || q == PA_BF16);
}

pa_status status_of(int hip_err) { return hip_err == 0 ? PA_OK : PA_ERR_LAUNCH; }

// The softmax scale: a NaN selects 1/sqrt(d_k) of the attention formula
// ("KV-Cache evolution", section 1), the float32 nearest to 1/sqrt(head_dim)
// (evaluated in double, rounded once).
float resolve_scale(float scale, int head_dim) {
  return isnan(scale) ? (float)(1.0 / sqrt((double)head_dim)) : scale;
}

// Shared checks of pa_decode and pa_decode_partials.
pa_status check_decode(const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *block_tables, const int32_t *context_lens, int num_seqs,
                       int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                       int num_blocks, int max_blocks_per_seq, float scale, int q_dtype,
                       int kv_dtype, float k_scale, float v_scale, int partition_size) {
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL_POINTER;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return PA_ERR_BAD_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_BAD_SHAPE;
  if (!known_dtype(q_dtype) || !known_dtype(kv_dtype)) return PA_ERR_UNSUPPORTED;
  if (!supported_head_dim(head_dim) || !pa::decode_block_size_ok(block_size) ||
      !supported_decode_pair(q_dtype, kv_dtype))
    return PA_ERR_UNSUPPORTED;
  if (partition_size > 0 && partition_size % block_size != 0) return PA_ERR_BAD_SHAPE;
  // partitions are whole 16-token units of the kernels (8-token blocks: an
  // even number of blocks)
  if (partition_size > 0 && partition_size % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (partition_size < 0 && num_seqs > pa::kMaxBalancedSeqs) return PA_ERR_UNSUPPORTED;
  if (isinf(scale)) return PA_ERR_BAD_SHAPE;  // NaN: the default scale
  if (quantised(kv_dtype) && (!isfinite(k_scale) || !isfinite(v_scale)))
    return PA_ERR_BAD_SHAPE;
  // launch-grid and in-kernel 32-bit offset limits
  const long long row_bytes = (long long)num_kv_heads * head_dim * elem_bytes(kv_dtype);
  if (row_bytes * block_size >= INT_MAX) return PA_ERR_UNSUPPORTED;
  const int group = num_q_heads / num_kv_heads;
  const long long grid_y = (long long)num_kv_heads * (group / pa::heads_per_workgroup(group));
  if (grid_y > 65535 || num_seqs > 65535) return PA_ERR_UNSUPPORTED;
  if (partition_size < -pa::kMaxAutoSplits) return PA_ERR_UNSUPPORTED;
  if ((long long)max_blocks_per_seq * block_size > INT_MAX) return PA_ERR_UNSUPPORTED;
  // the kernels address the pool in 16-token sub-blocks with 32-bit ids
  if ((long long)num_blocks * (block_size / 16) > INT_MAX) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

}  // namespace

extern "C" {

const char *pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case PA_ERR_BAD_SHAPE: return "invalid or inconsistent sizes";
    case PA_ERR_UNSUPPORTED: return "configuration not supported by this build";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_SCRATCH_LIMIT:
      return "split partials exceed the fixed scratch of pa_decode_noalloc "
             "(pa_decode_noalloc_scratch_bytes); use pa_decode with a workspace";
  }
  return "unknown status";
}

int pa_version(void) { return 100; }

int pa_num_partitions(int max_blocks_per_seq, int block_size, int partition_size) {
  if (partition_size <= 0 || max_blocks_per_seq <= 0 || block_size <= 0) return 0;
  const long long tokens = (long long)max_blocks_per_seq * block_size;
  return (int)((tokens + partition_size - 1) / partition_size);
}

size_t pa_decode_workspace_size(int num_seqs, int num_q_heads, int head_dim,
                                int max_blocks_per_seq, int block_size, int partition_size) {
  if (partition_size == 0 || num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  if (partition_size < 0) {
    // balanced split: per query head, one piece per (share, sequence) boundary
    const size_t splits = partition_size == -1 ? (size_t)pa::kMaxAutoSplits
                                               : (size_t)(-(long long)partition_size);
    return (size_t)num_q_heads * (splits + (size_t)num_seqs) * ((size_t)head_dim + 2) *
           sizeof(float);
  }
  const size_t np = (size_t)pa_num_partitions(max_blocks_per_seq, block_size, partition_size);
  return (size_t)num_seqs * num_q_heads * np * ((size_t)head_dim + 2) * sizeof(float);
}

int pa_decode_balanced_splits(int num_q_heads, int num_kv_heads, int head_dim, int q_dtype,
                              int kv_dtype) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return 0;
  if (!supported_head_dim(head_dim) || !supported_decode_pair(q_dtype, kv_dtype)) return 0;
  pa::DecodeLaunch a{};
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.q_dtype = q_dtype;
  a.kv_dtype = kv_dtype;
  return pa::balanced_num_splits(a);
}

pa_status pa_decode_partials(float *tmp_out, float *max_logits, float *exp_sums,
                             int max_partitions, const void *q, const void *k_cache,
                             const void *v_cache, const int32_t *block_tables,
                             const int32_t *context_lens, int num_seqs, int num_q_heads,
                             int num_kv_heads, int head_dim, int block_size, int num_blocks,
                             int max_blocks_per_seq, float scale, int q_dtype, int kv_dtype,
                             float k_scale, float v_scale, int partition_size, void *stream) {
  if (!tmp_out || !max_logits || !exp_sums) return PA_ERR_NULL_POINTER;
  pa_status st = check_decode(q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                              num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                              max_blocks_per_seq, scale, q_dtype, kv_dtype, k_scale, v_scale,
                              partition_size);
  if (st != PA_OK) return st;
  // fixed partitions, or a balanced split with an explicit share count
  if (partition_size == 0 || partition_size == -1) return PA_ERR_BAD_SHAPE;
  if (partition_size > 0 &&
      max_partitions < pa_num_partitions(max_blocks_per_seq, block_size, partition_size))
    return PA_ERR_BAD_SHAPE;
  if (partition_size < 0 && (long long)max_partitions < -(long long)partition_size + num_seqs)
    return PA_ERR_BAD_SHAPE;
  if (num_seqs == 0) return PA_OK;
  pa::DecodeLaunch a{};
  a.tmp_out = tmp_out;
  a.max_logits = max_logits;
  a.exp_sums = exp_sums;
  a.max_partitions = max_partitions;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.scale = resolve_scale(scale, head_dim);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.q_dtype = q_dtype;
  a.kv_dtype = kv_dtype;
  a.partition_size = partition_size;
  a.mode = partition_size > 0 ? pa::kSplitFixed : pa::kSplitBalanced;
  a.num_splits = partition_size > 0 ? 0 : -partition_size;
  a.direct = 0;
  return status_of(pa::launch_decode(a, stream));
}

pa_status pa_decode_reduce(void *out, const float *tmp_out, const float *max_logits,
                           const float *exp_sums, const int32_t *context_lens, int num_seqs,
                           int num_q_heads, int head_dim, int max_partitions, int partition_size,
                           int out_dtype, void *stream) {
  if (!out || !tmp_out || !max_logits || !exp_sums || !context_lens) return PA_ERR_NULL_POINTER;
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_partitions <= 0 ||
      partition_size == 0 || partition_size == -1)
    return PA_ERR_BAD_SHAPE;
  if (out_dtype != PA_F32 && out_dtype != PA_F16 && out_dtype != PA_BF16)
    return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  // merge grids: (sequences, head runs of 256 / head_dim) or (heads, sequences)
  if (num_seqs > 65535 || num_q_heads > 65535 * (256 / head_dim)) return PA_ERR_UNSUPPORTED;
  if (partition_size > 0 && partition_size % 16 != 0) return PA_ERR_BAD_SHAPE;
  if (partition_size < 0) {
    if (num_seqs > pa::kMaxBalancedSeqs || partition_size < -pa::kMaxAutoSplits)
      return PA_ERR_UNSUPPORTED;
    if ((long long)max_partitions < -(long long)partition_size + num_seqs) return PA_ERR_BAD_SHAPE;
  }
  if (num_seqs == 0) return PA_OK;
  pa::ReduceLaunch r{};
  r.out = out;
  r.tmp_out = tmp_out;
  r.max_logits = max_logits;
  r.exp_sums = exp_sums;
  r.context_lens = context_lens;
  r.num_seqs = num_seqs;
  r.num_q_heads = num_q_heads;
  r.head_dim = head_dim;
  r.block_size = 16;
  r.max_partitions = max_partitions;
  r.mode = partition_size > 0 ? pa::kSplitFixed : pa::kSplitBalanced;
  r.partition_size = partition_size;
  r.num_splits = partition_size > 0 ? 0 : -partition_size;
  r.skip_single = 0;
  r.out_dtype = out_dtype;
  return status_of(pa::launch_reduce(r, stream));
}

namespace {

// Scale tables of pa_decode_scaled (k == nullptr: per-tensor scales).
struct Tables {
  const float *k, *v;
  int block_stride, head_stride;
};

// pa_decode, pa_decode_append when new_k / new_v are given, and
// pa_decode_scaled with scale tables.
pa_status decode_impl(void *out, const void *q, const void *new_k, const void *new_v,
                      const void *k_cache, const void *v_cache, const int32_t *block_tables,
                      const int32_t *context_lens, int num_seqs, int num_q_heads,
                      int num_kv_heads, int head_dim, int block_size, int num_blocks,
                      int max_blocks_per_seq, float scale, int q_dtype, int kv_dtype,
                      float k_scale, float v_scale, int partition_size, void *workspace,
                      size_t workspace_bytes, void *stream, const Tables &tables = {}) {
  if (!out) return PA_ERR_NULL_POINTER;
  pa_status st = check_decode(q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                              num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                              max_blocks_per_seq, scale, q_dtype, kv_dtype, k_scale, v_scale,
                              partition_size);
  if (st != PA_OK) return st;
  pa::DecodeLaunch a{};
  a.out = out;
  a.new_k = new_k;
  a.new_v = new_v;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.scale = resolve_scale(scale, head_dim);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.q_dtype = q_dtype;
  a.kv_dtype = kv_dtype;
  a.partition_size = partition_size;
  a.direct = 1;
  a.k_scales = tables.k;
  a.v_scales = tables.v;
  a.scale_block_stride = tables.block_stride;
  a.scale_head_stride = tables.head_stride;
  size_t need = 0;
  size_t pieces = 0;  // partial-array entries per (sequence, head) or per head
  if (partition_size > 0) {
    a.mode = pa::kSplitFixed;
    a.max_partitions = pa_num_partitions(max_blocks_per_seq, block_size, partition_size);
    pieces = (size_t)num_seqs * num_q_heads * a.max_partitions;
    need = pieces * ((size_t)head_dim + 2) * sizeof(float);
  } else if (partition_size < 0) {
    a.mode = pa::kSplitBalanced;
    // the workspace checks that need no device query come first
    const size_t least = (size_t)num_q_heads * (1 + (size_t)num_seqs) * ((size_t)head_dim + 2) *
                         sizeof(float);
    if (!workspace) return PA_ERR_NULL_POINTER;
    if (workspace_bytes < least) return PA_ERR_WORKSPACE_TOO_SMALL;
    a.num_splits = partition_size == -1 ? pa::balanced_num_splits(a) : -partition_size;
    a.max_partitions = a.num_splits + num_seqs;
    pieces = (size_t)num_q_heads * a.max_partitions;
    need = pieces * ((size_t)head_dim + 2) * sizeof(float);
  } else {
    a.mode = pa::kSplitSingle;
  }
  if (need > 0) {
    if (!workspace) return PA_ERR_NULL_POINTER;
    if (workspace_bytes < need) return PA_ERR_WORKSPACE_TOO_SMALL;
  }
  if (num_seqs == 0) return PA_OK;
  if (a.mode == pa::kSplitSingle) return status_of(pa::launch_decode(a, stream));
  // split context: partials into the workspace (sequences held in one piece
  // are written to `out` directly), then the merge
  a.tmp_out = static_cast<float *>(workspace);
  a.max_logits = a.tmp_out + pieces * head_dim;
  a.exp_sums = a.max_logits + pieces;
  st = status_of(pa::launch_decode(a, stream));
  if (st != PA_OK) return st;
  pa::ReduceLaunch r{};
  r.out = out;
  r.tmp_out = a.tmp_out;
  r.max_logits = a.max_logits;
  r.exp_sums = a.exp_sums;
  r.context_lens = context_lens;
  r.num_seqs = num_seqs;
  r.num_q_heads = num_q_heads;
  r.head_dim = head_dim;
  r.block_size = block_size;
  r.max_partitions = a.max_partitions;
  r.mode = a.mode;
  r.partition_size = partition_size;
  r.num_splits = a.num_splits;
  r.skip_single = 1;
  r.out_dtype = q_dtype;
  return status_of(pa::launch_reduce(r, stream));
}

}  // namespace

pa_status pa_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, const int32_t *context_lens, int num_seqs,
                    int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                    int num_blocks, int max_blocks_per_seq, float scale, int q_dtype,
                    int kv_dtype, float k_scale, float v_scale, int partition_size,
                    void *workspace, size_t workspace_bytes, void *stream) {
  return decode_impl(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, scale, q_dtype, kv_dtype, k_scale, v_scale,
                     partition_size, workspace, workspace_bytes, stream);
}

pa_status pa_decode_noalloc(void *out, const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, const int32_t *context_lens,
                            int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                            int block_size, int num_blocks, int max_blocks_per_seq, float scale,
                            int q_dtype, int kv_dtype, float k_scale, float v_scale,
                            int partition_size, void *stream) {
  if (!out) return PA_ERR_NULL_POINTER;
  pa_status st = check_decode(q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                              num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                              max_blocks_per_seq, scale, q_dtype, kv_dtype, k_scale, v_scale,
                              partition_size);
  if (st != PA_OK) return st;
  void *ws = nullptr;
  size_t ws_bytes = 0;
  if (partition_size != 0 && num_seqs > 0) {
    if (pa::noalloc_scratch(&ws) != 0) return PA_ERR_LAUNCH;
    ws_bytes = pa::kNoallocScratchBytes;
  }
  st = decode_impl(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens,
                   num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                   max_blocks_per_seq, scale, q_dtype, kv_dtype, k_scale, v_scale,
                   partition_size, ws, ws_bytes, stream);
  return st == PA_ERR_WORKSPACE_TOO_SMALL ? PA_ERR_SCRATCH_LIMIT : st;
}

size_t pa_decode_noalloc_scratch_bytes(void) { return pa::kNoallocScratchBytes; }

pa_status pa_decode_scaled(void *out, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *block_tables, const int32_t *context_lens,
                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int block_size, int num_blocks, int max_blocks_per_seq, float scale,
                           int q_dtype, int kv_dtype, const float *k_scales,
                           const float *v_scales, int scale_layout, int partition_size,
                           void *workspace, size_t workspace_bytes, void *stream) {
  if (!k_scales || !v_scales) return PA_ERR_NULL_POINTER;
  Tables t{k_scales, v_scales, 0, 0};
  if (num_kv_heads > 0 &&
      !pa::scale_strides(scale_layout, num_kv_heads, &t.block_stride, &t.head_stride))
    return PA_ERR_BAD_SHAPE;
  if (known_dtype(kv_dtype) && !quantised(kv_dtype)) return PA_ERR_UNSUPPORTED;
  // a 16-token unit of 8-token blocks would carry two blocks' scales
  if (block_size == pa::kHalfBlockSize) return PA_ERR_UNSUPPORTED;
  return decode_impl(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, scale, q_dtype, kv_dtype, 1.0f, 1.0f, partition_size,
                     workspace, workspace_bytes, stream, t);
}

pa_status pa_decode_append(void *out, const void *q, const void *key, const void *value,
                           void *k_cache, void *v_cache, const int32_t *block_tables,
                           const int32_t *context_lens, int num_seqs, int num_q_heads,
                           int num_kv_heads, int head_dim, int block_size, int num_blocks,
                           int max_blocks_per_seq, float scale, int q_dtype, int kv_dtype,
                           float k_scale, float v_scale, int partition_size, void *workspace,
                           size_t workspace_bytes, void *stream) {
  if (!key || !value) return PA_ERR_NULL_POINTER;
  // the new token's rows are written as pa_reshape_and_cache writes them
  if (quantised(kv_dtype) &&
      (!isfinite(k_scale) || !isfinite(v_scale) || k_scale == 0.0f || v_scale == 0.0f))
    return PA_ERR_BAD_SHAPE;
  // the appended row's slot is found in 16-token units (block sizes 16 to 256)
  if (block_size == pa::kHalfBlockSize) return PA_ERR_UNSUPPORTED;
  return decode_impl(out, q, key, value, k_cache, v_cache, block_tables, context_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, scale, q_dtype, kv_dtype, k_scale, v_scale,
                     partition_size, workspace, workspace_bytes, stream);
}

pa_status pa_reshape_and_cache(const void *key, const void *value, void *k_cache, void *v_cache,
                               const int64_t *slot_mapping, int num_tokens, int num_kv_heads,
                               int head_dim, int block_size, int num_blocks, int src_dtype,
                               int cache_dtype, float k_scale, float v_scale, void *stream) {
  if (num_tokens == 0 && k_cache && v_cache) return PA_OK;  // no-op; token arrays may be empty
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL_POINTER;
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0)
    return PA_ERR_BAD_SHAPE;
  if (!known_dtype(src_dtype) || !known_dtype(cache_dtype)) return PA_ERR_UNSUPPORTED;
  if (quantised(src_dtype)) return PA_ERR_UNSUPPORTED;
  if (src_dtype != cache_dtype && !quantised(cache_dtype)) return PA_ERR_UNSUPPORTED;
  if (quantised(cache_dtype) && src_dtype != cache_dtype &&
      (!isfinite(k_scale) || !isfinite(v_scale) || k_scale == 0.0f || v_scale == 0.0f))
    return PA_ERR_BAD_SHAPE;
  // rows are moved in 16-byte pieces of the source
  const long long row_src_bytes = (long long)num_kv_heads * head_dim * elem_bytes(src_dtype);
  if (row_src_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (row_src_bytes > INT_MAX) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  return status_of(pa::launch_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping,
                                                num_tokens, num_kv_heads, head_dim, src_dtype,
                                                cache_dtype, k_scale, v_scale,
                                                pa::ScaleTables{}, stream));
}

pa_status pa_reshape_and_cache_scaled(const void *key, const void *value, void *k_cache,
                                      void *v_cache, const int64_t *slot_mapping,
                                      int num_tokens, int num_kv_heads, int head_dim,
                                      int block_size, int num_blocks, int src_dtype,
                                      int cache_dtype, const float *k_scales,
                                      const float *v_scales, int scale_layout, void *stream) {
  if (!k_scales || !v_scales) return PA_ERR_NULL_POINTER;
  pa::ScaleTables t{const_cast<float *>(k_scales), const_cast<float *>(v_scales), 0, 0,
                    block_size};
  if (num_kv_heads > 0 &&
      !pa::scale_strides(scale_layout, num_kv_heads, &t.block_stride, &t.head_stride))
    return PA_ERR_BAD_SHAPE;
  if (known_dtype(cache_dtype) && !quantised(cache_dtype)) return PA_ERR_UNSUPPORTED;
  if (known_dtype(src_dtype) && quantised(src_dtype)) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0 && k_cache && v_cache) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL_POINTER;
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0)
    return PA_ERR_BAD_SHAPE;
  if (!known_dtype(src_dtype) || !known_dtype(cache_dtype)) return PA_ERR_UNSUPPORTED;
  // a 16-byte piece of the source never spans two heads (one scale per piece)
  if ((long long)head_dim * elem_bytes(src_dtype) % 16 != 0) return PA_ERR_UNSUPPORTED;
  const long long row_src_bytes = (long long)num_kv_heads * head_dim * elem_bytes(src_dtype);
  if (row_src_bytes > INT_MAX) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  return status_of(pa::launch_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping,
                                                num_tokens, num_kv_heads, head_dim, src_dtype,
                                                cache_dtype, 1.0f, 1.0f, t, stream));
}

pa_status pa_copy_blocks(void *k_cache, void *v_cache, const int64_t *block_mapping,
                         int num_pairs, int num_kv_heads, int head_dim, int block_size,
                         int num_blocks, int cache_dtype, void *stream) {
  if (num_pairs == 0 && k_cache && v_cache) return PA_OK;  // no-op; the pair array may be empty
  if (!k_cache || !v_cache || !block_mapping) return PA_ERR_NULL_POINTER;
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_BAD_SHAPE;
  if (!known_dtype(cache_dtype)) return PA_ERR_UNSUPPORTED;
  const size_t block_bytes =
      (size_t)block_size * num_kv_heads * head_dim * (size_t)elem_bytes(cache_dtype);
  if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  return status_of(pa::launch_copy_blocks(k_cache, v_cache, block_mapping, num_pairs, block_bytes,
                                          nullptr, nullptr, 0, stream));
}

pa_status pa_copy_blocks_scaled(void *k_cache, void *v_cache, float *k_scales, float *v_scales,
                                const int64_t *block_mapping, int num_pairs, int num_kv_heads,
                                int head_dim, int block_size, int num_blocks, int cache_dtype,
                                int scale_layout, void *stream) {
  if (!k_scales || !v_scales) return PA_ERR_NULL_POINTER;
  int sb = 0, sh = 0;
  if (num_kv_heads > 0 && !pa::scale_strides(scale_layout, num_kv_heads, &sb, &sh))
    return PA_ERR_BAD_SHAPE;
  if (known_dtype(cache_dtype) && !quantised(cache_dtype)) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0 && k_cache && v_cache) return PA_OK;
  if (!k_cache || !v_cache || !block_mapping) return PA_ERR_NULL_POINTER;
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_BAD_SHAPE;
  if (!known_dtype(cache_dtype)) return PA_ERR_UNSUPPORTED;
  const size_t block_bytes =
      (size_t)block_size * num_kv_heads * head_dim * (size_t)elem_bytes(cache_dtype);
  if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  // entries per block: the table's block stride (0 for a per-head table)
  return status_of(pa::launch_copy_blocks(k_cache, v_cache, block_mapping, num_pairs, block_bytes,
                                          k_scales, v_scales, sb, stream));
}


}  // extern "C"

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of a shared-prefix decode: q_stack, the prefix and suffix tables
// and lengths, the sequence slots, then both passes' partials; each part
// 256-byte aligned. Fills *ws when base is non-null; returns the total.
size_t shared_prefix_layout(char *base, int B, int G, int M, int Hq, int d, int mbs, int q_bytes,
                            int a_splits, int b_splits, pa::SharedPrefixWorkspace *ws) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char *p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  const size_t a_pieces = (size_t)Hq * M * ((size_t)a_splits + G);
  const size_t b_pieces = (size_t)Hq * ((size_t)b_splits + B);
  char *q_stack = take((size_t)G * Hq * M * d * q_bytes);
  char *prefix_tables = take((size_t)G * mbs * 4);
  char *prefix_ctx = take((size_t)G * 4);
  char *suffix_tables = take((size_t)B * mbs * 4);
  char *suffix_lens = take((size_t)B * 4);
  char *seq_slot = take((size_t)B * 4);
  char *a_out = take(a_pieces * d * 4);
  char *a_max = take(a_pieces * 4);
  char *a_sum = take(a_pieces * 4);
  char *b_out = take(b_pieces * d * 4);
  char *b_max = take(b_pieces * 4);
  char *b_sum = take(b_pieces * 4);
  if (ws) {
    ws->q_stack = q_stack;
    ws->prefix_tables = reinterpret_cast<int32_t *>(prefix_tables);
    ws->prefix_ctx = reinterpret_cast<int32_t *>(prefix_ctx);
    ws->suffix_tables = reinterpret_cast<int32_t *>(suffix_tables);
    ws->suffix_lens = reinterpret_cast<int32_t *>(suffix_lens);
    ws->seq_slot = reinterpret_cast<int32_t *>(seq_slot);
    ws->a_out = reinterpret_cast<float *>(a_out);
    ws->a_max = reinterpret_cast<float *>(a_max);
    ws->a_sum = reinterpret_cast<float *>(a_sum);
    ws->b_out = reinterpret_cast<float *>(b_out);
    ws->b_max = reinterpret_cast<float *>(b_max);
    ws->b_sum = reinterpret_cast<float *>(b_sum);
  }
  return off;
}

}  // namespace

extern "C" {

size_t pa_decode_shared_prefix_workspace_size(int num_seqs, int num_groups, int group_size,
                                              int num_q_heads, int head_dim,
                                              int max_blocks_per_seq, int q_dtype) {
  if (num_seqs <= 0 || num_groups <= 0 || group_size <= 0 || num_q_heads <= 0 ||
      head_dim <= 0 || max_blocks_per_seq <= 0 || !known_dtype(q_dtype) ||
      quantised(q_dtype))
    return 0;
  return shared_prefix_layout(nullptr, num_seqs, num_groups, group_size, num_q_heads, head_dim,
                              max_blocks_per_seq, elem_bytes(q_dtype), pa::kMaxAutoSplits,
                              pa::kMaxAutoSplits, nullptr);
}

pa_status pa_decode_shared_prefix(void *out, const void *q, const void *k_cache,
                                  const void *v_cache, const int32_t *block_tables,
                                  const int32_t *context_lens, const int32_t *group_members,
                                  const int32_t *prefix_lens, int num_seqs, int num_groups,
                                  int group_size, int num_q_heads, int num_kv_heads,
                                  int head_dim, int block_size, int num_blocks,
                                  int max_blocks_per_seq, float scale, int q_dtype,
                                  int kv_dtype, float k_scale, float v_scale, void *workspace,
                                  size_t workspace_bytes, void *stream) {
  if (!out || !group_members || !prefix_lens) return PA_ERR_NULL_POINTER;
  pa_status st = check_decode(q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                              num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                              max_blocks_per_seq, scale, q_dtype, kv_dtype, k_scale, v_scale, -1);
  if (st != PA_OK) return st;
  if (num_groups <= 0 || group_size <= 0) return PA_ERR_BAD_SHAPE;
  if (num_groups > pa::kMaxBalancedSeqs) return PA_ERR_UNSUPPORTED;
  // the prefix pass has group_size times the query heads
  const long long hq_stacked = (long long)num_q_heads * group_size;
  if (hq_stacked > INT_MAX / 2 || (long long)num_groups * group_size > INT_MAX / 2)
    return PA_ERR_UNSUPPORTED;
  const int gs = (int)(hq_stacked / num_kv_heads);
  if ((long long)num_kv_heads * (gs / pa::heads_per_workgroup(gs)) > 65535)
    return PA_ERR_UNSUPPORTED;
  if (!workspace) return PA_ERR_NULL_POINTER;
  if (num_seqs == 0) return PA_OK;
  pa::SharedPrefixLaunch a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.group_members = group_members;
  a.prefix_lens = prefix_lens;
  a.num_seqs = num_seqs;
  a.num_groups = num_groups;
  a.group_size = group_size;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.scale = resolve_scale(scale, head_dim);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.q_dtype = q_dtype;
  a.kv_dtype = kv_dtype;
  a.q_elem_bytes = elem_bytes(q_dtype);
  pa::DecodeLaunch probe{};
  probe.q_dtype = q_dtype;
  probe.kv_dtype = kv_dtype;
  probe.head_dim = head_dim;
  probe.num_kv_heads = num_kv_heads;
  probe.num_q_heads = (int)hq_stacked;
  a.prefix_splits = pa::balanced_num_splits(probe);
  a.suffix_splits = 0;  // the suffix pass is a single pass: B x Hq partials
  const size_t need = shared_prefix_layout(nullptr, num_seqs, num_groups, group_size, num_q_heads,
                                           head_dim, max_blocks_per_seq, a.q_elem_bytes,
                                           a.prefix_splits, a.suffix_splits, nullptr);
  if (workspace_bytes < need) return PA_ERR_WORKSPACE_TOO_SMALL;
  shared_prefix_layout(static_cast<char *>(workspace), num_seqs, num_groups, group_size,
                       num_q_heads, head_dim, max_blocks_per_seq, a.q_elem_bytes,
                       a.prefix_splits, a.suffix_splits, &a.ws);
  return status_of(pa::launch_shared_prefix(a, stream));
}

}  // extern "C"

extern "C" {

pa_status pa_prefill(void *out, const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *block_tables, const int32_t *context_lens,
                     const int32_t *query_start, int num_seqs, int total_query_tokens,
                     int max_query_len, int num_q_heads, int num_kv_heads, int head_dim,
                     int block_size, int num_blocks, int max_blocks_per_seq, float scale,
                     int q_dtype, int kv_dtype, float k_scale, float v_scale, void *stream) {
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return PA_ERR_NULL_POINTER;
  if (num_seqs < 0 || total_query_tokens < 0 || max_query_len < 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0)
    return PA_ERR_BAD_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_BAD_SHAPE;
  if (!known_dtype(q_dtype) || !known_dtype(kv_dtype)) return PA_ERR_UNSUPPORTED;
  // 16-bit queries; caches of the query's type or 8-bit codes
  if (q_dtype != PA_F16 && q_dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (kv_dtype != q_dtype && !quantised(kv_dtype)) return PA_ERR_UNSUPPORTED;
  if (!supported_head_dim(head_dim) || pa::sub_block_log2(block_size) < 0)
    return PA_ERR_UNSUPPORTED;
  if (isinf(scale)) return PA_ERR_BAD_SHAPE;
  if (quantised(kv_dtype) && (!isfinite(k_scale) || !isfinite(v_scale))) return PA_ERR_BAD_SHAPE;
  const long long row_bytes = (long long)num_kv_heads * head_dim * elem_bytes(kv_dtype);
  if (row_bytes * 16 >= INT_MAX) return PA_ERR_UNSUPPORTED;
  if ((long long)num_blocks * (block_size / 16) > INT_MAX) return PA_ERR_UNSUPPORTED;
  if ((long long)max_blocks_per_seq * block_size > INT_MAX) return PA_ERR_UNSUPPORTED;
  const int group = num_q_heads / num_kv_heads;
  const int tq = pa::prefill_tokens_per_tile(group);
  const long long tiles = ((long long)max_query_len + tq - 1) / tq;
  const long long grid_y = (long long)num_kv_heads * group / (128 / tq);
  if (tiles * grid_y * num_seqs > (1ll << 30)) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || total_query_tokens == 0 || max_query_len == 0) return PA_OK;
  pa::PrefillLaunch a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_query_len = max_query_len;
  a.scale = resolve_scale(scale, head_dim);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.q_dtype = q_dtype;
  a.kv_dtype = kv_dtype;
  return status_of(pa::launch_prefill(a, stream));
}

}  // extern "C"

