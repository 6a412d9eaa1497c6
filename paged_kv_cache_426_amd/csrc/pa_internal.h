// Host-side launch interface between the C ABI (pa_api.cpp) and the gfx950
// kernels. Plain C++: no HIP types, so the validation unit stays host-only.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pa {

struct DecodeLaunch {
  // outputs: single pass writes `out`; split writes the three partial arrays
  void *out;
  float *tmp_out;
  float *max_logits;
  float *exp_sums;
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
  int partition_size;  // 0 = single pass
};

// Each returns 0 on success or the runtime's error code.
int launch_decode(const DecodeLaunch &a, void *stream);
int launch_reduce(void *out, const float *tmp_out, const float *max_logits,
                  const float *exp_sums, const int32_t *context_lens, int num_seqs,
                  int num_q_heads, int head_dim, int max_partitions, int partition_size,
                  int out_dtype, void *stream);
int launch_reshape_and_cache(const void *key, const void *value, void *k_cache, void *v_cache,
                             const int64_t *slot_mapping, int num_tokens, int num_kv_heads,
                             int head_dim, int src_dtype, int cache_dtype, float k_scale,
                             float v_scale, void *stream);
int launch_copy_blocks(void *k_cache, void *v_cache, const int64_t *block_mapping,
                       int num_pairs, size_t block_bytes, void *stream);

// heads of one KV group that one workgroup serves (a divisor of the group, <= 8)
inline int heads_per_workgroup(int group) {
  return group % 8 == 0 ? 8 : group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
}

}  // namespace pa
