/*
 * pa.h -- C ABI of libpa: paged-attention decode and its cache operations on
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes (restated from the pages; see each entry point):
 *
 *   - Attention is softmax(q K^T / sqrt(d_k)) V ("KV-Cache evolution",
 *     smallfiredragon.com, section 1). In decode, each sequence contributes
 *     one new query token that attends over all of its cached tokens ("vLLM
 *     inference principles", krshare.site, section on the two phases).
 *   - Grouped-query attention: query heads come in groups that share one K/V
 *     head ("KV-Cache evolution", section 3A). Query head h reads KV head
 *     h / (num_q_heads / num_kv_heads) (contiguous groups).
 *   - The KV cache is cut into fixed-size physical blocks; a per-sequence
 *     block table maps logical block j (tokens j*block_size ... in sequence
 *     order) to a physical block id ("PagedAttention deep dive", juejin.cn,
 *     section 2.1; "vLLM inference principles", block-table figure).
 *   - New tokens are written into the slot the host block manager assigned
 *     ("PagedAttention deep dive", section 2.2), and a block shared by several
 *     sequences is copied before one of them writes a different token into it
 *     (copy-on-write, "PagedAttention deep dive", section 2.3; "KV-cache
 *     sharing article", intelliparadigm.com, section 3.1).
 *
 * Conventions shared by every entry point:
 *
 *   - Every data pointer is a DEVICE pointer to contiguous row-major memory
 *     owned by the caller. The library borrows it for the work it enqueues
 *     and keeps no reference afterwards; the caller keeps it alive until the
 *     stream has passed that work. The library allocates no memory and is
 *     reentrant; its process-wide data is a cache of device properties
 *     (compute-unit count, kernel occupancy) behind a mutex, and the fixed
 *     per-device scratch array of pa_decode_noalloc (the one entry point
 *     whose overlapping calls on a device race, see there).
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream. All work is enqueued asynchronously on it.
 *   - Cache layout: k_cache and v_cache are [num_blocks, block_size,
 *     num_kv_heads, head_dim], so one token's row of one KV head is head_dim
 *     contiguous elements.
 *   - Everything that can be checked on the host is checked before anything
 *     is enqueued, and a failed check returns a status without side effects.
 *     Contract breaches that live in device memory are NOT checked (block ids
 *     outside [0, num_blocks), context lengths above max_blocks_per_seq *
 *     block_size, duplicate slots in one call, overlapping copy pairs): their
 *     result is undefined.
 *   - A launch failure reported by the runtime returns PA_ERR_LAUNCH.
 *
 * Supported configurations: head_dim 64 or 128; block_size 16, 32, 64, 128
 * or 256 for decode (the pages give 16 as the usual size and suggest 16 to
 * 128, or 64 to 256: "PagedAttention deep dive" section 2.1, "KV-cache
 * sharing article" sections 2 and 4), and also 8 for pa_decode,
 * pa_decode_partials, pa_decode_noalloc and pa_decode_shared_prefix (not for
 * pa_decode_append, pa_decode_scaled or pa_prefill: PA_ERR_UNSUPPORTED); any
 * block size for the slot write and the block copy; any num_q_heads that is a
 * multiple of num_kv_heads; (q, kv) element types (f32, f32), (f16, f16),
 * (bf16, bf16), (f16, fp8_e4m3fn), (bf16, fp8_e4m3fn), (f16, int8),
 * (bf16, int8). Decode reads a block of 16 * 2^k tokens as 2^k consecutive
 * 16-token sub-blocks, and two consecutive 8-token blocks of a block table as
 * one 16-token unit.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL_POINTER = 1,      /* a required pointer is NULL                         */
  PA_ERR_BAD_SHAPE = 2,         /* a size is negative/zero where it may not be, or    */
                                /* sizes are inconsistent (Hq % Hkv != 0, ...)        */
  PA_ERR_UNSUPPORTED = 3,       /* valid but not built: head_dim, block_size, dtypes  */
  PA_ERR_WORKSPACE_TOO_SMALL = 4,
  PA_ERR_LAUNCH = 5,            /* the HIP runtime refused a kernel launch            */
  PA_ERR_SCRATCH_LIMIT = 6      /* pa_decode_noalloc: partials exceed its scratch     */
} pa_status;

/* Element types. fp8_e4m3fn is OCP E4M3FN (bias 7, max 448, no infinities).
 * int8 is a symmetric int8 code c in [-127, 127] standing for c * scale (the
 * pages name INT8 and FP8 KV quantisation: "PagedAttention deep dive",
 * section 4; "KV-Cache evolution", section 3C). Both 8-bit types are cache
 * types only, with one fp32 scale per tensor (k_scale, v_scale), or with a
 * table of scales per KV head, per block or per (block, KV head) (the
 * *_scaled entry points below). */
typedef enum pa_dtype {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_FP8_E4M3FN = 3,
  PA_INT8 = 4
} pa_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char *pa_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int pa_version(void);

/*
 * Context splitting. Every decode entry point takes a partition_size:
 *
 *   0      single pass: one workgroup reads a sequence's whole context.
 *   P > 0  fixed split: partition p of sequence b covers logical tokens
 *          [p*P, min((p+1)*P, n)); P is a multiple of block_size and
 *          of 16 (else PA_ERR_BAD_SHAPE, or PA_ERR_UNSUPPORTED for a
 *          multiple of 8 that is not one of 16).
 *   -S     balanced split with S >= 2 shares: the 16-token sub-blocks of
 *          all sequences (whatever the block size), taken end to end in
 *          sequence order (ceil(n_b / 16) of them for sequence b, T in
 *          total), are cut into S shares, share
 *          s being blocks [floor(s*T/S), floor((s+1)*T/S)) (S is first
 *          clamped to T). Each piece = (share, sequence) intersection is one
 *          partial; every share holds the same number of blocks, so the work
 *          is even whatever the length mix. At most 1024 sequences.
 *   -1     (pa_decode only) balanced split with the share count that fills
 *          every compute unit of the current device once:
 *          pa_decode_balanced_splits(...).
 *
 * Splits change only the order of the floating-point reductions, never the
 * mathematical result. The balanced split of one sequence depends on the
 * other sequences' lengths (through T).
 */

/*
 * Number of partitions a fixed split uses for a block table of
 * max_blocks_per_seq entries: ceil(max_blocks_per_seq * block_size /
 * partition_size). Returns 0 for partition_size <= 0.
 */
int pa_num_partitions(int max_blocks_per_seq, int block_size, int partition_size);

/*
 * Share count of the automatic balanced split (partition_size = -1) on the
 * current device for this head and type configuration: the number of
 * workgroups that fill every compute unit once (one workgroup per unit for
 * the four-wave kernels, which measured faster than two; as many as fit
 * otherwise), divided by the workgroups per share (num_kv_heads *
 * query-head runs), at least 2 and at most 2048. Returns 0 for an
 * unsupported configuration. Queries the device (HIP runtime) on first use.
 */
int pa_decode_balanced_splits(int num_q_heads, int num_kv_heads, int head_dim, int q_dtype,
                              int kv_dtype);

/*
 * Bytes of device workspace pa_decode needs:
 *   partition_size == 0: 0;
 *   P > 0:  num_seqs * num_q_heads * NP * (head_dim + 2) * 4, NP as above;
 *   -S:     num_q_heads * (S + num_seqs) * (head_dim + 2) * 4, with S = 2048
 *           (the largest automatic choice) for partition_size = -1.
 */
size_t pa_decode_workspace_size(int num_seqs, int num_q_heads, int head_dim,
                                int max_blocks_per_seq, int block_size,
                                int partition_size);

/*
 * pa_decode -- one decode step of paged attention.
 *
 * For every sequence b and query head h, with n = context_lens[b] and
 * g = h / (num_q_heads / num_kv_heads):
 *
 *   s_j     = scale * k_scale * < q[b, h, :], K[j] >        for j < n,
 *   out[b,h] = v_scale * sum_j exp(s_j - max s) V[j] / sum_j exp(s_j - max s),
 *
 * where K[j] / V[j] is row (block_tables[b, j / block_size], j % block_size,
 * g, :) of k_cache / v_cache. A sequence with n == 0 gets out[b] = 0.
 * Sources: the attention formula ("KV-Cache evolution", section 1); the
 * block-table gather ("PagedAttention deep dive", section 2.1; "vLLM
 * inference principles", block-table figure); fp8 storage of the cache
 * ("PagedAttention deep dive", sections 3.2 and 4; "KV-Cache evolution",
 * section 3C) with per-tensor scales k_scale / v_scale (ignored unless
 * kv_dtype is PA_FP8_E4M3FN or PA_INT8: an 8-bit code then stands for its
 * value times the scale).
 *
 *   out           [num_seqs, num_q_heads, head_dim], q_dtype; must not alias
 *                 any input.
 *   q             [num_seqs, num_q_heads, head_dim], q_dtype.
 *   k_cache/v_cache [num_blocks, block_size, num_kv_heads, head_dim], kv_dtype;
 *                 never written.
 *   block_tables  [num_seqs, max_blocks_per_seq] int32; only the first
 *                 ceil(n / block_size) entries of row b are read.
 *   context_lens  [num_seqs] int32, each in [0, max_blocks_per_seq*block_size].
 *   scale         softmax scale. A NaN selects the attention formula's
 *                 1/sqrt(d_k): the float32 nearest to 1/sqrt(head_dim). An
 *                 infinite scale gives PA_ERR_BAD_SHAPE. (The same holds for
 *                 every decode entry point below.)
 *   partition_size see "Context splitting" above. A split decode runs the
 *                 partial kernel into `workspace` (a sequence that falls in
 *                 one piece is written to `out` directly), then the merge
 *                 kernel into `out`, on the same stream.
 *   workspace     device buffer of at least pa_decode_workspace_size(...)
 *                 bytes when partition_size != 0 (may be NULL otherwise). Its
 *                 contents on entry do not matter; one call at a time may use
 *                 a given workspace.
 */
pa_status pa_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, const int32_t *context_lens,
                    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                    int block_size, int num_blocks, int max_blocks_per_seq,
                    float scale, int q_dtype, int kv_dtype, float k_scale, float v_scale,
                    int partition_size, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * pa_decode_noalloc -- pa_decode without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.
 *
 * Arguments, result and errors as pa_decode. A split decode
 * (partition_size != 0) keeps its partials in a fixed device array inside
 * the library, pa_decode_noalloc_scratch_bytes() bytes (16 MiB) per device,
 * held until the process ends; no memory is allocated per call. A split
 * whose partials exceed it returns PA_ERR_SCRATCH_LIMIT without enqueuing
 * anything (the partials need pa_decode_workspace_size(...) bytes, with the
 * share count resolved: num_q_heads * (S + num_seqs) * (head_dim + 2) * 4
 * for the balanced split, e.g. 1.6 MB for 32 sequences, 32 query heads,
 * head_dim 128 and 64 shares). The array is shared by every call on a
 * device: calls that overlap on one device (different streams or host
 * threads without ordering between them) race on it; calls ordered on one
 * stream do not. Nothing in it needs clearing between calls (every partial
 * is written before it is read). The first split call on a device looks up
 * the array's address (hipGetSymbolAddress); a failure there returns
 * PA_ERR_LAUNCH.
 */
pa_status pa_decode_noalloc(void *out, const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, const int32_t *context_lens,
                            int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                            int block_size, int num_blocks, int max_blocks_per_seq, float scale,
                            int q_dtype, int kv_dtype, float k_scale, float v_scale,
                            int partition_size, void *stream);

/* Bytes of the fixed per-device scratch pa_decode_noalloc uses. */
size_t pa_decode_noalloc_scratch_bytes(void);

/*
 * pa_decode_append -- one decode step with the new token appended.
 *
 * The decode phase ("vLLM inference principles", two phases: decode) extends
 * each sequence's cache by the new token's K/V and then lets its query attend
 * over the whole context, the new token included. Here the new token of
 * sequence b is its last position, n - 1 with n = context_lens[b] > 0:
 *
 *   1. key[b], value[b] are written to slot
 *        block_tables[b][(n - 1) / block_size] * block_size + (n - 1) % block_size
 *      of k_cache / v_cache, exactly as pa_reshape_and_cache writes them
 *      (a bit copy, or fp8 e4m3fn of x / k_scale resp. x / v_scale);
 *   2. out = pa_decode(...) over the caches after that write.
 *
 * Both happen in one kernel launch (plus the merge of a split): the
 * workgroups that attend over a sequence's last block take the new token's
 * rows from key / value and one of them writes them to the cache. The result
 * (caches and out) equals pa_reshape_and_cache with those slots followed by
 * pa_decode, bit for bit.
 *
 * Arguments as pa_decode, plus:
 *   key, value    [num_seqs, num_kv_heads, head_dim], device, in q_dtype. Rows
 *                 of sequences with n = 0 are not read.
 *   k_cache, v_cache  written at the new tokens' slots only.
 * The block holding position n - 1 must be private to sequence b (copy a
 * shared block with pa_copy_blocks first). fp8 caches need finite, non-zero
 * k_scale and v_scale (PA_ERR_BAD_SHAPE otherwise); NULL key or value gives
 * PA_ERR_NULL_POINTER. Other errors as pa_decode.
 */
pa_status pa_decode_append(void *out, const void *q, const void *key, const void *value,
                           void *k_cache, void *v_cache, const int32_t *block_tables,
                           const int32_t *context_lens, int num_seqs, int num_q_heads,
                           int num_kv_heads, int head_dim, int block_size, int num_blocks,
                           int max_blocks_per_seq, float scale, int q_dtype, int kv_dtype,
                           float k_scale, float v_scale, int partition_size, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * pa_decode_partials -- the per-piece half of split-context decode.
 *
 * For each piece (a fixed partition p of sequence b, or a balanced-split
 * piece: share s intersected with sequence b) over logical tokens J and each
 * query head h, it writes in float32
 *
 *   max_logits = m = max_{j in J} s_j                       (s_j as in pa_decode)
 *   exp_sums   = l = sum_{j in J} exp(s_j - m)
 *   tmp_out    =     sum_{j in J} exp(s_j - m) * v_scale * V[j] / l
 *
 * Fixed split (partition_size = P > 0): entry [b, h, p] for p < ceil(n / P);
 *   tmp_out [num_seqs, num_q_heads, max_partitions, head_dim],
 *   max_logits / exp_sums [num_seqs, num_q_heads, max_partitions],
 *   max_partitions >= pa_num_partitions(max_blocks_per_seq, block_size, P).
 * Balanced split (partition_size = -S, S >= 2; -1 is refused here: resolve
 * the automatic count with pa_decode_balanced_splits first): entry
 * [h, s + b] for each non-empty piece (s, b);
 *   tmp_out [num_q_heads, max_partitions, head_dim],
 *   max_logits / exp_sums [num_q_heads, max_partitions],
 *   max_partitions >= S + num_seqs.
 * Other entries are not written. Merging the pieces of a sequence
 * (pa_decode_reduce) gives the same attention as pa_decode; the pieces of
 * one sequence may also be produced on different devices and merged
 * afterwards. Other arguments as in pa_decode.
 */
pa_status pa_decode_partials(float *tmp_out, float *max_logits, float *exp_sums,
                             int max_partitions, const void *q, const void *k_cache,
                             const void *v_cache, const int32_t *block_tables,
                             const int32_t *context_lens, int num_seqs, int num_q_heads,
                             int num_kv_heads, int head_dim, int block_size, int num_blocks,
                             int max_blocks_per_seq, float scale, int q_dtype, int kv_dtype,
                             float k_scale, float v_scale, int partition_size, void *stream);

/*
 * pa_decode_reduce -- merge split-context partials into the decode output.
 *
 * For each (b, h), over the pieces of sequence b (fixed split: the first
 * ceil(n / P) partitions; balanced split: the shares s0..s1 that hold its
 * blocks): M = max_p m_p, w_p = l_p * exp(m_p - M), out[b, h] =
 * sum_p w_p * tmp_out[p] / sum_p w_p, rounded to out_dtype (round to nearest
 * even). n == 0 gives 0.
 *
 *   out          [num_seqs, num_q_heads, head_dim], out_dtype (f32, f16, bf16)
 *   tmp_out, max_logits, exp_sums, max_partitions, partition_size: as given
 *                to pa_decode_partials (same context_lens).
 *   head_dim     64 or 128.
 */
pa_status pa_decode_reduce(void *out, const float *tmp_out, const float *max_logits,
                           const float *exp_sums, const int32_t *context_lens,
                           int num_seqs, int num_q_heads, int head_dim, int max_partitions,
                           int partition_size, int out_dtype, void *stream);

/*
 * pa_reshape_and_cache -- write new tokens' K/V rows into their slots.
 *
 * For each token t with s = slot_mapping[t] >= 0:
 *   k_cache[s / block_size, s % block_size, :, :] = enc(key[t, :, :], k_scale)
 *   v_cache[s / block_size, s % block_size, :, :] = enc(value[t, :, :], v_scale)
 * enc is a bit copy when cache_dtype == src_dtype; for an fp8 cache it is
 * E4M3FN(float32(x) / scale) with a correctly rounded float32 division,
 * round-to-nearest-even and saturation to +-448 (NaN -> 0x7F | sign).
 * Tokens with a negative slot are skipped. Sources: "PagedAttention deep
 * dive", section 2.2 (a sequence fills its current block, then a new one);
 * "vLLM inference principles", two phases (decode extends the cache).
 *
 *   key, value    [num_tokens, num_kv_heads, head_dim], src_dtype (f32, f16,
 *                 bf16)
 *   k_cache, v_cache [num_blocks, block_size, num_kv_heads, head_dim],
 *                 cache_dtype == src_dtype, or PA_FP8_E4M3FN / PA_INT8 from
 *                 f16/bf16/f32: fp8 e4m3fn(x / scale) rounded to nearest even
 *                 and saturated to +-448, or int8 rint(x / scale) (ties to
 *                 even) saturated to [-127, 127] (NaN -> 0), the division in
 *                 IEEE float32
 *   slot_mapping  [num_tokens] int64, slots distinct among non-negative entries
 * num_tokens == 0 is a no-op (key, value and slot_mapping may then be NULL).
 */
pa_status pa_reshape_and_cache(const void *key, const void *value, void *k_cache,
                               void *v_cache, const int64_t *slot_mapping, int num_tokens,
                               int num_kv_heads, int head_dim, int block_size, int num_blocks,
                               int src_dtype, int cache_dtype, float k_scale, float v_scale,
                               void *stream);

/*
 * pa_copy_blocks -- copy-on-write block copies.
 *
 * For each pair i: k_cache[dst_i] = k_cache[src_i] and v_cache[dst_i] =
 * v_cache[src_i], bit for bit, where (src_i, dst_i) = block_mapping[i, :].
 * Destinations must be distinct and never a source of the same call (the
 * result then does not depend on pair order). Sources: "PagedAttention deep
 * dive", section 2.3; "KV-cache sharing article", section 3.1.
 *
 *   block_mapping [num_pairs, 2] int64, device memory
 *   cache_dtype   element type of both caches (only its size matters)
 * num_pairs == 0 is a no-op (block_mapping may then be NULL).
 */
pa_status pa_copy_blocks(void *k_cache, void *v_cache, const int64_t *block_mapping,
                         int num_pairs, int num_kv_heads, int head_dim, int block_size,
                         int num_blocks, int cache_dtype, void *stream);

/*
 * 8-bit caches with scale tables.
 *
 * The pages name INT8 and FP8 storage of the KV cache, combined with paging,
 * to shrink each cache unit ("PagedAttention deep dive", section 4 item 1;
 * "KV-Cache evolution", section 3C; "KV-cache sharing article", section 6),
 * but not the granularity of the scales. Besides one scale per tensor, the
 * library takes a table of float32 scales, one per KV head, per physical
 * block, or per (physical block, KV head): a code c of KV head g in physical
 * block e stands for value(c) * S[e, g], where S is the table read through
 * its layout:
 *
 *   PA_SCALE_PER_HEAD        k_scales[num_kv_heads]:            S[e, g] = k_scales[g]
 *   PA_SCALE_PER_BLOCK       k_scales[num_blocks]:              S[e, g] = k_scales[e]
 *   PA_SCALE_PER_BLOCK_HEAD  k_scales[num_blocks, num_kv_heads]: S[e, g] = k_scales[e, g]
 *
 * and likewise v_scales for V. A block's scales are the scales of its
 * contents: the slot write quantises with them, decode dequantises with
 * them, and a copy-on-write copy carries them to the new block. How the
 * scales are chosen (e.g. a block's largest magnitude over the codec's
 * largest code, fixed before the block's first write) is the caller's
 * policy; the library only applies them. The tables are device memory;
 * their values are not checked (a zero, negative or non-finite scale gives
 * the corresponding non-finite or sign-flipped values).
 */
typedef enum pa_scale_layout {
  PA_SCALE_PER_HEAD = 1,
  PA_SCALE_PER_BLOCK = 2,
  PA_SCALE_PER_BLOCK_HEAD = 3
} pa_scale_layout;

/*
 * pa_reshape_and_cache_scaled -- pa_reshape_and_cache into an 8-bit cache
 * with scale tables: for each token t with s = slot_mapping[t] >= 0 and each
 * KV head g, with e = s / block_size,
 *   k_cache[e, s % block_size, g, :] = enc(key[t, g, :], S_k[e, g])
 *   v_cache[e, s % block_size, g, :] = enc(value[t, g, :], S_v[e, g])
 * with enc as in pa_reshape_and_cache (correctly rounded float32 division,
 * round to nearest even, saturation).
 *
 *   cache_dtype   PA_FP8_E4M3FN or PA_INT8; src_dtype f32, f16 or bf16, with
 *                 head_dim * sizeof(src element) a multiple of 16 bytes.
 *   k_scales, v_scales  device float32 tables of scale_layout (read only).
 * Errors: PA_ERR_NULL_POINTER for missing tables; PA_ERR_BAD_SHAPE for an
 * unknown layout; PA_ERR_UNSUPPORTED for other cache or source types; others
 * as pa_reshape_and_cache.
 */
pa_status pa_reshape_and_cache_scaled(const void *key, const void *value, void *k_cache,
                                      void *v_cache, const int64_t *slot_mapping,
                                      int num_tokens, int num_kv_heads, int head_dim,
                                      int block_size, int num_blocks, int src_dtype,
                                      int cache_dtype, const float *k_scales,
                                      const float *v_scales, int scale_layout, void *stream);

/*
 * pa_copy_blocks_scaled -- pa_copy_blocks for an 8-bit cache with scale
 * tables: each pair copies the block's codes and, for PA_SCALE_PER_BLOCK
 * and PA_SCALE_PER_BLOCK_HEAD, its scale entries (k_scales[dst] =
 * k_scales[src], one entry or num_kv_heads entries; likewise v_scales), all
 * from the state before the call. A PA_SCALE_PER_HEAD table has no
 * per-block entries and is not touched. Errors as pa_copy_blocks, plus
 * PA_ERR_NULL_POINTER for missing tables and PA_ERR_BAD_SHAPE for an unknown
 * layout.
 */
pa_status pa_copy_blocks_scaled(void *k_cache, void *v_cache, float *k_scales, float *v_scales,
                                const int64_t *block_mapping, int num_pairs, int num_kv_heads,
                                int head_dim, int block_size, int num_blocks, int cache_dtype,
                                int scale_layout, void *stream);

/*
 * pa_decode_scaled -- pa_decode over an 8-bit cache with scale tables:
 *
 *   s_j      = scale * S_k[e_j, g] * < q[b, h, :], K[j] >
 *   out[b,h] = sum_j exp(s_j - max s) S_v[e_j, g] V[j] / sum_j exp(s_j - max s)
 *
 * where e_j = block_tables[b, j / block_size] is the physical block holding
 * token j and K[j], V[j] are its codes' values. Arguments, splitting,
 * workspace and errors as pa_decode, with kv_dtype PA_FP8_E4M3FN or PA_INT8
 * (PA_ERR_UNSUPPORTED otherwise) and the tables in place of k_scale /
 * v_scale (PA_ERR_NULL_POINTER when missing, PA_ERR_BAD_SHAPE for an unknown
 * layout). The decode kernels multiply each 16-token unit's logits by its
 * block's K scale and its probabilities by its V scale before P.V (the
 * softmax sums use the probabilities alone).
 */
pa_status pa_decode_scaled(void *out, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *block_tables, const int32_t *context_lens,
                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int block_size, int num_blocks, int max_blocks_per_seq, float scale,
                           int q_dtype, int kv_dtype, const float *k_scales,
                           const float *v_scales, int scale_layout, int partition_size,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_decode_shared_prefix -- decode for groups of sequences that share a
 * prompt prefix, reading each shared block once per group.
 *
 * Sequences forked from one prompt (parallel sampling, beam search) hold the
 * prompt's blocks by reference ("PagedAttention deep dive", section 2.3;
 * "KV-cache sharing article", sections 3.1 and 4.2). Group g lists its
 * member sequences in group_members[g, 0 .. group_size) (-1 marks an empty
 * slot; every sequence is in at most one group) and its shared prefix length
 * prefix_lens[g] in tokens. The result is the same attention as pa_decode
 * for every sequence (up to floating-point rounding order):
 *
 *   out[b, h, :] = softmax(scale * q[b, h] . K_b^T) V_b over all context_lens[b]
 *                  tokens of sequence b.
 *
 * It is computed in two passes: the prefix of each group, in the balanced
 * split, with the members' query rows stacked as extra query heads of each
 * KV head (so a prefix block is read once for all members), and each
 * sequence's suffix past its group's prefix, in a single pass; then the
 * pieces of both passes are merged with their softmax statistics, as in
 * pa_decode_reduce.
 *
 * Arguments as pa_decode (balanced split), plus
 *   group_members  [num_groups, group_size] int32, device: sequence ids.
 *   prefix_lens    [num_groups] int32, device: shared prefix tokens of each
 *                  group. Only whole blocks count: the prefix used is
 *                  floor(prefix_lens[g] / block_size) blocks (capped at
 *                  max_blocks_per_seq); tokens past it are read per sequence.
 *   workspace      device scratch of at least
 *                  pa_decode_shared_prefix_workspace_size(...) bytes; its
 *                  contents are ignored and overwritten.
 *
 * Preconditions (device data, unchecked): the first prefix blocks of every
 * member's block table are the same physical blocks, and every member's
 * context length is at least its group's prefix; a sequence appears in at
 * most one slot. Sequences in no group are decoded over their whole context.
 * num_seqs and num_groups at most 1024; q_dtype f32, f16 or bf16 (the output
 * type).
 *
 * Errors: as pa_decode; PA_ERR_BAD_SHAPE for num_groups or group_size < 1;
 * PA_ERR_NULL_POINTER without group_members, prefix_lens or workspace;
 * PA_ERR_WORKSPACE_TOO_SMALL.
 */
size_t pa_decode_shared_prefix_workspace_size(int num_seqs, int num_groups, int group_size,
                                              int num_q_heads, int head_dim,
                                              int max_blocks_per_seq, int q_dtype);

pa_status pa_decode_shared_prefix(void *out, const void *q, const void *k_cache,
                                  const void *v_cache, const int32_t *block_tables,
                                  const int32_t *context_lens, const int32_t *group_members,
                                  const int32_t *prefix_lens, int num_seqs, int num_groups,
                                  int group_size, int num_q_heads, int num_kv_heads,
                                  int head_dim, int block_size, int num_blocks,
                                  int max_blocks_per_seq, float scale, int q_dtype,
                                  int kv_dtype, float k_scale, float v_scale, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * pa_prefill -- paged prefill and chunked prefill: many new query tokens per
 * sequence attend causally over the sequence's paged K/V.
 *
 * Prefill processes a request's input tokens and builds their K/V state
 * before decode extends it one token at a time; a long input may be cut
 * into chunks that are scheduled beside decode work ("vLLM inference
 * principles", section on the two phases of one generation; "PagedAttention
 * deep dive", section 1, on the compute/memory asymmetry of the phases).
 * For sequence b let n = context_lens[b] and C = query_start[b + 1] -
 * query_start[b]: the chunk is the sequence's last C tokens, their K/V
 * already written to the cache (pa_reshape_and_cache), and query row
 * query_start[b] + i (i < C) sits at position n - C + i. With g = h /
 * (num_q_heads / num_kv_heads):
 *
 *   out[r, h] = softmax_j(scale * k_scale * < q[r, h], K[j] >) v_scale V[j]
 *               over j = 0 .. n - C + i (causal),
 *
 * K[j] / V[j] being row (block_tables[b, j / block_size], j % block_size, g,
 * :) of k_cache / v_cache ("KV-Cache evolution", sections 1 and 3A;
 * "PagedAttention deep dive", section 2.1). C = n is a whole prompt; C = 1
 * is one decode step.
 *
 *   out           [total_query_tokens, num_q_heads, head_dim], q_dtype; must
 *                 not alias an input.
 *   q             [total_query_tokens, num_q_heads, head_dim], f16 or bf16.
 *   k_cache/v_cache [num_blocks, block_size, num_kv_heads, head_dim]: the
 *                 query's type, or fp8_e4m3fn / int8 codes (k_scale,
 *                 v_scale as in pa_decode); never written.
 *   block_tables  [num_seqs, max_blocks_per_seq] int32; only the blocks
 *                 holding positions < n are read.
 *   context_lens  [num_seqs] int32.
 *   query_start   [num_seqs + 1] int32, device: query_start[0] = 0,
 *                 non-decreasing, query_start[num_seqs] = total_query_tokens,
 *                 each chunk C <= n.
 *   max_query_len at least the longest chunk (the launch grid covers this
 *                 many query tokens per sequence).
 *   scale         as in pa_decode (NaN: 1/sqrt(head_dim)).
 * Supported: head_dim 64 or 128, the block sizes of pa_decode, any GQA group.
 * The device-data preconditions (query_start, C <= n, block ids, n within
 * the table) are unchecked. Errors as pa_decode; a zero chunk total is a
 * no-op. Computed on MFMA with fp32 accumulation; the probabilities enter
 * the P.V product rounded to the query's 16-bit type.
 */
pa_status pa_prefill(void *out, const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *block_tables, const int32_t *context_lens,
                     const int32_t *query_start, int num_seqs, int total_query_tokens,
                     int max_query_len, int num_q_heads, int num_kv_heads, int head_dim,
                     int block_size, int num_blocks, int max_blocks_per_seq, float scale,
                     int q_dtype, int kv_dtype, float k_scale, float v_scale, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
