// Shared-prefix decode for gfx950: sequences forked from one prompt share the
// prompt's cache blocks by reference ("PagedAttention deep dive" §2.3;
// "KV-cache sharing article" §3.1, shared prompt blocks stored once), and
// here they are also READ once. Attention over a sequence's context splits
// exactly into attention over the shared prefix and over its own suffix,
// merged by the softmax statistics (m, l) of the two parts, so:
//
//   1. prep_kernel: per group, the members' query rows are stacked as extra
//      query heads of each KV head (member-major inside a KV group), the
//      prefix's block-table row is taken from a member, and every sequence
//      gets a suffix table (its table past the prefix) and suffix length;
//   2. the balanced-split decode kernel over the groups' prefixes, with
//      group_size times the query heads: each prefix block is read once for
//      all members of its group;
//   3. the same kernel over every sequence's suffix, in a single pass (one
//      partial per sequence and query head: a suffix is a few blocks, too
//      short for the balanced split's preamble to pay off);
//   4. merge_kernel: per sequence and query head, the pieces of both passes
//      merged into the output.
//
// Only the reading order changes; the result is the sequence's plain decode
// (up to floating-point rounding order).

#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPrepThreads = 256;
constexpr int kMergeThreads = 256;
constexpr float kLog2eP = 1.4426950408889634f;

struct PrepParams {
  const uint8_t *q;         // [B, Hq, d]
  uint8_t *q_stack;         // [G, Hq * M, d]
  const int32_t *block_tables;   // [B, MBS]
  const int32_t *context_lens;   // [B]
  const int32_t *members;        // [G, M]
  const int32_t *prefix_lens;    // [G]
  int32_t *prefix_tables;        // [G, MBS]
  int32_t *prefix_ctx;           // [G]
  int32_t *suffix_tables;        // [B, MBS]
  int32_t *suffix_lens;          // [B]
  int32_t *seq_slot;             // [B]: g * M + m, or -1
  int num_seqs, num_groups, group_size, num_q_heads, gqa, row_bytes, mbs, block_size;
};

// A group's prefix as the kernels use it: whole blocks, within the table.
__device__ __forceinline__ int prefix_blocks(const PrepParams &p, int g) {
  const int pl = p.prefix_lens[g];
  return pl > 0 ? min(pl / p.block_size, p.mbs) : 0;
}

// Stacked query head of member m for query head h: KV head kv = h / gqa keeps
// its rows together, member-major: kv * (M * gqa) + m * gqa + h % gqa.
__device__ __forceinline__ int stacked_head(int h, int m, int M, int gqa) {
  return (h / gqa) * (M * gqa) + m * gqa + h % gqa;
}

// Workgroups [0, B): sequence b. Workgroups [B, B + G): group g.
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(const PrepParams p) {
  __shared__ int s_found;
  const int M = p.group_size;
  const int GM = p.num_groups * M;
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < p.num_seqs) {
    const int b = blockIdx.x;
    if (tid == 0) s_found = INT_MAX;
    __syncthreads();
    for (int i = tid; i < GM; i += kPrepThreads)
      if (p.members[i] == b) atomicMin(&s_found, i);
    __syncthreads();
    const int slot = s_found == INT_MAX ? -1 : s_found;
    const int g = slot >= 0 ? slot / M : 0;
    const int pb = slot >= 0 ? prefix_blocks(p, g) : 0;
    const int n = p.context_lens[b];
    const int32_t *row = p.block_tables + (size_t)b * p.mbs;
    int32_t *srow = p.suffix_tables + (size_t)b * p.mbs;
    for (int i = tid; i < p.mbs; i += kPrepThreads) srow[i] = pb + i < p.mbs ? row[pb + i] : 0;
    if (tid == 0) {
      p.suffix_lens[b] = max(0, n - pb * p.block_size);
      p.seq_slot[b] = slot;
    }
    if (slot >= 0) {
      // the sequence's query rows, 16 bytes per thread and step, all heads at once
      const int m = slot % M;
      const int per_row = p.row_bytes / 16;
      const int n16 = p.num_q_heads * per_row;
      const u32x4 *src = reinterpret_cast<const u32x4 *>(p.q + (size_t)b * p.num_q_heads * p.row_bytes);
      u32x4 *dst = reinterpret_cast<u32x4 *>(p.q_stack + (size_t)g * p.num_q_heads * M * p.row_bytes);
      for (int i = tid; i < n16; i += kPrepThreads) {
        const int h = i / per_row;
        dst[(size_t)stacked_head(h, m, M, p.gqa) * per_row + i % per_row] = src[i];
      }
    }
    return;
  }
  const int g = blockIdx.x - p.num_seqs;
  const int pb = prefix_blocks(p, g);
  // the prefix row comes from the group's first member (every member holds
  // the same blocks there)
  int first = -1;
  for (int m = M - 1; m >= 0; --m) {
    const int b = p.members[g * M + m];
    if (b >= 0 && b < p.num_seqs) first = b;
  }
  int32_t *prow = p.prefix_tables + (size_t)g * p.mbs;
  for (int i = tid; i < p.mbs; i += kPrepThreads)
    prow[i] = (first >= 0 && i < pb) ? p.block_tables[(size_t)first * p.mbs + i] : 0;
  if (tid == 0) p.prefix_ctx[g] = first >= 0 ? pb * p.block_size : 0;
  // rows of empty member slots are zero (their results are never read)
  for (int m = 0; m < M; ++m) {
    const int b = p.members[g * M + m];
    if (b >= 0 && b < p.num_seqs) continue;
    for (int h = 0; h < p.num_q_heads; ++h) {
      uint8_t *dst = p.q_stack +
                     ((size_t)g * p.num_q_heads * M + stacked_head(h, m, M, p.gqa)) * p.row_bytes;
      for (int i = tid; i < p.row_bytes / 16; i += kPrepThreads)
        reinterpret_cast<u32x4 *>(dst)[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// The pieces of sequence idx in a balanced split over lens[0 .. n): first
// column and count (see the library header's definition of the split). All
// threads of the workgroup call it.
__device__ __forceinline__ void balanced_span(const int32_t *lens, int n, int idx, int num_splits,
                                              int (*s_red)[kMergeThreads / kWave], int &first,
                                              int &np) {
  const int tid = threadIdx.x;
  auto nb = [](int x) { return x > 0 ? (x + 15) / 16 : 0; };
  int before = 0, all = 0;
  for (int i = tid; i < n; i += kMergeThreads) {
    const int c = nb(lens[i]);
    all += c;
    if (i < idx) before += c;
  }
  before = (int)group_sum_i<kWave>(before);
  all = (int)group_sum_i<kWave>(all);
  __syncthreads();
  if ((tid & (kWave - 1)) == 0) {
    s_red[0][tid >> 6] = before;
    s_red[1][tid >> 6] = all;
  }
  __syncthreads();
  int st = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kMergeThreads / kWave; ++w) {
    st += s_red[0][w];
    total += s_red[1][w];
  }
  const int nblk = nb(lens[idx]);
  first = 0;
  np = 0;
  if (nblk > 0) {
    const long long S = min(num_splits, total);
    const int s0 = (int)(((long long)(st + 1) * S - 1) / total);
    const int s1 = (int)(((long long)(st + nblk) * S - 1) / total);
    first = s0 + idx;
    np = s1 - s0 + 1;
  }
}

struct MergeParams {
  void *out;
  // prefix pass: per stacked head, columns of its balanced split over the groups
  const float *a_out, *a_max, *a_sum;
  int a_cols, a_splits;
  const int32_t *prefix_ctx;
  // suffix pass: one partial per (sequence, query head), [B, Hq]
  const float *b_out, *b_max, *b_sum;
  const int32_t *suffix_lens;
  const int32_t *seq_slot;
  int num_seqs, num_groups, group_size, num_q_heads, gqa;
};

template <int OT, int D>
__device__ __forceinline__ void store_out(void *out, size_t idx, float v) {
  if constexpr (OT == PA_F32) static_cast<float *>(out)[idx] = v;
  else if constexpr (OT == PA_BF16) static_cast<uint16_t *>(out)[idx] = f32_to_bf16_rne(v);
  else static_cast<uint16_t *>(out)[idx] = f32_to_f16_rne(v);
}

// One workgroup per (sequence, run of 256 / D query heads); thread = (head, d).
// The pieces are merged in a fixed order (prefix pieces, then suffix
// pieces): w_p = l_p exp(m_p - M), out = sum w_p o_p / sum w_p, with M the
// running maximum of the batches read so far.
template <int OT, int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const MergeParams p) {
  constexpr int HPW = kMergeThreads / D;
  __shared__ int s_red[2][kMergeThreads / kWave];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int h = blockIdx.y * HPW + tid / D;
  const int d = tid % D;
  const int M = p.group_size;
  const int slot = p.seq_slot[b];
  const int g = slot >= 0 ? slot / M : 0;
  int a_first, a_np;
  balanced_span(p.prefix_ctx, p.num_groups, g, p.a_splits, s_red, a_first, a_np);
  const int b_np = p.suffix_lens[b] > 0 ? 1 : 0;
  if (slot < 0) a_np = 0;
  if (h >= p.num_q_heads) return;
  const int hs = stacked_head(h, slot >= 0 ? slot % M : 0, M, p.gqa);
  const size_t a_base = (size_t)hs * p.a_cols + a_first;
  const size_t b_base = (size_t)b * p.num_q_heads + h;
  // Pieces (prefix ones first, then suffix ones) are read R at a time, every
  // load of a batch issued before any is used: a batch costs one memory
  // round trip. The running max rescales what is summed so far.
  constexpr int R = 8;
  const int np = a_np + b_np;
  float mx = -INFINITY, W = 0.0f, O = 0.0f;
  for (int i0 = 0; i0 < np; i0 += R) {
    float mm[R], ll[R], tt[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int i = i0 + u;
      const bool in_a = i < a_np;
      const size_t col = in_a ? a_base + i : b_base + (i - a_np);
      const bool ok = i < np;
      mm[u] = ok ? (in_a ? p.a_max : p.b_max)[col] : -INFINITY;
      ll[u] = ok ? (in_a ? p.a_sum : p.b_sum)[col] : 0.0f;
      tt[u] = ok ? (in_a ? p.a_out : p.b_out)[col * D + d] : 0.0f;
    }
    float bm = mx;
#pragma unroll
    for (int u = 0; u < R; ++u) bm = fmaxf(bm, mm[u]);
    const float rs = bm == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f((mx - bm) * kLog2eP);
    W *= rs;
    O *= rs;
#pragma unroll
    for (int u = 0; u < R; ++u) {
      if (i0 + u < np) {
        const float w = ll[u] * __builtin_amdgcn_exp2f((mm[u] - bm) * kLog2eP);
        W += w;
        O = fmaf(w, tt[u], O);
      }
    }
    mx = bm;
  }
  store_out<OT, D>(p.out, ((size_t)b * p.num_q_heads + h) * D + d, W > 0.0f ? O / W : 0.0f);
}

}  // namespace

int launch_shared_prefix(const SharedPrefixLaunch &a, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int M = a.group_size;
  const int gqa = a.num_q_heads / a.num_kv_heads;
  PrepParams pp;
  pp.q = static_cast<const uint8_t *>(a.q);
  pp.q_stack = static_cast<uint8_t *>(a.ws.q_stack);
  pp.block_tables = a.block_tables;
  pp.context_lens = a.context_lens;
  pp.members = a.group_members;
  pp.prefix_lens = a.prefix_lens;
  pp.prefix_tables = a.ws.prefix_tables;
  pp.prefix_ctx = a.ws.prefix_ctx;
  pp.suffix_tables = a.ws.suffix_tables;
  pp.suffix_lens = a.ws.suffix_lens;
  pp.seq_slot = a.ws.seq_slot;
  pp.num_seqs = a.num_seqs;
  pp.num_groups = a.num_groups;
  pp.group_size = M;
  pp.num_q_heads = a.num_q_heads;
  pp.gqa = gqa;
  pp.row_bytes = a.head_dim * a.q_elem_bytes;
  pp.mbs = a.max_blocks_per_seq;
  pp.block_size = a.block_size;
  hipLaunchKernelGGL(prep_kernel, dim3(a.num_seqs + a.num_groups), dim3(kPrepThreads), 0, s, pp);
  int e = (int)hipGetLastError();
  if (e) return e;

  // prefix pass: groups as sequences, members' rows as extra query heads
  DecodeLaunch d{};
  d.q = a.ws.q_stack;
  d.k_cache = a.k_cache;
  d.v_cache = a.v_cache;
  d.block_tables = a.ws.prefix_tables;
  d.context_lens = a.ws.prefix_ctx;
  d.num_seqs = a.num_groups;
  d.num_q_heads = a.num_q_heads * M;
  d.num_kv_heads = a.num_kv_heads;
  d.head_dim = a.head_dim;
  d.block_size = a.block_size;
  d.max_blocks_per_seq = a.max_blocks_per_seq;
  d.scale = a.scale;
  d.k_scale = a.k_scale;
  d.v_scale = a.v_scale;
  d.q_dtype = a.q_dtype;
  d.kv_dtype = a.kv_dtype;
  d.mode = kSplitBalanced;
  d.direct = 0;
  d.num_splits = a.prefix_splits;
  d.max_partitions = a.prefix_splits + a.num_groups;
  d.tmp_out = a.ws.a_out;
  d.max_logits = a.ws.a_max;
  d.exp_sums = a.ws.a_sum;
  e = launch_decode(d, stream);
  if (e) return e;

  // suffix pass: every sequence past its prefix, one range each; its partial
  // goes to column 0 of [B, Hq, 1] (a sequence with an empty suffix writes
  // zeros to `out`, which the merge overwrites)
  DecodeLaunch f = d;
  f.out = a.out;
  f.q = a.q;
  f.block_tables = a.ws.suffix_tables;
  f.context_lens = a.ws.suffix_lens;
  f.num_seqs = a.num_seqs;
  f.num_q_heads = a.num_q_heads;
  f.mode = kSplitSingle;
  f.num_splits = 0;
  f.max_partitions = 1;
  f.tmp_out = a.ws.b_out;
  f.max_logits = a.ws.b_max;
  f.exp_sums = a.ws.b_sum;
  e = launch_decode(f, stream);
  if (e) return e;

  MergeParams mp;
  mp.out = a.out;
  mp.a_out = a.ws.a_out;
  mp.a_max = a.ws.a_max;
  mp.a_sum = a.ws.a_sum;
  mp.a_cols = d.max_partitions;
  mp.a_splits = a.prefix_splits;
  mp.prefix_ctx = a.ws.prefix_ctx;
  mp.b_out = a.ws.b_out;
  mp.b_max = a.ws.b_max;
  mp.b_sum = a.ws.b_sum;
  mp.suffix_lens = a.ws.suffix_lens;
  mp.seq_slot = a.ws.seq_slot;
  mp.num_seqs = a.num_seqs;
  mp.num_groups = a.num_groups;
  mp.group_size = M;
  mp.num_q_heads = a.num_q_heads;
  mp.gqa = gqa;
  const int hpw = kMergeThreads / a.head_dim;
  const dim3 grid(a.num_seqs, (a.num_q_heads + hpw - 1) / hpw);
#define PA_MERGE(OT, D)                                                                   \
  if (a.q_dtype == OT && a.head_dim == D) {                                               \
    hipLaunchKernelGGL((merge_kernel<OT, D>), grid, dim3(kMergeThreads), 0, s, mp);       \
    return (int)hipGetLastError();                                                        \
  }
  PA_MERGE(PA_F32, 64)
  PA_MERGE(PA_F32, 128)
  PA_MERGE(PA_F16, 64)
  PA_MERGE(PA_F16, 128)
  PA_MERGE(PA_BF16, 64)
  PA_MERGE(PA_BF16, 128)
#undef PA_MERGE
  return (int)hipErrorInvalidValue;
}

}  // namespace pa
