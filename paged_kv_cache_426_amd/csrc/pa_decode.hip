// Decode dispatch (element-type pair, head size, heads per workgroup, split
// mode) and the merge of split partials, for gfx950. The decode kernels
// themselves are in pa_decode_kernel.h, instantiated one element-type pair per
// translation unit.

#include <limits.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <utility>

#include "pa_decode_kernel.h"

namespace pa {
namespace {

// ---------------------------------------------------------------------------
// merge of split partials
// ---------------------------------------------------------------------------

struct ReduceParams {
  void *out;
  const float *tmp_out;
  const float *max_logits;
  const float *exp_sums;
  const int32_t *context_lens;
  int num_seqs;
  int num_q_heads;
  int max_partitions;
  int mode;              // kSplitFixed or kSplitBalanced
  int partition_blocks;  // fixed
  int num_splits;        // balanced
  int skip_single;       // sequences with one piece were written directly
};

constexpr int kReduceThreads = 256;

// One workgroup per (sequence, run of 256 / D query heads); thread = (head, d).
template <int OT, int D>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(const ReduceParams p) {
  constexpr int HPW = kReduceThreads / D;
  __shared__ int s_red[2][kReduceThreads / kWave];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int h = blockIdx.y * HPW + tid / D;
  const int d = tid % D;
  const int Hq = p.num_q_heads;
  const int n = p.context_lens[b];
  const int nblk = num_blocks_of(n);

  int first = 0, np = 0;
  if (p.mode == kSplitBalanced) {
    // first block of sequence b and the total, by a workgroup-wide sum
    int before = 0, all = 0;
    for (int bb = tid; bb < p.num_seqs; bb += kReduceThreads) {
      const int c = num_blocks_of(p.context_lens[bb]);
      all += c;
      if (bb < b) before += c;
    }
    before = (int)group_sum_i<kWave>(before);
    all = (int)group_sum_i<kWave>(all);
    if ((tid & (kWave - 1)) == 0) {
      s_red[0][tid >> 6] = before;
      s_red[1][tid >> 6] = all;
    }
    __syncthreads();
    int st = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kReduceThreads / kWave; ++w) {
      st += s_red[0][w];
      total += s_red[1][w];
    }
    if (nblk > 0) {
      const long long S = min(p.num_splits, total);
      // share of block x: the largest s with floor(s * total / S) <= x
      const int s0 = (int)(((long long)(st + 1) * S - 1) / total);
      const int s1 = (int)(((long long)(st + nblk) * S - 1) / total);
      first = s0 + b;
      np = s1 - s0 + 1;
    }
  } else {
    np = (nblk + p.partition_blocks - 1) / p.partition_blocks;
  }
  if (h >= Hq) return;
  const size_t bh = (size_t)b * Hq + h;
  if (np == 0) {
    store_elem<OT>(p.out, bh * D + d, 0.0f);
    return;
  }
  if (np == 1 && p.skip_single) return;
  const size_t base = (p.mode == kSplitBalanced) ? (size_t)h * p.max_partitions + first
                                                 : bh * p.max_partitions;
  // Pieces are merged in one pass, R at a time: every load of a batch is
  // issued before any is used (a batch costs one memory round trip), and the
  // running maximum rescales what is summed so far. Weights
  // w_p = l_p exp(m_p - M) are summed in piece order.
  constexpr int R = 16;
  float M = -INFINITY, W = 0.0f, O = 0.0f;
  for (int i0 = 0; i0 < np; i0 += R) {
    float mm[R], ll[R], tt[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const bool ok = i0 + u < np;
      mm[u] = ok ? p.max_logits[base + i0 + u] : -INFINITY;
      ll[u] = ok ? p.exp_sums[base + i0 + u] : 0.0f;
      tt[u] = ok ? p.tmp_out[(base + i0 + u) * D + d] : 0.0f;
    }
    float bm = M;
#pragma unroll
    for (int u = 0; u < R; ++u) bm = fmaxf(bm, mm[u]);
    const float rs = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((M - bm) * kLog2e);
    W *= rs;
    O *= rs;
#pragma unroll
    for (int u = 0; u < R; ++u)
      if (i0 + u < np) {
        const float w = ll[u] * __builtin_amdgcn_exp2f((mm[u] - bm) * kLog2e);
        W += w;
        O = fmaf(w, tt[u], O);
      }
    M = bm;
  }
  store_elem<OT>(p.out, bh * D + d, O / W);
}

// Merge of a fixed split: one workgroup per (query head, sequence), its four
// waves taking the sequence's partitions in turn (partition i to wave i % 4),
// so that a wave issues the loads of up to kFixedMergeBatch partitions at
// once and long contexts cost one memory round trip per batch rather than
// per partition; each lane holds D / 64 elements of the output row. The
// waves' (max, weight, sum) triples are then merged in LDS in wave order.
constexpr int kFixedMergeWaves = 4;
constexpr int kFixedMergeBatch = 16;

template <int OT, int D>
__global__ __launch_bounds__(kFixedMergeWaves * kWave) void reduce_fixed_kernel(
    const ReduceParams p) {
  constexpr int EPL = D / kWave;  // output elements per lane
  constexpr int NWV = kFixedMergeWaves;
  constexpr int R = kFixedMergeBatch;
  __shared__ float s_m[NWV], s_w[NWV];
  __shared__ float s_o[NWV][D];
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int n = p.context_lens[b];
  const int np = (num_blocks_of(n) + p.partition_blocks - 1) / p.partition_blocks;
  const size_t bh = (size_t)b * p.num_q_heads + h;
  if (np == 0) {
    for (int i = threadIdx.x; i < D; i += NWV * kWave) store_elem<OT>(p.out, bh * D + i, 0.0f);
    return;
  }
  if (np == 1 && p.skip_single) return;
  const size_t base = bh * p.max_partitions;
  float M = -INFINITY, W = 0.0f, O[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) O[e] = 0.0f;
  for (int i0 = wave; i0 < np; i0 += NWV * R) {
    float mm[R], ll[R], tt[R][EPL];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int i = i0 + u * NWV;
      const bool ok = i < np;
      // loads of partition 0 (always present) in place of a missing one,
      // then a select: no branch around each load
      const size_t col = base + (ok ? i : 0);
      const float mv = p.max_logits[col], lv = p.exp_sums[col];
      mm[u] = ok ? mv : -INFINITY;
      ll[u] = ok ? lv : 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float tv = p.tmp_out[col * D + lane * EPL + e];
        tt[u][e] = ok ? tv : 0.0f;
      }
    }
    float bm = M;
#pragma unroll
    for (int u = 0; u < R; ++u) bm = fmaxf(bm, mm[u]);
    const float rs = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((M - bm) * kLog2e);
    W *= rs;
#pragma unroll
    for (int e = 0; e < EPL; ++e) O[e] *= rs;
#pragma unroll
    for (int u = 0; u < R; ++u)
      if (i0 + u * NWV < np) {
        const float w = ll[u] * __builtin_amdgcn_exp2f((mm[u] - bm) * kLog2e);
        W += w;
#pragma unroll
        for (int e = 0; e < EPL; ++e) O[e] = fmaf(w, tt[u][e], O[e]);
      }
    M = bm;
  }
  if (lane == 0) {
    s_m[wave] = M;
    s_w[wave] = W;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) s_o[wave][lane * EPL + e] = O[e];
  __syncthreads();
  if (wave != 0) return;
  float Mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < NWV; ++w) Mx = fmaxf(Mx, s_m[w]);
  float Wt = 0.0f, Ot[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) Ot[e] = 0.0f;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    // a wave that took no partition has M = -inf and weight 0
    const float sc = s_m[w] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((s_m[w] - Mx) * kLog2e);
    Wt += s_w[w] * sc;
#pragma unroll
    for (int e = 0; e < EPL; ++e) Ot[e] = fmaf(s_o[w][lane * EPL + e], sc, Ot[e]);
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) store_elem<OT>(p.out, bh * D + lane * EPL + e, Ot[e] / Wt);
}

KernelRef decode_kernel_for(int q_dtype, int kv_dtype, int d, int gh, int kind, bool append,
                            bool large, bool scaled) {
#define PA_PAIR(Q, KV, NAME)                                                                   \
  if (q_dtype == Q && kv_dtype == KV)                                                          \
    return large ? decode_kernels_##NAME##_large(d, gh, kind, append, scaled)                  \
                 : decode_kernels_##NAME(d, gh, kind, append, scaled);
  PA_PAIR(PA_F32, PA_F32, f32_f32)
  PA_PAIR(PA_F16, PA_F16, f16_f16)
  PA_PAIR(PA_BF16, PA_BF16, bf16_bf16)
  PA_PAIR(PA_F16, PA_FP8_E4M3FN, f16_fp8)
  PA_PAIR(PA_BF16, PA_FP8_E4M3FN, bf16_fp8)
  PA_PAIR(PA_F16, PA_INT8, f16_int8)
  PA_PAIR(PA_BF16, PA_INT8, bf16_int8)
#undef PA_PAIR
  return {nullptr, 0};
}

}  // namespace


// Workgroups of one decode kernel that fill a device once: compute units x
// resident workgroups per unit (one for four-wave kernels, see below). Looked
// up once per (device, kernel) and kept for the life of the process (a
// device property, not state of a call).
int fill_workgroups(const void *fn, int threads) {
  static std::mutex mu;
  static std::map<std::pair<int, const void *>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, fn);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  // Four-wave kernels (16 heads per workgroup, most fp32) fit two per unit,
  // but one per unit with twice the shares each measured faster (the
  // hardware serves co-resident workgroups unevenly; shared-prefix call 53.7
  // -> 51.3 us, while a third of the shares or fewer leaves units idle).
  const int n = cus * (per_cu <= 0 ? 1 : threads <= 4 * kWave ? 1 : per_cu);
  cache[key] = n;
  return n;
}

// The balanced-split kernel of a launch: one wave per head row where the
// head rows fill whole eight-wave workgroups and that kernel is built,
// otherwise shares dealt to all waves of a workgroup.
struct BalancedChoice {
  KernelRef k;
  bool row_waves;
  int rowgroups;  // grid.y: workgroups per share
};

BalancedChoice balanced_kernel(const DecodeLaunch &a, bool append, bool large) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const int gh = heads_per_workgroup(group);
  const long long rows = (long long)a.num_kv_heads * (group / gh);
  const bool scaled = a.k_scales != nullptr;
  if (rows % 8 == 0) {
    const KernelRef k = decode_kernel_for(a.q_dtype, a.kv_dtype, a.head_dim, gh, kKindRowWaves,
                                          append, large, scaled);
    if (k.fn) return {k, true, (int)(rows / 8)};
  }
  return {decode_kernel_for(a.q_dtype, a.kv_dtype, a.head_dim, gh, kKindShares, append, large,
                            scaled),
          false, (int)rows};
}

// The single-pass / fixed-split kernel of a launch. A fixed split runs one
// wave per head row (each workgroup reads whole cache blocks: all of their
// KV heads) where the head rows fill eight-wave workgroups and that kernel
// is built; a single pass, with one workgroup per sequence and head-row
// group, would leave the device mostly idle that way, and runs four-wave
// workgroups per head row (kKindSingle).
struct FixedChoice {
  KernelRef k;
  bool row_waves;
};

FixedChoice fixed_kernel(const DecodeLaunch &a, bool append, bool large, bool scaled) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const int gh = heads_per_workgroup(group);
  const long long rows = (long long)a.num_kv_heads * (group / gh);
  if (a.mode == kSplitFixed && rows % 8 == 0) {
    const KernelRef k = decode_kernel_for(a.q_dtype, a.kv_dtype, a.head_dim, gh, kKindRowWaves,
                                          append, large, scaled);
    if (k.fn) return {k, true};
  }
  const int kind = a.mode == kSplitSingle ? kKindSingle : kKindRanges;
  return {decode_kernel_for(a.q_dtype, a.kv_dtype, a.head_dim, gh, kind, append, large,
                            scaled),
          false};
}

int balanced_num_splits(const DecodeLaunch &a) {
  const BalancedChoice c = balanced_kernel(a, false, false);
  if (!c.k.fn) return 2;
  const int cus = fill_workgroups(c.k.fn, c.k.threads);
  if (cus <= 0) return kMaxAutoSplits / 8;
  // row waves: one share per workgroup; otherwise two shares per workgroup;
  // as many workgroups as fit at once
  const long long per = ((long long)cus + c.rowgroups - 1) / c.rowgroups;
  long long s = c.row_waves ? per : 2 * per;
  if (s < 2) s = 2;
  if (s > kMaxAutoSplits) s = kMaxAutoSplits;
  return (int)s;
}

int launch_decode(const DecodeLaunch &a, void *stream) {
  DecodeParams p;
  p.out = a.out;
  p.tmp_out = a.tmp_out;
  p.max_logits = a.max_logits;
  p.exp_sums = a.exp_sums;
  p.q = static_cast<const uint8_t *>(a.q);
  p.k_cache = static_cast<const uint8_t *>(a.k_cache);
  p.v_cache = static_cast<const uint8_t *>(a.v_cache);
  p.block_tables = a.block_tables;
  p.context_lens = a.context_lens;
  p.num_seqs = a.num_seqs;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.max_blocks_per_seq = a.max_blocks_per_seq;
  // the kernels count 16-token units: sub-blocks of a block of 16 << sub_log2
  // tokens, or pairs of 8-token blocks (kHalfBlocks; the SUB kernels)
  const bool halves = a.block_size == kHalfBlockSize;
  p.sub_log2 = halves ? kHalfBlocks : sub_block_log2(a.block_size);
  if (!halves && p.sub_log2 < 0) return (int)hipErrorInvalidValue;
  if (halves && (a.new_k != nullptr || a.k_scales != nullptr ||
                 (a.mode == kSplitFixed && a.partition_size % kBs != 0)))
    return (int)hipErrorInvalidValue;
  p.mode = a.mode;
  p.partition_blocks = a.mode != kSplitSingle ? a.partition_size / kBs
                       : halves              ? (a.max_blocks_per_seq + 1) / 2
                                             : a.max_blocks_per_seq << p.sub_log2;
  p.max_partitions = a.max_partitions;
  p.num_splits = a.num_splits;
  const bool wide = p.mode == kSplitBalanced;
  p.direct = a.direct;
  p.swz_rows = 0;
  p.group = a.num_q_heads / a.num_kv_heads;
  const bool q8 = a.kv_dtype == PA_FP8_E4M3FN || a.kv_dtype == PA_INT8;
  // scale tables: each block's scales are applied per block in the kernel
  const bool scaled = a.k_scales != nullptr;
  const bool tensor_scales = q8 && !scaled;
  const float ks = tensor_scales ? a.k_scale : 1.0f;
  p.scale_log2 = a.scale * ks * kLog2e;
  p.v_scale = tensor_scales ? a.v_scale : 1.0f;
  p.k_scales = a.k_scales;
  p.v_scales = a.v_scales;
  p.scale_sb = a.scale_block_stride;
  p.scale_sh = a.scale_head_stride;
  p.new_k = static_cast<const uint8_t *>(a.new_k);
  p.new_v = static_cast<const uint8_t *>(a.new_v);
  p.k_cache_w = const_cast<uint8_t *>(p.k_cache);
  p.v_cache_w = const_cast<uint8_t *>(p.v_cache);
  p.k_scale = a.k_scale;
  p.v_scale_w = a.v_scale;
  const int gh = heads_per_workgroup(p.group);
  const bool append = a.new_k != nullptr;
  const bool large = p.sub_log2 != 0;
  const int head_groups = a.num_kv_heads * (p.group / gh);
  KernelRef k;
  dim3 grid;
  if (wide) {
    const BalancedChoice c = balanced_kernel(a, append, large);
    k = c.k;
    grid = c.row_waves ? dim3(p.num_splits, c.rowgroups, 1)
                       : dim3((p.num_splits + 1) / 2, head_groups, 1);
  } else {
    const FixedChoice c = fixed_kernel(a, append, large, scaled);
    k = c.k;
    const int y = c.row_waves ? head_groups / 8 : head_groups;
    grid = a.mode == kSplitFixed ? dim3(a.max_partitions, y, a.num_seqs) : dim3(1, y, a.num_seqs);
    // a fixed split runs on a one-dimensional grid that spreads every
    // sequence's partitions over the XCDs (see decode_kernel)
    if (a.mode == kSplitFixed && k.fn) {
      const long long xp = (a.max_partitions + 7LL) / 8 * 8;
      const long long n = xp * a.num_seqs * y;
      // (the dispatch packet counts work-items in 32 bits)
      if (n * k.threads <= (long long)UINT32_MAX) {
        p.swz_rows = y;
        grid = dim3((unsigned)n, 1, 1);
      }
    }
  }
  if (!k.fn) return (int)hipErrorInvalidValue;
  void *args[] = {&p};
  hipError_t e = hipLaunchKernel(k.fn, grid, dim3(k.threads), args, 0,
                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return (int)e;
  return (int)hipGetLastError();
}

int launch_reduce(const ReduceLaunch &a, void *stream) {
  ReduceParams p;
  p.out = a.out;
  p.tmp_out = a.tmp_out;
  p.max_logits = a.max_logits;
  p.exp_sums = a.exp_sums;
  p.context_lens = a.context_lens;
  p.num_seqs = a.num_seqs;
  p.num_q_heads = a.num_q_heads;
  p.max_partitions = a.max_partitions;
  p.mode = a.mode;
  p.partition_blocks = a.mode == kSplitFixed ? a.partition_size / kBs : 0;
  p.num_splits = a.num_splits;
  p.skip_single = a.skip_single;
  const int hpw = kReduceThreads / a.head_dim;
  const dim3 grid(a.num_seqs, (a.num_q_heads + hpw - 1) / hpw);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.mode == kSplitFixed) {
    const dim3 fgrid(a.num_q_heads, a.num_seqs);
#define PA_REDF(OT, D)                                                                         \
  if (a.out_dtype == OT && a.head_dim == D) {                                                  \
    hipLaunchKernelGGL((reduce_fixed_kernel<OT, D>), fgrid, dim3(kFixedMergeWaves * kWave), 0, \
                       s, p);                                                                  \
    return (int)hipGetLastError();                                                             \
  }
    PA_REDF(PA_F32, 64)
    PA_REDF(PA_F32, 128)
    PA_REDF(PA_F16, 64)
    PA_REDF(PA_F16, 128)
    PA_REDF(PA_BF16, 64)
    PA_REDF(PA_BF16, 128)
#undef PA_REDF
    return (int)hipErrorInvalidValue;
  }
#define PA_RED(OT, D)                                                                          \
  if (a.out_dtype == OT && a.head_dim == D) {                                                  \
    hipLaunchKernelGGL((reduce_kernel<OT, D>), grid, dim3(kReduceThreads), 0, s, p);          \
    return (int)hipGetLastError();                                                             \
  }
  PA_RED(PA_F32, 64)
  PA_RED(PA_F32, 128)
  PA_RED(PA_F16, 64)
  PA_RED(PA_F16, 128)
  PA_RED(PA_BF16, 64)
  PA_RED(PA_BF16, 128)
#undef PA_RED
  return (int)hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// fixed device scratch of pa_decode_noalloc
// ---------------------------------------------------------------------------

// The split partials of pa_decode_noalloc live here instead of in a caller's
// workspace. Each device the library runs on holds its own copy for the life
// of the process. In host code `scratch` is only a stand-in for the device
// variable: its device address comes from hipGetSymbolAddress, once per
// device, and only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

int noalloc_scratch(void **ptr) {
  static std::mutex mu;
  static std::map<int, void *> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return (int)e;
  }
  std::lock_guard<std::mutex> lock(mu);
  const auto it = addr.find(dev);
  if (it != addr.end()) {
    *ptr = it->second;
    return 0;
  }
  void *p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || p == nullptr) {
    (void)hipGetLastError();
    return e != hipSuccess ? (int)e : (int)hipErrorInvalidSymbol;
  }
  addr[dev] = p;
  *ptr = p;
  return 0;
}

}  // namespace pa
