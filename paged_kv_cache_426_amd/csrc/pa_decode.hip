// Paged-attention decode for gfx950 (CDNA4, wave64).
//
// What is computed: for each sequence b and query head h, one query row
// attends over the sequence's n cached tokens, softmax(q K^T * scale) V
// ("KV-Cache evolution" §1, attention formula), where token j's K/V row sits
// in physical block block_tables[b][j / 16] at offset j % 16 ("PagedAttention
// deep dive" §2.1; "vLLM inference principles", block-table figure), and
// query head h reads KV head h / group ("KV-Cache evolution" §3A, GQA).
//
// Work decomposition. One workgroup (4 waves) serves one (sequence, KV head,
// run of GH query heads of that KV head's group, token range). The token
// range is the whole context (single pass) or one partition of P tokens
// (split context, followed by reduce_kernel). Because the GH query heads of a
// group share one KV head, each K/V byte of the range is read from HBM once
// and used GH times; the GH query rows live in registers of every lane.
//
// The range is walked in chunks; each wave owns `bpw` whole blocks of a chunk.
// Lanes are laid out so that one 16-byte load per lane covers `tpi` token
// rows: lane = r * lpt + c reads bytes [16c, 16c+16) of token row r, so each
// row is read by lpt adjacent lanes in one coalesced access. Per chunk:
//   A. every wave issues all its K and V loads (gathered through the block
//      table, the physical id being a wave-uniform scalar load), then forms
//      the partial dot products of its K rows with the GH query rows and sums
//      them across the lpt lanes of a row with DPP (no LDS); logits (log2
//      domain) go to LDS;
//   B. one wave per head turns the chunk's logits into exp2(s - m_new) in
//      place, with the running max m and sum l kept in LDS (online softmax
//      across chunks, rescale factor alpha = exp2(m_old - m_new));
//   C. every wave rescales its fp32 accumulators by alpha and adds p * V for
//      its rows.
// At the end the accumulators are summed across rows (shuffles) and waves
// (LDS) and either normalised into `out` or written as split partials.
//
// Masking: tokens at or beyond the range end get a logit of -inf (a select,
// never a product, so stale or NaN cache contents cannot leak in), and their
// V words are zeroed before use. Block-table entries past the range end are
// never read; loads of such blocks are redirected to the range's first block.
//
// The arithmetic order depends only on logical token positions, never on
// physical block ids: results are bitwise invariant under any relabelling of
// physical blocks and identical for aliased and private copies of a block.

#include <hip/hip_runtime.h>
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kBlockSize = 16;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct DecodeParams {
  void *out;
  float *tmp_out;
  float *max_logits;
  float *exp_sums;
  const uint8_t *q;
  const uint8_t *k_cache;
  const uint8_t *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  int num_q_heads;
  int num_kv_heads;
  int max_blocks_per_seq;
  int max_partitions;
  int partition_size;  // 0: whole context
  int group;           // query heads per KV head
  float scale_log2;    // scale * k_scale * log2(e)
  float v_scale;
};

// Lane geometry for a cache element type and head size.
template <int KT, int D>
struct Geo {
  static constexpr int kb = ElemBytes<KT>::value;
  static constexpr int epl = 16 / kb;                    // cache elements per 16-byte load
  static constexpr int lpt = D / epl;                    // lanes per token row
  static constexpr int tpi = kWave / lpt;                // token rows per wave load
  static constexpr int nlb = kBlockSize / tpi;           // loads per lane per block
  static constexpr int bpw = nlb >= 8 ? 1 : 8 / nlb;     // blocks per wave per chunk
  static constexpr int chunk = kWaves * bpw * kBlockSize;
  static_assert(lpt >= 1 && lpt <= kWave && tpi <= kBlockSize, "unsupported geometry");
};

template <int QT>
__device__ __forceinline__ void store_elem(void *out, size_t idx, float v) {
  if constexpr (QT == PA_F32) {
    static_cast<float *>(out)[idx] = v;
  } else if constexpr (QT == PA_BF16) {
    static_cast<uint16_t *>(out)[idx] = f32_to_bf16_rne(v);
  } else {
    static_cast<uint16_t *>(out)[idx] = f32_to_f16_rne(v);
  }
}

// 16 cache bytes -> fp32 elements.
template <int KT>
__device__ __forceinline__ void widen(const u32x4 w, float *v) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (KT == PA_F32) {
      v[i] = u2f(ws[i]);
    } else if constexpr (KT == PA_BF16) {
      v[2 * i] = bf16_lo(ws[i]);
      v[2 * i + 1] = bf16_hi(ws[i]);
    } else if constexpr (KT == PA_F16) {
      v[2 * i] = f16_lo(ws[i]);
      v[2 * i + 1] = f16_hi(ws[i]);
    } else {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(ws[i], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(ws[i], true);
      v[4 * i] = lo.x;
      v[4 * i + 1] = lo.y;
      v[4 * i + 2] = hi.x;
      v[4 * i + 3] = hi.y;
    }
  }
}

// The query fragment of one lane for one head, in the form the dot product
// consumes: packed 16-bit pairs for 16-bit and fp8 caches (fp8 K is widened
// exactly to the query's 16-bit type), fp32 for fp32 caches.
template <int QT, int KT>
struct QFrag {
  static constexpr int words = (KT == PA_FP8_E4M3FN) ? 8 : 4;
  uint32_t w[words];
};

template <int QT, int KT, int D>
__device__ __forceinline__ void load_q(QFrag<QT, KT> &f, const uint8_t *qrow, int c) {
  // qrow points at element 0 of one query head
  if constexpr (KT == PA_FP8_E4M3FN) {
    const u32x4 a = *reinterpret_cast<const u32x4 *>(qrow + c * 32);
    const u32x4 b = *reinterpret_cast<const u32x4 *>(qrow + c * 32 + 16);
    f.w[0] = a.x; f.w[1] = a.y; f.w[2] = a.z; f.w[3] = a.w;
    f.w[4] = b.x; f.w[5] = b.y; f.w[6] = b.z; f.w[7] = b.w;
  } else {
    const u32x4 a = *reinterpret_cast<const u32x4 *>(qrow + c * 16);
    f.w[0] = a.x; f.w[1] = a.y; f.w[2] = a.z; f.w[3] = a.w;
  }
}

// fp8 pair (byte half `hi` of a word) widened exactly to a 16-bit pair
template <int QT, bool HI>
__device__ __forceinline__ uint32_t fp8_pair_to_16(uint32_t w) {
  if constexpr (QT == PA_BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  }
}

template <int QT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  if constexpr (QT == PA_BF16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), acc, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b),
                                  acc, false);
  }
}

// Partial dot products of one 16-byte K piece with the GH query fragments.
template <int QT, int KT, int GH>
__device__ __forceinline__ void partial_dots(const u32x4 k, const QFrag<QT, KT> (&qf)[GH],
                                             float (&out)[GH]) {
  const uint32_t ks[4] = {k.x, k.y, k.z, k.w};
  if constexpr (KT == PA_F32) {
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      float s = u2f(qf[h].w[0]) * u2f(ks[0]);
      s = fmaf(u2f(qf[h].w[1]), u2f(ks[1]), s);
      s = fmaf(u2f(qf[h].w[2]), u2f(ks[2]), s);
      s = fmaf(u2f(qf[h].w[3]), u2f(ks[3]), s);
      out[h] = s;
    }
  } else if constexpr (KT == PA_FP8_E4M3FN) {
    uint32_t k16[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      k16[2 * i] = fp8_pair_to_16<QT, false>(ks[i]);
      k16[2 * i + 1] = fp8_pair_to_16<QT, true>(ks[i]);
    }
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) s = dot2<QT>(k16[i], qf[h].w[i], s);
      out[h] = s;
    }
  } else {
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) s = dot2<QT>(ks[i], qf[h].w[i], s);
      out[h] = s;
    }
  }
}

template <int QT, int KT, int D, int GH>
__global__ __launch_bounds__(kThreads) void decode_kernel(const DecodeParams p) {
  using G = Geo<KT, D>;
  constexpr int EPL = G::epl, LPT = G::lpt, TPI = G::tpi, NLB = G::nlb, BPW = G::bpw;
  constexpr int CH = G::chunk;
  constexpr int QB = ElemBytes<QT>::value;

  __shared__ float s_p[2][CH * GH];  // logits, then probabilities; double-buffered per chunk
  __shared__ float s_m[GH], s_l[GH], s_alpha[GH];
  __shared__ float s_o[kWaves][GH][D];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane / LPT;
  const int c = lane % LPT;

  const int b = blockIdx.z;
  const int hg = blockIdx.y;
  const int part = blockIdx.x;
  const int Hq = p.num_q_heads;
  const int g = hg / (p.group / GH);
  const int h0 = hg * GH;
  const int n = p.context_lens[b];

  int start = 0, end = n;
  if (p.partition_size > 0) {
    start = part * p.partition_size;
    if (start >= n) return;
    end = min(n, start + p.partition_size);
  } else if (n <= 0) {
    for (int i = tid; i < GH * D; i += kThreads)
      store_elem<QT>(p.out, ((size_t)b * Hq + h0) * D + i, 0.0f);
    return;
  }

  if (tid < GH) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.0f;
  }

  QFrag<QT, KT> qf[GH];
  {
    const uint8_t *qb = p.q + ((size_t)b * Hq + h0) * D * QB;
#pragma unroll
    for (int h = 0; h < GH; ++h) load_q<QT, KT, D>(qf[h], qb + (size_t)h * D * QB, c);
  }

  float acc[GH][EPL];
#pragma unroll
  for (int h = 0; h < GH; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;

  const uint32_t row_bytes = (uint32_t)p.num_kv_heads * D * G::kb;
  const size_t blk_bytes = (size_t)row_bytes * kBlockSize;
  const uint32_t lane_off = r * row_bytes + c * 16;
  const uint8_t *kg = p.k_cache + (size_t)g * D * G::kb;
  const uint8_t *vg = p.v_cache + (size_t)g * D * G::kb;
  const int32_t *bt = p.block_tables + (size_t)b * p.max_blocks_per_seq;
  const int first_blk = start / kBlockSize;
  const float sl2 = p.scale_log2;

  __syncthreads();

  int buf = 0;
  for (int cs = start; cs < end; cs += CH, buf ^= 1) {
    const int wb0 = cs / kBlockSize + wave * BPW;
    float *sp = s_p[buf];

    u32x4 kr[BPW][NLB], vr[BPW][NLB];
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      const int j = wb0 + bi;
      const int phys = bt[(j * kBlockSize < end) ? j : first_blk];
      const uint8_t *kb = kg + (size_t)phys * blk_bytes;
      const uint8_t *vb = vg + (size_t)phys * blk_bytes;
#pragma unroll
      for (int i = 0; i < NLB; ++i)
        kr[bi][i] = *reinterpret_cast<const u32x4 *>(kb + (size_t)i * TPI * row_bytes + lane_off);
#pragma unroll
      for (int i = 0; i < NLB; ++i)
        vr[bi][i] = *reinterpret_cast<const u32x4 *>(vb + (size_t)i * TPI * row_bytes + lane_off);
    }

    // A: logits of this wave's rows
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      const int j = wb0 + bi;
#pragma unroll
      for (int i = 0; i < NLB; ++i) {
        const int tl = (wave * BPW + bi) * kBlockSize + i * TPI + r;
        const bool valid = j * kBlockSize + i * TPI + r < end;
        float d[GH];
        partial_dots<QT, KT, GH>(kr[bi][i], qf, d);
#pragma unroll
        for (int h = 0; h < GH; ++h) d[h] = group_sum<LPT>(d[h]);
#pragma unroll
        for (int hh = 0; hh < GH; hh += LPT) {
          float v = d[hh];
#pragma unroll
          for (int x = 1; x < LPT && hh + x < GH; ++x) v = (c == x) ? d[hh + x] : v;
          if (hh + c < GH) sp[tl * GH + hh + c] = valid ? v * sl2 : -INFINITY;
        }
      }
    }
    __syncthreads();

    // B: chunk softmax statistics, one wave per head
    for (int h = wave; h < GH; h += kWaves) {
      constexpr int PER = CH / kWave;
      float s[PER];
      float mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        s[k] = sp[(lane + k * kWave) * GH + h];
        mx = fmaxf(mx, s[k]);
      }
      mx = group_max<kWave>(mx);
      const float m_old = s_m[h];
      const float m_new = fmaxf(m_old, mx);
      float sum = 0.0f;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const float e = __builtin_amdgcn_exp2f(s[k] - m_new);
        sp[(lane + k * kWave) * GH + h] = e;
        sum += e;
      }
      sum = group_sum<kWave>(sum);
      if (lane == 0) {
        const float alpha = __builtin_amdgcn_exp2f(m_old - m_new);
        s_alpha[h] = alpha;
        s_l[h] = s_l[h] * alpha + sum;
        s_m[h] = m_new;
      }
    }
    __syncthreads();

    // C: rescale and accumulate p * V
    {
      float al[GH];
#pragma unroll
      for (int h = 0; h < GH; ++h) al[h] = s_alpha[h];
#pragma unroll
      for (int h = 0; h < GH; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= al[h];
    }
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      const int j = wb0 + bi;
      const bool full = (j + 1) * kBlockSize <= end;
#pragma unroll
      for (int i = 0; i < NLB; ++i) {
        const int tl = (wave * BPW + bi) * kBlockSize + i * TPI + r;
        u32x4 w = vr[bi][i];
        if (!full) {
          const bool valid = j * kBlockSize + i * TPI + r < end;
          w.x = valid ? w.x : 0u;
          w.y = valid ? w.y : 0u;
          w.z = valid ? w.z : 0u;
          w.w = valid ? w.w : 0u;
        }
        float v[EPL];
        widen<KT>(w, v);
        float pw[GH];
#pragma unroll
        for (int h = 0; h < GH; ++h) pw[h] = sp[tl * GH + h];
#pragma unroll
        for (int h = 0; h < GH; ++h)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pw[h], v[e], acc[h][e]);
      }
    }
  }

  // sum the accumulators over the rows of a wave, then over the waves
#pragma unroll
  for (int h = 0; h < GH; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e)
#pragma unroll
      for (int off = LPT; off < kWave; off <<= 1) acc[h][e] += __shfl_xor(acc[h][e], off);
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < GH; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[wave][h][c * EPL + e] = acc[h][e];
  }
  __syncthreads();

  for (int i = tid; i < GH * D; i += kThreads) {
    const int h = i / D, d = i % D;
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) o += s_o[w][h][d];
    const float l = s_l[h];
    const float res = o * p.v_scale / l;
    const size_t bh = (size_t)b * Hq + h0 + h;
    if (p.partition_size > 0) {
      const size_t pi = bh * p.max_partitions + part;
      p.tmp_out[pi * D + d] = res;
      if (d == 0) {
        p.max_logits[pi] = s_m[h] * kLn2;
        p.exp_sums[pi] = l;
      }
    } else {
      store_elem<QT>(p.out, bh * D + d, res);
    }
  }
}

template <int OT>
__global__ __launch_bounds__(128) void reduce_kernel(void *out, const float *tmp_out,
                                                     const float *max_logits,
                                                     const float *exp_sums,
                                                     const int32_t *context_lens, int Hq,
                                                     int D, int max_partitions, int P) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int n = max(context_lens[b], 0);
  const int np = (n + P - 1) / P;
  const size_t base = ((size_t)b * Hq + h) * max_partitions;
  float M = -INFINITY;
  for (int i = 0; i < np; ++i) M = fmaxf(M, max_logits[base + i]);
  float W = 0.0f;
  for (int i = 0; i < np; ++i)
    W += exp_sums[base + i] * __builtin_amdgcn_exp2f((max_logits[base + i] - M) * kLog2e);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float o = 0.0f;
    for (int i = 0; i < np; ++i) {
      const float w =
          exp_sums[base + i] * __builtin_amdgcn_exp2f((max_logits[base + i] - M) * kLog2e);
      o = fmaf(w, tmp_out[(base + i) * D + d], o);
    }
    store_elem<OT>(out, ((size_t)b * Hq + h) * D + d, np > 0 ? o / W : 0.0f);
  }
}

template <int QT, int KT, int D, int GH>
hipError_t launch_one(const DecodeParams &p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<QT, KT, D, GH>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int QT, int KT, int D>
hipError_t by_gh(int gh, const DecodeParams &p, dim3 grid, hipStream_t s) {
  switch (gh) {
    case 1: return launch_one<QT, KT, D, 1>(p, grid, s);
    case 2: return launch_one<QT, KT, D, 2>(p, grid, s);
    case 4: return launch_one<QT, KT, D, 4>(p, grid, s);
    case 8: return launch_one<QT, KT, D, 8>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

template <int QT, int KT>
hipError_t by_d(int d, int gh, const DecodeParams &p, dim3 grid, hipStream_t s) {
  switch (d) {
    case 64: return by_gh<QT, KT, 64>(gh, p, grid, s);
    case 128: return by_gh<QT, KT, 128>(gh, p, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

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
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.max_blocks_per_seq = a.max_blocks_per_seq;
  p.max_partitions = a.max_partitions;
  p.partition_size = a.partition_size;
  p.group = a.num_q_heads / a.num_kv_heads;
  const float ks = a.kv_dtype == PA_FP8_E4M3FN ? a.k_scale : 1.0f;
  p.scale_log2 = a.scale * ks * kLog2e;
  p.v_scale = a.kv_dtype == PA_FP8_E4M3FN ? a.v_scale : 1.0f;
  const int gh = heads_per_workgroup(p.group);
  const int parts = a.partition_size > 0 ? a.max_partitions : 1;
  const dim3 grid(parts, a.num_kv_heads * (p.group / gh), a.num_seqs);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipErrorInvalidValue;
  if (a.q_dtype == PA_F32 && a.kv_dtype == PA_F32) e = by_d<PA_F32, PA_F32>(a.head_dim, gh, p, grid, s);
  else if (a.q_dtype == PA_F16 && a.kv_dtype == PA_F16) e = by_d<PA_F16, PA_F16>(a.head_dim, gh, p, grid, s);
  else if (a.q_dtype == PA_BF16 && a.kv_dtype == PA_BF16) e = by_d<PA_BF16, PA_BF16>(a.head_dim, gh, p, grid, s);
  else if (a.q_dtype == PA_F16 && a.kv_dtype == PA_FP8_E4M3FN) e = by_d<PA_F16, PA_FP8_E4M3FN>(a.head_dim, gh, p, grid, s);
  else if (a.q_dtype == PA_BF16 && a.kv_dtype == PA_FP8_E4M3FN) e = by_d<PA_BF16, PA_FP8_E4M3FN>(a.head_dim, gh, p, grid, s);
  return (int)e;
}

int launch_reduce(void *out, const float *tmp_out, const float *max_logits, const float *exp_sums,
                  const int32_t *context_lens, int num_seqs, int num_q_heads, int head_dim,
                  int max_partitions, int partition_size, int out_dtype, void *stream) {
  const dim3 grid(num_q_heads, num_seqs);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (out_dtype) {
    case PA_F32:
      hipLaunchKernelGGL(reduce_kernel<PA_F32>, grid, dim3(128), 0, s, out, tmp_out, max_logits,
                         exp_sums, context_lens, num_q_heads, head_dim, max_partitions,
                         partition_size);
      break;
    case PA_F16:
      hipLaunchKernelGGL(reduce_kernel<PA_F16>, grid, dim3(128), 0, s, out, tmp_out, max_logits,
                         exp_sums, context_lens, num_q_heads, head_dim, max_partitions,
                         partition_size);
      break;
    case PA_BF16:
      hipLaunchKernelGGL(reduce_kernel<PA_BF16>, grid, dim3(128), 0, s, out, tmp_out, max_logits,
                         exp_sums, context_lens, num_q_heads, head_dim, max_partitions,
                         partition_size);
      break;
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // namespace pa
