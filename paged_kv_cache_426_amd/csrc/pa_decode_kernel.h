// Paged-attention decode kernels for gfx950 (CDNA4, wave64). Included by one
// translation unit per element-type pair (pa_decode_<q>_<kv>.hip), each of
// which instantiates its pair's kernels, so that the pairs build in parallel.
//
// What is computed: for each sequence b and query head h, one query row
// attends over the sequence's n cached tokens, softmax(q K^T * scale) V
// ("KV-Cache evolution" §1, attention formula), where token j's K/V row sits
// in physical block block_tables[b][j / bs] at offset j % bs ("PagedAttention
// deep dive" §2.1; "vLLM inference principles", block-table figure), and
// query head h reads KV head h / group ("KV-Cache evolution" §3A, GQA).
//
// Block size. The kernels work in 16-token sub-blocks. A cache of blocks of
// bs = 16 * 2^k tokens, [NB, bs, Hkv, d], is byte for byte a pool of NB * 2^k
// sub-blocks [NB * 2^k, 16, Hkv, d]: sub-block j of a sequence is sub-block
// (block_tables[b][j >> k] << k) + (j & (2^k - 1)) of that pool. Everything
// below ("block", "blocks per partition", ids) counts sub-blocks.
//
// Work decomposition. A workgroup (2 to 8 waves) serves one KV head and a run of
// GH of its query heads, over a range of that KV head's cache blocks: a whole
// sequence (single pass), one fixed-size partition of a sequence (split
// context), or an equal share of all blocks of all sequences taken end to end
// (balanced split: every workgroup reads the same number of blocks, so the
// grid finishes in one round whatever the length mix). Each K/V byte of the
// range is read from HBM once and used for all GH heads.
//
// Inside a range, the waves take units of NBI blocks round-robin and run
// independently, each with its own online softmax; the next unit's K/V are
// loaded into registers while the current one is computed. Per unit:
//   * logits: one 16x16 MFMA tile per block, rows = query heads (row m holds
//     head m % GH), columns = the block's 16 tokens, reduced over head_dim in
//     D/32 steps (16-bit types; fp8 K is first widened exactly to the query's
//     type) or D/4 steps (fp32). Lane l loads token l%16's row elements
//     [D/4 * (l/16), +D/4) -- 64 contiguous bytes for bf16 d=128 -- and the
//     query fragment of each lane covers the same elements, so the product is
//     the full dot product whatever the MFMA's internal k order;
//   * online softmax: block max over the 16 token lanes with DPP, running max
//     m and per-lane partial sums l, rescale alpha = exp2(m_old - m_new);
//   * P.V: lane (r, c) of a V load holds 8 elements [8c, 8c+8) of token row
//     r. With 16-bit queries, d = 128 and 4 to 16 heads per workgroup it runs
//     on 16x16x16 MFMAs (see PVM below: the probabilities in two 16-bit parts,
//     V exactly, fp32 accumulators); otherwise on the vector ALU, the
//     probabilities reaching the V layout through a small per-wave LDS buffer,
//     fp32 accumulators acc[head][8].
// At the end of a range the waves' (m, l, acc) are merged in LDS, in fixed
// wave order, and written as the output or as one split partial.
//
// Masking: tokens at or beyond the range end get a logit of -inf (a select,
// never a product, so stale or NaN cache contents cannot leak in), and their
// V words are zeroed before use. Block-table entries past the range end are
// never read; loads for such blocks are redirected to the range's first block.
//
// The arithmetic order depends only on logical token positions (and, in the
// balanced split, on the context lengths), never on physical block ids:
// results are bitwise invariant under any relabelling of physical blocks and
// identical for aliased and private copies of a block.

#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kBs = 16;  // tokens per cache block
constexpr int kStages = 2;  // register stages of the load pipeline
// Waves per workgroup (NW below): a fixed partition is split between
// kFixedWaves waves, a whole sequence (single pass) between kSingleWaves; a
// balanced split runs one wide workgroup per compute unit where the
// registers allow (see balanced_waves). A single pass has one workgroup per
// sequence and head row, few for the device, so more waves share each range
// (four against two: 302 against 587 us for 8 long sequences with 2 KV
// heads, 64 against 87 us for the Llama-shaped batch); for fixed partitions
// two waves measured as fast or faster (8-bit caches: 32 against 37 us).
constexpr int kFixedWaves = 2;
constexpr int kSingleWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
// lazy softmax reference maximum: probabilities stay below 2^kLazyMax
constexpr float kLazyMax = 8.0f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int max_blocks_per_seq;  // block-table row stride (physical blocks)
  // log2(block_size / 16), or kHalfBlocks for 8-token blocks (kernels
  // built with SUB only): a 16-token unit is then two physical blocks
  int sub_log2;
  int mode;              // a SplitMode
  int partition_blocks;  // fixed / single: sub-blocks per partition
  int max_partitions;    // stride of the partial arrays (see DecodeLaunch)
  int num_splits;        // balanced: number of shares S
  int direct;            // a range that is a whole sequence writes `out` directly
  // fixed split on a one-dimensional grid (0: grid (partitions, rows,
  // sequences)): the number of head-row groups; see decode_kernel
  int swz_rows;
  int group;             // query heads per KV head
  float scale_log2;      // scale * k_scale * log2(e)
  float v_scale;
  // decode with the new token appended: every sequence's token at position
  // n - 1 comes from new_k / new_v ([B, Hkv, d], q's type; fp8 caches
  // quantised with k_scale / v_scale) and is written to its slot; null
  // otherwise
  const uint8_t *new_k;
  const uint8_t *new_v;
  uint8_t *k_cache_w;
  uint8_t *v_cache_w;
  float k_scale, v_scale_w;
  // scale tables of an 8-bit cache (kernels built with SC): the scale of
  // (physical block e, KV head g) is k_scales[e * scale_sb + g * scale_sh];
  // scale_log2 and v_scale then carry no cache scale
  const float *k_scales;
  const float *v_scales;
  int scale_sb, scale_sh;
};

// ---------------------------------------------------------------------------
// per-type geometry
// ---------------------------------------------------------------------------

template <int QT, int KT, int D>
struct Geo {
  static constexpr int kb = ElemBytes<KT>::value;   // cache element bytes
  static constexpr int row = D * kb;                // bytes of one head's row
  // K in the MFMA operand layout: lane l holds token l%16; its piece i is
  // row bytes k_byte(i, l/16) = [64 i + 16 jq, +16)
  static constexpr int k_lane_bytes = D / 4 * kb;
  static constexpr int nkl = k_lane_bytes / 16;     // 16-byte K pieces per lane per block
  static __device__ __forceinline__ uint32_t k_byte(int i, int jq) { return 64 * i + 16 * jq; }
  // first element of MFMA step s for lane group jq (8 consecutive elements,
  // or one for fp32)
  static __device__ __forceinline__ int q_elem(int s, int jq) {
    if constexpr (QT == PA_F32) return 16 * (s / 4) + 4 * jq + s % 4;
    else if constexpr (kb == 1) return 64 * (s / 2) + 16 * jq + 8 * (s % 2);
    else return 32 * s + 8 * jq;
  }
  static constexpr int ksteps = (QT == PA_F32) ? D / 4 : D / 32;  // MFMAs per block
  // V, accumulate layout: lane (r, c) holds elements [8c, 8c+8) of row r
  static constexpr int v_piece = 8 * kb;            // bytes per lane per V load
  static constexpr int lpt = D / 8;                 // lanes per token row
  static constexpr int rv = kWave / lpt;            // token rows per V load
  static constexpr int nvl = kBs / rv;              // V loads per lane per block
  // K global loads are row-contiguous like V (16 bytes per lane, lanes of a
  // quad on adjacent bytes, so each quad is one cache access): lane (rk, ck)
  // of load i reads bytes [16 ck, +16) of row i * rvk + rk. The tile then
  // goes through LDS, rows padded by 16 bytes (the 16 rows of a transposed
  // read land in distinct banks), into the MFMA operand layout.
  static constexpr int lpk = row / 16;              // lanes per row of a K load
  static constexpr int rvk = kWave / lpk;           // rows per K load
  static constexpr int krs = row + 16;              // LDS row stride of the K tile
  static_assert(nkl >= 1 && nvl >= 1 && rvk * nkl == kBs, "unsupported geometry");
};

// 16-token sub-blocks holding n tokens
__device__ __forceinline__ int num_blocks_of(int n) { return n > 0 ? (n + kBs - 1) / kBs : 0; }

template <int QT> struct QOpT { using type = u32x4; };  // 8 x 16-bit
template <> struct QOpT<PA_F32> { using type = float; };

// One V load: 8 cache elements.
template <int KT> struct VPiece { uint32_t w[2 * ElemBytes<KT>::value]; };

// Buffer resources: the hardware range check of a raw buffer load returns
// zeros without touching memory for bytes at or beyond num_records, which
// turns the loads of units past a range's end into no-ops while keeping every
// load instruction unconditional (one resource per block and cache).
constexpr int kRsrcFlags = 0x00020000;  // gfx9 word 3: 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint8_t *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), (short)0, (int)bytes,
                                           kRsrcFlags);
}

// K and V are streamed once: loads carry the non-temporal hint (aux bit 1,
// "nt" on gfx950), which measurably raises the sustained read rate.
constexpr int kLoadAux = 2;
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kLoadAux);
}

template <int KT>
__device__ __forceinline__ void buf_load_v(VPiece<KT> &pc, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (ElemBytes<KT>::value == 4) {
    const u32x4 a = buf_load16(r, off);
    const u32x4 b = buf_load16(r, off + 16);
    pc.w[0] = a.x; pc.w[1] = a.y; pc.w[2] = a.z; pc.w[3] = a.w;
    pc.w[4] = b.x; pc.w[5] = b.y; pc.w[6] = b.z; pc.w[7] = b.w;
  } else if constexpr (ElemBytes<KT>::value == 2) {
    const u32x4 a = buf_load16(r, off);
    pc.w[0] = a.x; pc.w[1] = a.y; pc.w[2] = a.z; pc.w[3] = a.w;
  } else {
    const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kLoadAux);
    pc.w[0] = a.x; pc.w[1] = a.y;
  }
}

// Byte n of w as a signed int8 code, in float (exact; one sign-extending
// byte-select conversion).
__device__ __forceinline__ float int8_byte(uint32_t w, int n) {
  return (float)(int)(signed char)(w >> (8 * n));
}

// Two floats that are exact in the query's 16-bit type, packed (low, high).
template <int QT>
__device__ __forceinline__ uint32_t pack16_exact(float lo, float hi) {
  if constexpr (QT == PA_BF16) {
    typedef __bf16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, h2{(__bf16)lo, (__bf16)hi});
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, h2{(_Float16)lo, (_Float16)hi});
  }
}

// 8 V elements -> fp32; all zero when the token is masked.
template <int KT>
__device__ __forceinline__ void widen_v(const VPiece<KT> &pc, bool ok, float (&x)[8]) {
  constexpr int NW = 2 * ElemBytes<KT>::value;
  uint32_t w[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) w[i] = ok ? pc.w[i] : 0u;
  if constexpr (KT == PA_F32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = u2f(w[i]);
  } else if constexpr (KT == PA_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(w[i]);
      x[2 * i + 1] = bf16_hi(w[i]);
    }
  } else if constexpr (KT == PA_F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = f16_lo(w[i]);
      x[2 * i + 1] = f16_hi(w[i]);
    }
  } else if constexpr (KT == PA_INT8) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) x[4 * i + k] = int8_byte(w[i], k);
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
      x[4 * i] = lo.x;
      x[4 * i + 1] = lo.y;
      x[4 * i + 2] = hi.x;
      x[4 * i + 3] = hi.y;
    }
  }
}

// fp8 pair (bytes 0,1 or 2,3 of a word) widened exactly to the query's 16-bit type
template <int QT, bool HI>
__device__ __forceinline__ uint32_t fp8_pair_to_16(uint32_t w) {
  if constexpr (QT == PA_BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  }
}

// int8 pair (bytes 0,1 or 2,3 of a word) widened exactly to the query's
// 16-bit type: codes are integers of at most 8 significant bits.
template <int QT, bool HI>
__device__ __forceinline__ uint32_t int8_pair_to_16(uint32_t w) {
  return pack16_exact<QT>(int8_byte(w, HI ? 2 : 0), int8_byte(w, HI ? 3 : 1));
}

// B operand of MFMA step s from the lane's K loads of one block.
template <int QT, int KT, int D>
__device__ __forceinline__ typename QOpT<QT>::type k_operand(const u32x4 *k, int s) {
  if constexpr (QT == PA_F32) {
    const u32x4 w = k[s / 4];
    const int t = s % 4;
    return u2f(t == 0 ? w.x : t == 1 ? w.y : t == 2 ? w.z : w.w);
  } else if constexpr (ElemBytes<KT>::value == 1) {
    const u32x4 w = k[s / 2];
    const uint32_t a = (s % 2) ? w.z : w.x;
    const uint32_t b = (s % 2) ? w.w : w.y;
    u32x4 r;
    if constexpr (KT == PA_INT8) {
      r.x = int8_pair_to_16<QT, false>(a);
      r.y = int8_pair_to_16<QT, true>(a);
      r.z = int8_pair_to_16<QT, false>(b);
      r.w = int8_pair_to_16<QT, true>(b);
    } else {
      r.x = fp8_pair_to_16<QT, false>(a);
      r.y = fp8_pair_to_16<QT, true>(a);
      r.z = fp8_pair_to_16<QT, false>(b);
      r.w = fp8_pair_to_16<QT, true>(b);
    }
    return r;
  } else {
    return k[s];
  }
}

template <int QT>
__device__ __forceinline__ f32x4 mfma(typename QOpT<QT>::type a, typename QOpT<QT>::type b,
                                      f32x4 c) {
  if constexpr (QT == PA_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else if constexpr (QT == PA_F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
}

// 16x16x16 MFMA on 16-bit operands (four per lane, as two packed words):
// lane l holds A[l % 16][4 (l / 16) + 0..3] and B[4 (l / 16) + 0..3][l % 16],
// and gets D[4 (l / 16) + 0..3][l % 16].
template <int QT>
__device__ __forceinline__ f32x4 mfma16(u32x2 a, u32x2 b, f32x4 c) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  if constexpr (QT == PA_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
}

// Two fp32 values as a sum of two values of the query's 16-bit type each,
// packed in pairs: hi = round(x) (nearest even), lo = round(x - hi), where
// x - hi is exact in fp32. hi + lo carries about 16 significant bits, so a
// product over such pairs is as accurate as fp32 accumulation needs.
// (The casts compile to the hardware's packed conversions, which round to
// nearest even.)
template <int QT>
__device__ __forceinline__ void split16(float a, float b, uint32_t &hi, uint32_t &lo) {
  if constexpr (QT == PA_BF16) {
    typedef __bf16 h2 __attribute__((ext_vector_type(2)));
    const h2 h = {(__bf16)a, (__bf16)b};
    const h2 l = {(__bf16)(a - (float)h.x), (__bf16)(b - (float)h.y)};
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 h = {(_Float16)a, (_Float16)b};
    const h2 l = {(_Float16)(a - (float)h.x), (_Float16)(b - (float)h.y)};
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
  }
}

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

// Orders a wave's LDS accesses (one wave writes and reads its own region;
// LDS instructions of a wave execute in order, so a compiler fence suffices).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }


template <int QT, int KT, int D, int GH, int NBI, int NW>
struct Shared {
  float p[NW][NBI * kBs][GH];   // probabilities of the current unit
  float alpha[NW][GH];          // rescale factor of the current unit
  float m[NW][GH];              // per-wave softmax state at the end of a range
  float l[NW][GH];
  float mt[NW][GH];             // per-wave true maxima at the end of a range
  float acc[NW][GH][D];
  // K tiles of the current unit, one per wave and block
  uint8_t kt[NW][NBI][kBs * (D * ElemBytes<KT>::value + 16)] __attribute__((aligned(16)));
  int start[kMaxBalancedSeqs + 1];  // balanced split: first block of each sequence
  int ctx[kMaxBalancedSeqs];        // balanced split: context length of each sequence
  int wave_sum[NW];
  int first[2];  // balanced split: the sequence holding the first block of each share taken
  int progress[NW];  // one wave per head row: units computed by each wave
};

// The appended token of a segment's sequence (decode with append): the raw
// source bytes of its K row piece (lane i < lpk: the source elements of
// cache bytes [16 i, 16 i + 16)) and of its V piece (lane (r, c): elements
// [8c, 8c + 8)), and where the token sits.
template <int QT, int KT, int D>
struct AppendRow {
  static constexpr int kb = ElemBytes<KT>::value;
  static constexpr int qb = ElemBytes<QT>::value;
  static constexpr int kcache = 16 * kb / qb;   // cache bytes per 16 source bytes
  static constexpr int klanes = D * qb / 16;    // lanes holding the K row
  static constexpr int vsrc = 8 * qb;           // source bytes per V piece
  u32x4 k;  // lane i < klanes: source elements of cache bytes [kcache i, kcache (i + 1))
  u32x4 v[vsrc / 16];
  int blk;  // sub-block (within the sequence) holding the new token; -1: none here
  int t;    // its row in that sub-block
  int id;   // the physical block's id (block-table entry)
  int sub;  // the sub-block within that physical block
};

// The same row in cache encoding: lane i < klanes holds cache bytes
// [kcache i, kcache (i + 1)) of the K row (in kc.x .. or all of kc), lane
// (r, c) the V piece of elements [8c, 8c + 8).
template <int QT, int KT, int D>
struct AppendEnc {
  u32x4 k;
  VPiece<KT> v;
  int blk, t, id;
};

// 8 source elements (16 bytes, 16-bit types) -> 8 cache bytes of x / scale
// (fp8 e4m3fn or int8, round to nearest even, saturating), as the slot write
// does.
template <int QT, int KT>
__device__ __forceinline__ u32x2 q8_of(const u32x4 &src, float scale) {
  const uint32_t w[4] = {src.x, src.y, src.z, src.w};
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = QT == PA_BF16 ? bf16_lo(w[i]) : f16_lo(w[i]);
    x[2 * i + 1] = QT == PA_BF16 ? bf16_hi(w[i]) : f16_hi(w[i]);
  }
  auto enc = [](float v) { return KT == PA_INT8 ? f32_to_int8(v) : f32_to_e4m3fn(v); };
  uint32_t o[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    o[i] = enc(x[4 * i] / scale) | (enc(x[4 * i + 1] / scale) << 8) |
           (enc(x[4 * i + 2] / scale) << 16) | (enc(x[4 * i + 3] / scale) << 24);
  return u32x2{o[0], o[1]};
}

// Source elements -> one V piece (8 cache elements) in cache encoding.
template <int QT, int KT, int N>
__device__ __forceinline__ VPiece<KT> cache_vpiece(const u32x4 (&src)[N], float scale) {
  VPiece<KT> pc;
  if constexpr (QT == KT) {
#pragma unroll
    for (int i = 0; i < 2 * ElemBytes<KT>::value; ++i) {
      const u32x4 q = src[i / 4];
      pc.w[i] = (i % 4 == 0) ? q.x : (i % 4 == 1) ? q.y : (i % 4 == 2) ? q.z : q.w;
    }
  } else {
    static_assert(ElemBytes<KT>::value == 1 && N == 1, "8 source elements of 16 bits");
    const u32x2 o = q8_of<QT, KT>(src[0], scale);
    pc.w[0] = o.x;
    pc.w[1] = o.y;
  }
  return pc;
}

template <int QT, int KT, int D>
__device__ __forceinline__ AppendEnc<QT, KT, D> encode_append(const AppendRow<QT, KT, D> &a,
                                                              float k_scale, float v_scale) {
  AppendEnc<QT, KT, D> e;
  if constexpr (QT == KT) {
    e.k = a.k;
  } else {
    const u32x2 k8 = q8_of<QT, KT>(a.k, k_scale);
    e.k = u32x4{k8.x, k8.y, 0u, 0u};
  }
  e.v = cache_vpiece<QT, KT>(a.v, v_scale);
  e.blk = a.blk;
  e.t = a.t;
  e.id = a.id;
  return e;
}

template <int QT, int KT, int D, int GH, int NBI>
struct Stage {
  using G = Geo<QT, KT, D>;
  u32x4 k[NBI][G::nkl];
  VPiece<KT> v[NBI][G::nvl];
};

// A range is the blocks [blo, bhi) of sequence b, written as partial
// `piece` (or to `out` when it is the whole sequence). The units of all
// ranges of a workgroup are dealt to its waves in turn, counting on across
// ranges (so the waves' shares of the work differ by one unit at most); a
// segment is up to kIdsUnits of a wave's units of one range (chunk c), the
// span one register of block ids covers.
// A workgroup's work item: the query heads h0 .. h0 + GH - 1 (KV head g)
// over one balanced share (blocks [lo, hi) of all sequences end to end), or
// over a single range in the other modes.
struct Item {
  int h0, g;
  int share, lo, hi;
};

// Block ids of a segment's units, one per lane (see fetch_ids).
struct Ids {
  int entry;  // block-table entry
  int sub;    // 16-token sub-block within that block; with 8-token blocks,
              // the unit's second block (its table entry, or -1 past the context)
  int ok;     // the lane holds a unit's block (scale tables only)
  float ks, vs;  // that block's K and V scales for the segment's KV head (scale tables only)
};

struct Seg {
  int item;   // work item of the range
  int h0, g;  // its query heads and KV head
  int share, ihi;  // balanced: its share and the share's end block
  int b, blo, bhi, piece;
  int n;      // context length of sequence b
  int whole;  // the range is the whole sequence
  int u0;     // units of the workgroup's earlier ranges
  int w0;     // this wave's first unit of the range
  int c;      // chunk of the range
  int nk;     // this wave's units in the range
  int kn;     // this wave's units in this segment
  int last;   // last segment of its range: the range's epilogue follows it
  int valid;
};

// All ranges of a workgroup's work items (one range, or the ranges of one
// or two balanced shares), all waves. The segments of a wave form one
// pipelined stream: while the last units of a segment are computed, the
// first unit of the next segment is already being loaded (its block ids and
// query fragments were fetched one segment ahead), so a switch between
// ranges costs only the epilogue of the finished range.
template <int QT, int KT, int D, int GH, int NBI, int NS, int NW, bool APP, bool SUB, bool RW,
          bool SC>
__device__ __forceinline__ void run_ranges(const DecodeParams &p,
                                           Shared<QT, KT, D, GH, NBI, NW> &sh, const Item (&items)[2],
                                           int n_items, int b_first, int n_first, int blo_first,
                                           int bhi_first, int piece_first, bool whole_first) {
  using G = Geo<QT, KT, D>;
  using QOp = typename QOpT<QT>::type;
  using St = Stage<QT, KT, D, GH, NBI>;
  using AR = AppendRow<QT, KT, D>;
  using AE = AppendEnc<QT, KT, D>;
  constexpr int QB = ElemBytes<QT>::value;
  constexpr int kIdsUnits = kWave / NBI;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = uniform(tid >> 6);
  // waves that share a range's units: all NW, or (RW: one wave per head
  // row) the wave alone; dw is this wave's place among them
  constexpr int ND = RW ? 1 : NW;
  const int dw = RW ? 0 : wave;
  const int jq = lane >> 4;  // MFMA lane group
  const int tl = lane & 15;  // MFMA column: token within a block
  const int r = lane / G::lpt;  // V layout: token row within a load
  const int c = lane % G::lpt;  // V layout: 8-element column group
  const int Hq = p.num_q_heads;
  const int B = p.num_seqs;
  const bool balanced = p.mode == kSplitBalanced;

  // ---- segments ------------------------------------------------------------
  auto make_seg = [&](int item, const Item &it, int b, int n, int blo, int bhi, int piece,
                      bool whole, int u0, int ch) {
    Seg sg;
    sg.item = item;
    sg.h0 = it.h0;
    sg.g = it.g;
    sg.share = it.share;
    sg.ihi = it.hi;
    sg.b = b;
    sg.n = n;
    sg.blo = blo;
    sg.bhi = bhi;
    sg.piece = piece;
    sg.whole = whole;
    sg.u0 = u0;
    sg.w0 = (dw - u0 % ND + ND) % ND;
    sg.c = ch;
    const int nunits = (bhi - blo + NBI - 1) / NBI;
    sg.nk = sg.w0 < nunits ? (nunits - sg.w0 + ND - 1) / ND : 0;
    const int nchunks = max(1, (sg.nk + kIdsUnits - 1) / kIdsUnits);
    sg.kn = max(0, min(kIdsUnits, sg.nk - ch * kIdsUnits));
    sg.last = ch == nchunks - 1;
    sg.valid = 1;
    return sg;
  };
  // first chunk of the range of sequence b within balanced item it
  auto range_seg = [&](int item, const Item &it, int b, int u0) {
    const int st = uniform(sh.start[b]), en = uniform(sh.start[b + 1]);
    const int blo = max(it.lo, st) - st, bhi = min(it.hi, en) - st;
    return make_seg(item, it, b, uniform(sh.ctx[b]), blo, bhi, it.share + b,
                    blo == 0 && bhi == en - st, u0, 0);
  };
  // the segment after sg: the next chunk of its range, else the first chunk
  // of the next non-empty sequence of the share, else the first range of
  // the next item
  auto next_seg = [&](const Seg &sg) {
    Seg nx = sg;
    nx.valid = 0;
    if (!sg.valid) return nx;
    if (!sg.last) {
      nx.c = sg.c + 1;
      nx.kn = max(0, min(kIdsUnits, sg.nk - nx.c * kIdsUnits));
      nx.last = nx.c == max(1, (sg.nk + kIdsUnits - 1) / kIdsUnits) - 1;
      nx.valid = 1;
      return nx;
    }
    if (!balanced) return nx;
    const int u0 = sg.u0 + (sg.bhi - sg.blo + NBI - 1) / NBI;
    int b = sg.b + 1;
    while (b < B && sh.start[b] < sg.ihi && sh.start[b + 1] == sh.start[b]) ++b;
    b = uniform(b);
    if (b < B && uniform(sh.start[b]) < sg.ihi) {
      const int st = uniform(sh.start[b]), en = uniform(sh.start[b + 1]);
      const int bhi = min(sg.ihi, en) - st;
      Seg r = make_seg(sg.item, Item{sg.h0, sg.g, sg.share, 0, sg.ihi}, b, uniform(sh.ctx[b]), 0,
                       bhi, sg.share + b, bhi == en - st, u0, 0);
      return r;
    }
    if (sg.item != 0 || n_items < 2) return nx;
    return range_seg(1, items[1], uniform(sh.first[1]), u0);
  };
  // lane i: block i % NBI of the segment's unit i / NBI -- the block-table
  // entry of its physical block (loaded; used only where the unit's loads
  // are issued, so that nothing waits for it earlier) and its sub-block
  // within that physical block
  auto fetch_ids = [&](const Seg &sg) {
    const int kk = sg.c * kIdsUnits + lane / NBI;
    const int j = sg.blo + (sg.w0 + kk * ND) * NBI + lane % NBI;
    const bool ok = sg.valid && kk < sg.nk && j < sg.bhi;
    const int32_t *row = p.block_tables + (size_t)(sg.valid ? sg.b : 0) * p.max_blocks_per_seq;
    const int e = ok ? j : 0;
    if constexpr (SUB) {
      if (p.sub_log2 == kHalfBlocks) {
        // 8-token blocks: the unit's rows 8..15 sit in the table's next
        // entry, which exists only where the context reaches past row 7
        const bool two = ok && 2 * e + 1 < (sg.n + 7) / 8;
        const int second = row[two ? 2 * e + 1 : 0];
        return Ids{row[2 * e], two ? second : -1, ok, 0.f, 0.f};
      }
      return Ids{row[e >> p.sub_log2], e & ((1 << p.sub_log2) - 1), ok, 0.f, 0.f};
    } else {
      return Ids{row[e], 0, ok, 0.f, 0.f};
    }
  };
  // scale tables: each lane's block scales for KV head g, loaded where the
  // segment's ids are first used (their load is long done by then); lanes
  // holding no unit read entry 0
  auto load_scales = [&](Ids &ids, int g) {
    if constexpr (SC) {
      const size_t i =
          ids.ok ? (size_t)ids.entry * p.scale_sb + (size_t)g * p.scale_sh : (size_t)0;
      ids.ks = p.k_scales[i];
      ids.vs = p.v_scales[i];
    }
  };
  // the appended token of sg's sequence, when sg's range holds it (loads
  // are issued in any case, of nothing otherwise)
  constexpr bool appending = APP;
  auto load_app = [&](const Seg &sg) {
    AR a;
    // wave-uniform values, stated as such so that the descriptors below
    // stay scalar (see issue)
    const int n = uniform(sg.n);
    const int lb = n > 0 ? (n - 1) / kBs : 0;
    const bool here = appending && sg.valid && n > 0 && lb >= sg.blo && lb < sg.bhi;
    a.blk = here ? lb : -1;
    a.t = n > 0 ? (n - 1) % kBs : 0;
    const int b = uniform(sg.valid ? sg.b : 0);
    const size_t rowoff = ((size_t)b * p.num_kv_heads + uniform(sg.g)) * D * AR::qb;
    const uint32_t bytes = here ? (uint32_t)(D * AR::qb) : 0u;
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(appending ? p.new_k + rowoff : p.q, bytes);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(appending ? p.new_v + rowoff : p.q, bytes);
    a.k = __builtin_amdgcn_raw_buffer_load_b128(rk, (lane % AR::klanes) * 16, 0, 0);
#pragma unroll
    for (int i = 0; i < AR::vsrc / 16; ++i)
      a.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, c * AR::vsrc + 16 * i, 0, 0);
    const __amdgpu_buffer_rsrc_t rt = block_rsrc(
        reinterpret_cast<const uint8_t *>(p.block_tables + (size_t)b * p.max_blocks_per_seq),
        here ? (uint32_t)p.max_blocks_per_seq * 4u : 0u);
    // the physical block's id; its sub-block is added where it is used
    const int lbe = SUB ? lb >> p.sub_log2 : lb;
    a.id = (int)__builtin_amdgcn_raw_buffer_load_b32(rt, (uint32_t)lbe * 4u, 0, 0);
    a.sub = SUB ? lb & ((1 << p.sub_log2) - 1) : 0;
    return a;
  };
  // query fragments (A operand) of sequence b: row tl holds head h0 + tl % GH
  auto load_q = [&](int b, int h0, QOp (&qa)[G::ksteps]) {
    const uint8_t *qrow = p.q + ((size_t)b * Hq + h0 + tl % GH) * D * QB;
    if constexpr (QT == PA_F32) {
      const float *qf = reinterpret_cast<const float *>(qrow);
#pragma unroll
      for (int s = 0; s < G::ksteps; s += 4) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(qf + G::q_elem(s, jq));
        qa[s] = u2f(w.x);
        qa[s + 1] = u2f(w.y);
        qa[s + 2] = u2f(w.z);
        qa[s + 3] = u2f(w.w);
      }
    } else {
#pragma unroll
      for (int s = 0; s < G::ksteps; ++s)
        qa[s] = *reinterpret_cast<const u32x4 *>(qrow + G::q_elem(s, jq) * QB);
    }
  };

  // ---- per-wave softmax state ----------------------------------------------
  // m: reference maximum (lazy, see compute_unit), l: sum of exp2(s - m),
  // mt: the lane's true running maximum
  float m[4], l[4], mt[4];
  // P.V on MFMA for 4 to 16 query heads of a 128-wide head (16-bit queries;
  // per block of the unit): 16x16x16 products per 16 output columns replace the
  // GH x 8 fp32 FMAs per V element on the vector ALU (rows past GH repeat
  // the first GH, as in the logits tile).
  // Lane (r, c) of the V layout holds tokens 4i + r (i = 0..3), elements
  // [8c, 8c + 8): MFMA t takes those four tokens as its k = 4r .. 4r + 3 and
  // element 8c + t as column c, so its output column c is element 8c + t of
  // the rows' P.V; the probabilities go through LDS in the same token order
  // and enter as two 16-bit parts (split16), V exactly.
  // Output rows are heads 4 (l / 16) + j, the rows this lane's softmax state
  // already holds, so the rescale needs no exchange.
  constexpr bool PVM = GH >= 4 && D == 128 && QT != PA_F32;
  float acc[PVM ? 1 : GH][8];
  f32x4 acc2[PVM ? 8 : 1];
  auto reset = [&]() {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      m[v] = -INFINITY;
      mt[v] = -INFINITY;
      l[v] = 0.0f;
    }
    if constexpr (PVM) {
#pragma unroll
      for (int t = 0; t < 8; ++t) acc2[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    } else {
#pragma unroll
      for (int h = 0; h < GH; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
    }
  };

  const uint32_t rowstride = (uint32_t)p.num_kv_heads * G::row;
  const uint32_t blk_bytes = rowstride * kBs;          // < 2^31, checked on the host
  const uint32_t k_off = (lane / G::lpk) * rowstride + (lane % G::lpk) * 16;
  uint32_t v_off[G::nvl];
#pragma unroll
  for (int i = 0; i < G::nvl; ++i) v_off[i] = (i * G::rv + r) * rowstride + c * G::v_piece;
  const float sl2 = p.scale_log2;

  // Loads of a unit's rows 0..7 and 8..15 of KV head g from two cache
  // ranges: byte offsets off0 and off1 of rows 0 and 8 (8-token blocks: two
  // physical blocks, the second absent (has1 false) where the context ends
  // before row 8; otherwise one 16-token block or sub-block, off1 = off0 + 8
  // rows). A load instruction of up to eight rows reads one range, chosen at
  // compile time. (One range per 16-token block measured 1.3 to 1.6 us slower
  // per launch on the Llama-shaped batch, within the run-to-run spread on
  // the other batches.)
  // A K load of sixteen rows (8-bit cache, d = 64) is issued once per range,
  // each lane's offset pointing past the other range (2^31 bytes, above any
  // block: checked on the host), where the load returns zeros, and the two
  // results are or-ed.
  auto issue_halves = [&](size_t off0, size_t off1, bool valid, bool has1, int g,
                          u32x4 (&kst)[G::nkl], VPiece<KT> (&vst)[G::nvl]) {
    const uint32_t back = (kBs / 2) * rowstride;
    const uint32_t span = back - (uint32_t)g * G::row;
    const __amdgpu_buffer_rsrc_t rk0 = block_rsrc(p.k_cache + off0, valid ? span : 0u);
    const __amdgpu_buffer_rsrc_t rv0 = block_rsrc(p.v_cache + off0, valid ? span : 0u);
    const __amdgpu_buffer_rsrc_t rk1 = block_rsrc(p.k_cache + off1, valid && has1 ? span : 0u);
    const __amdgpu_buffer_rsrc_t rv1 = block_rsrc(p.v_cache + off1, valid && has1 ? span : 0u);
    constexpr uint32_t kFar = 0x80000000u;
#pragma unroll
    for (int i = 0; i < G::nkl; ++i) {
      if constexpr (G::rvk <= kBs / 2) {
        const int h = i * G::rvk / (kBs / 2);
        kst[i] = buf_load16(h ? rk1 : rk0, k_off + i * G::rvk * rowstride - h * back);
      } else {
        const bool low = lane / G::lpk < kBs / 2;
        const u32x4 a = buf_load16(rk0, low ? k_off : kFar);
        const u32x4 b = buf_load16(rk1, low ? kFar : k_off - back);
        kst[i] = u32x4{a.x | b.x, a.y | b.y, a.z | b.z, a.w | b.w};
      }
    }
#pragma unroll
    for (int i = 0; i < G::nvl; ++i) {
      static_assert(G::rv <= kBs / 2, "a V load reads rows of one 8-token block");
      const int h = i * G::rv / (kBs / 2);
      buf_load_v<KT>(vst[i], h ? rv1 : rv0, v_off[i] - h * back);
    }
  };

  // Loads of one unit of KV head g into a register stage: the unit whose
  // block ids start at lane u * NBI of `ids`; an invalid unit loads nothing.
  auto issue = [&](const Ids &ids, int u, bool valid, int g_in, St &st) {
    // g is the same in every lane; in several instantiations (scale tables,
    // d = 64, larger blocks, workgroups sharing ranges among waves) the
    // compiler otherwise loses track of that and wraps every buffer load of
    // the unit in a loop over the distinct descriptor values of the wave
    const int g = uniform(g_in);
    const size_t head = (size_t)g * G::row, half = (size_t)rowstride * (kBs / 2);
#pragma unroll
    for (int bi = 0; bi < NBI; ++bi) {
      const int lidx = min(u * NBI + bi, kWave - 1);
      const int id = __builtin_amdgcn_readlane(ids.entry, lidx);
      if (SUB && p.sub_log2 == kHalfBlocks) {
        // two 8-token blocks
        const int sub = __builtin_amdgcn_readlane(ids.sub, lidx);
        issue_halves((size_t)id * half + head, (size_t)(sub < 0 ? 0 : sub) * half + head, valid,
                     sub >= 0, g, st.k[bi], st.v[bi]);
      } else {
        // a 16-token block, or a sub-block of a larger one
        int sb = id;
        if constexpr (SUB) sb = (id << p.sub_log2) + __builtin_amdgcn_readlane(ids.sub, lidx);
        const size_t off = (size_t)sb * blk_bytes + head;
        issue_halves(off, off + half, valid, true, g, st.k[bi], st.v[bi]);
      }
    }
  };

  auto compute_unit = [&](int jb, int tok_lim, const QOp (&qa)[G::ksteps], const St &st,
                          const AE &app, int g, bool writer, const Ids &ids, int u) {
    // logits, log2 domain; masked tokens -inf
    float sv[NBI][4];
    // per block: the logit factor (the softmax scale in the log2 domain,
    // times the block's K scale with scale tables) and the V scale that
    // multiplies the block's probabilities in P.V (not in the sums l)
    float lf[NBI], vsc[NBI];
#pragma unroll
    for (int bi = 0; bi < NBI; ++bi) {
      if constexpr (SC) {
        const int li = u * NBI + bi;
        lf[bi] = sl2 * __builtin_bit_cast(
                           float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ids.ks), li));
        vsc[bi] = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ids.vs), li));
      } else {
        lf[bi] = sl2;
        vsc[bi] = 1.0f;
      }
    }
    // K tile: registers (row-contiguous) -> LDS -> MFMA operand layout, in
    // which lane (tl, jq) holds bytes k_byte(i, jq) of token row tl
#pragma unroll
    for (int bi = 0; bi < NBI; ++bi) {
#pragma unroll
      for (int i = 0; i < G::nkl; ++i)
        *reinterpret_cast<u32x4 *>(&sh.kt[wave][bi][(i * G::rvk + lane / G::lpk) * G::krs +
                                                    (lane % G::lpk) * 16]) = st.k[bi][i];
      if (APP && app.blk == jb + bi) {
        // the appended token: its K row replaces the cache's (which is never
        // read for it), and the first head row of the KV head writes it back
        if (lane < AR::klanes) {
          uint8_t *krow = &sh.kt[wave][bi][app.t * G::krs + lane * AR::kcache];
          uint8_t *kdst = p.k_cache_w + ((size_t)app.id * kBs + app.t) * rowstride +
                          (size_t)g * G::row + lane * AR::kcache;
          if constexpr (QT == KT) {
            *reinterpret_cast<u32x4 *>(krow) = app.k;
            if (writer) *reinterpret_cast<u32x4 *>(kdst) = app.k;
          } else {
            const u32x2 kp = {app.k.x, app.k.y};
            *reinterpret_cast<u32x2 *>(krow) = kp;
            if (writer) *reinterpret_cast<u32x2 *>(kdst) = kp;
          }
        }
        const VPiece<KT> &vp = app.v;
        if (writer && r == 0) {
          uint32_t *dst = reinterpret_cast<uint32_t *>(
              p.v_cache_w + ((size_t)app.id * kBs + app.t) * rowstride + (size_t)g * G::row +
              c * G::v_piece);
#pragma unroll
          for (int w = 0; w < 2 * ElemBytes<KT>::value; ++w) dst[w] = vp.w[w];
        }
      }
    }
    wave_lds_fence();
#pragma unroll
    for (int bi = 0; bi < NBI; ++bi) {
      u32x4 kop[G::nkl];
#pragma unroll
      for (int i = 0; i < G::nkl; ++i)
        kop[i] = *reinterpret_cast<const u32x4 *>(&sh.kt[wave][bi][tl * G::krs + G::k_byte(i, jq)]);
      f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < G::ksteps; ++s) d = mfma<QT>(qa[s], k_operand<QT, KT, D>(kop, s), d);
      const bool ok = (jb + bi) * kBs + tl < tok_lim;
      sv[bi][0] = ok ? d.x * lf[bi] : -INFINITY;
      sv[bi][1] = ok ? d.y * lf[bi] : -INFINITY;
      sv[bi][2] = ok ? d.z * lf[bi] : -INFINITY;
      sv[bi][3] = ok ? d.w * lf[bi] : -INFINITY;
    }
    // Online softmax per MFMA row v (head (4*jq + v) % GH), with a lazy
    // reference maximum: m moves only when a logit passes it by more than
    // kLazyMax (log2 domain), so the probabilities exp2(s - m) stay below
    // 2^kLazyMax. Most units move no row: then the row reductions, the
    // rescale factors and the rescale of the sums and accumulators are
    // skipped (a wave-wide decision). m stays at most the true running
    // maximum, and a partial's (m, l, o) means the same for any such m.
    float lm[4];
    bool up = false;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      lm[v] = sv[0][v];
#pragma unroll
      for (int bi = 1; bi < NBI; ++bi) lm[v] = fmaxf(lm[v], sv[bi][v]);
      up |= lm[v] > m[v] + kLazyMax;  // not ||: no per-lane branches
      mt[v] = fmaxf(mt[v], lm[v]);
    }
    const bool any_up = __builtin_amdgcn_ballot_w64(up) != 0;
    float al[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if (any_up) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float mn = fmaxf(m[v], group_max<16>(lm[v]));
        al[v] = __builtin_amdgcn_exp2f(m[v] - mn);
        m[v] = mn;
        l[v] *= al[v];
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float sum = 0.0f;
#pragma unroll
      for (int bi = 0; bi < NBI; ++bi) {
        const float e = __builtin_amdgcn_exp2f(sv[bi][v] - m[v]);
        sv[bi][v] = e;
        sum += e;
      }
      l[v] += sum;
    }
    // hand the probabilities (and alpha) to the V layout
    if (4 * jq < GH) {
#pragma unroll
      for (int bi = 0; bi < NBI; ++bi)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (v < GH) sh.p[wave][bi * kBs + tl][4 * jq + v] = SC ? sv[bi][v] * vsc[bi] : sv[bi][v];
      if (!PVM && any_up && tl == 0) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (v < GH) sh.alpha[wave][4 * jq + v] = al[v];
      }
    }
    wave_lds_fence();
    if constexpr (PVM) {
      // rows 4 jq + j of acc2 are this lane's softmax rows: alpha in hand
      if (any_up) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          acc2[t].x *= al[0];
          acc2[t].y *= al[1];
          acc2[t].z *= al[2];
          acc2[t].w *= al[3];
        }
      }
#pragma unroll
      for (int bi = 0; bi < NBI; ++bi) {
      // A: P[head tl][tokens 4i + jq], i = 0..3
      float pk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pk[i] = sh.p[wave][bi * kBs + 4 * i + jq][tl % GH];
      uint32_t h0, l0, h1, l1;  // probabilities, high and low parts
      split16<QT>(pk[0], pk[1], h0, l0);
      split16<QT>(pk[2], pk[3], h1, l1);
      const u32x2 aop = {h0, h1}, aol = {l0, l1};
      // B: the lane's V pieces (tokens 4i + r), the appended row in place of
      // the cache's, masked tokens zero
      const bool newblk = APP && app.blk == jb + bi;
      const VPiece<KT> &vp = app.v;
      VPiece<KT> pcs[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tk = 4 * i + r;
        const uint32_t keep = (jb + bi) * kBs + tk < tok_lim ? ~0u : 0u;
        const uint32_t mk = (newblk && tk == app.t) ? ~0u : 0u;
#pragma unroll
        for (int w = 0; w < 2 * ElemBytes<KT>::value; ++w)
          pcs[i].w[w] = ((vp.w[w] & mk) | (st.v[bi][i].w[w] & ~mk)) & keep;
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        u32x2 bop;
        if constexpr (ElemBytes<KT>::value == 2) {
          // element t of tokens (i0, i1): its 16-bit halves side by side
          const uint32_t sel = (t % 2) ? 0x07060302u : 0x05040100u;
          bop.x = __builtin_amdgcn_perm(pcs[1].w[t / 2], pcs[0].w[t / 2], sel);
          bop.y = __builtin_amdgcn_perm(pcs[3].w[t / 2], pcs[2].w[t / 2], sel);
        } else if constexpr (KT == PA_INT8) {
          // byte t of tokens (i0, i1), each converted straight from its word
          bop.x = pack16_exact<QT>(int8_byte(pcs[0].w[t / 4], t % 4),
                                   int8_byte(pcs[1].w[t / 4], t % 4));
          bop.y = pack16_exact<QT>(int8_byte(pcs[2].w[t / 4], t % 4),
                                   int8_byte(pcs[3].w[t / 4], t % 4));
        } else {
          // byte t of tokens (i0, i1) into bytes 0, 1, widened exactly
          const uint32_t sel = 0x0c0c0000u | ((4u + t % 4) << 8) | (uint32_t)(t % 4);
          const uint32_t w01 = __builtin_amdgcn_perm(pcs[1].w[t / 4], pcs[0].w[t / 4], sel);
          const uint32_t w23 = __builtin_amdgcn_perm(pcs[3].w[t / 4], pcs[2].w[t / 4], sel);
          bop.x = fp8_pair_to_16<QT, false>(w01);
          bop.y = fp8_pair_to_16<QT, false>(w23);
        }
        acc2[t] = mfma16<QT>(aop, bop, acc2[t]);
        acc2[t] = mfma16<QT>(aol, bop, acc2[t]);
      }
      }
    } else {
      if (any_up) {
        float a[GH];
#pragma unroll
        for (int h = 0; h < GH; ++h) a[h] = sh.alpha[wave][h];
#pragma unroll
        for (int h = 0; h < GH; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] *= a[h];
      }
#pragma unroll
      for (int bi = 0; bi < NBI; ++bi) {
        // the appended token's V piece, for the lanes holding its row
        const bool newblk = APP && app.blk == jb + bi;
        const VPiece<KT> &vp = app.v;
#pragma unroll
        for (int i = 0; i < G::nvl; ++i) {
          const int t = i * G::rv + r;
          const bool ok = (jb + bi) * kBs + t < tok_lim;
          float x[8];
          if (newblk) {
            // (a mask, not a select of references: both pieces stay in registers)
            const uint32_t mk = t == app.t ? ~0u : 0u;
            VPiece<KT> pc;
#pragma unroll
            for (int w = 0; w < 2 * ElemBytes<KT>::value; ++w)
              pc.w[w] = (vp.w[w] & mk) | (st.v[bi][i].w[w] & ~mk);
            widen_v<KT>(pc, ok, x);
          } else {
            widen_v<KT>(st.v[bi][i], ok, x);
          }
          float pw[GH];
#pragma unroll
          for (int h = 0; h < GH; ++h) pw[h] = sh.p[wave][bi * kBs + t][h];
#pragma unroll
          for (int h = 0; h < GH; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pw[h], x[e], acc[h][e]);
        }
      }
    }
    wave_lds_fence();
  };

  // One wave per head row: the two waves of a SIMD have the same work, but
  // the hardware issues for the older one first, which then finishes far
  // ahead (about 30 against 44 us on the Llama-shaped batch) and leaves its
  // SIMD half idle. A wave that is ahead of its SIMD partner (wave ^ 4)
  // drops its issue priority, one behind raises it. Only the issue order
  // changes, never the arithmetic.
  int done_units = 0;
  if (RW && lane == 0) sh.progress[wave] = 0;
  auto pace = [&]() {
    if constexpr (RW && NW == 8) {
      ++done_units;
      if (lane == 0) sh.progress[wave] = done_units;
      const int other = sh.progress[wave ^ 4];
      if (done_units > other) __builtin_amdgcn_s_setprio(0);
      else __builtin_amdgcn_s_setprio(2);
    }
  };

  // end of a range with one wave per head row (RW): the wave alone holds the
  // range's softmax state and writes its heads' partial (or the output, for
  // a whole sequence) with no exchange between waves
  // end of a range: the sums over a row's token lanes (against the
  // reference maximum m) and the row's true maximum. Partials carry the
  // range's true maximum Mt and l scaled to it, l * exp2(m - Mt) (a wave
  // with no unit in the range has l = 0 and m = Mt = -inf).
  auto row_totals = [&]() {
  #pragma unroll
    for (int v = 0; v < 4; ++v) {
      l[v] = group_sum<16>(l[v]);
      mt[v] = group_max<16>(mt[v]);
    }
  };
  auto to_true_max = [](float L, float M, float Mt) {
    return Mt == -INFINITY ? 0.0f : L * __builtin_amdgcn_exp2f(M - Mt);
  };

  auto epilogue_wave = [&](int b, int piece, bool whole, int h0) {
    row_totals();
    const bool to_out = whole && p.direct;
    auto put = [&](int h, int d0, const float (&x)[8], float M, float L, float Mt) {
      const size_t bh = (size_t)b * Hq + h0 + h;
      const float inv = p.v_scale / L;
      if (to_out) {
  #pragma unroll
        for (int e = 0; e < 8; ++e) store_elem<QT>(p.out, bh * D + d0 + e, x[e] * inv);
      } else {
        const size_t pi = (p.mode == kSplitBalanced)
                              ? (size_t)(h0 + h) * p.max_partitions + piece
                              : bh * p.max_partitions + piece;
        float *dst = p.tmp_out + pi * D + d0;
        *reinterpret_cast<f32x4 *>(dst) =
            f32x4{x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv};
        *reinterpret_cast<f32x4 *>(dst + 4) =
            f32x4{x[4] * inv, x[5] * inv, x[6] * inv, x[7] * inv};
        if (d0 == 0) {
          p.max_logits[pi] = Mt * kLn2;
          p.exp_sums[pi] = to_true_max(L, M, Mt);
        }
      }
    };
    if constexpr (PVM) {
      // lane (tl, jq): heads 4 jq + v, elements 8 tl + t (rows past GH
      // repeat the first GH and are not written)
      if (4 * jq < GH) {
  #pragma unroll
        for (int v = 0; v < 4; ++v) {
          float x[8];
  #pragma unroll
          for (int t = 0; t < 8; ++t)
            x[t] = v == 0 ? acc2[t].x : v == 1 ? acc2[t].y : v == 2 ? acc2[t].z : acc2[t].w;
          put(4 * jq + v, 8 * tl, x, m[v], l[v], mt[v]);
        }
      }
    } else {
      if (4 * jq < GH && tl == 0) {
  #pragma unroll
        for (int v = 0; v < 4; ++v)
          if (v < GH) {
            sh.m[wave][4 * jq + v] = m[v];
            sh.l[wave][4 * jq + v] = l[v];
            sh.mt[wave][4 * jq + v] = mt[v];
          }
      }
  #pragma unroll
      for (int h = 0; h < GH; ++h)
  #pragma unroll
        for (int e = 0; e < 8; ++e)
  #pragma unroll
          for (int off = G::lpt; off < kWave; off <<= 1) acc[h][e] += __shfl_xor(acc[h][e], off);
      wave_lds_fence();
      if (r == 0) {
  #pragma unroll
        for (int h = 0; h < GH; ++h)
          put(h, 8 * c, acc[h], sh.m[wave][h], sh.l[wave][h], sh.mt[wave][h]);
      }
      wave_lds_fence();
    }
  };

  // end of a range: merge the waves' softmax states and write the range's
  // partial (or the output, for a whole sequence)
  auto epilogue = [&](int b, int piece, bool whole, int h0) {
    if constexpr (RW) {
      epilogue_wave(b, piece, whole, h0);
      return;
    }
    // merge the waves: sums over the token lanes / rows, then across waves
    row_totals();
    if (4 * jq < GH && tl == 0) {
  #pragma unroll
      for (int v = 0; v < 4; ++v)
        if (v < GH) {
          sh.m[wave][4 * jq + v] = m[v];
          sh.l[wave][4 * jq + v] = l[v];
          sh.mt[wave][4 * jq + v] = mt[v];
        }
    }
    if constexpr (PVM) {
      // acc2[t] holds heads (4 jq + j) % GH, element 8 tl + t: whole sums
      // (rows past GH repeat the first GH)
      if (4 * jq < GH) {
  #pragma unroll
      for (int t = 0; t < 8; ++t) {
        sh.acc[wave][4 * jq + 0][8 * tl + t] = acc2[t].x;
        sh.acc[wave][4 * jq + 1][8 * tl + t] = acc2[t].y;
        sh.acc[wave][4 * jq + 2][8 * tl + t] = acc2[t].z;
        sh.acc[wave][4 * jq + 3][8 * tl + t] = acc2[t].w;
      }
      }
    } else {
  #pragma unroll
      for (int h = 0; h < GH; ++h)
  #pragma unroll
        for (int e = 0; e < 8; ++e)
  #pragma unroll
          for (int off = G::lpt; off < kWave; off <<= 1) acc[h][e] += __shfl_xor(acc[h][e], off);
      if (r == 0) {
  #pragma unroll
        for (int h = 0; h < GH; ++h)
  #pragma unroll
          for (int e = 0; e < 8; ++e) sh.acc[wave][h][c * 8 + e] = acc[h][e];
      }
    }
    __syncthreads();

    const bool to_out = whole && p.direct;
    for (int i = tid; i < GH * D; i += (NW * kWave)) {
      const int h = i / D, d = i % D;
      float M = -INFINITY;
  #pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, sh.m[w][h]);
      float L = 0.0f, O = 0.0f;
  #pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float sc = __builtin_amdgcn_exp2f(sh.m[w][h] - M);
        L += sh.l[w][h] * sc;
        O += sh.acc[w][h][d] * sc;
      }
      const float res = O * p.v_scale / L;
      const size_t bh = (size_t)b * Hq + h0 + h;
      if (to_out) {
        store_elem<QT>(p.out, bh * D + d, res);
      } else {
        const size_t pi = (p.mode == kSplitBalanced)
                              ? (size_t)(h0 + h) * p.max_partitions + piece
                              : bh * p.max_partitions + piece;
        p.tmp_out[pi * D + d] = res;
        if (d == 0) {
          float Mt = -INFINITY;
  #pragma unroll
          for (int w = 0; w < NW; ++w) Mt = fmaxf(Mt, sh.mt[w][h]);
          p.max_logits[pi] = Mt * kLn2;
          p.exp_sums[pi] = to_true_max(L, M, Mt);
        }
      }
    }
    __syncthreads();
  };

  // ---- the stream ------------------------------------------------------------
  Seg cur = make_seg(0, items[0], b_first, n_first, blo_first, bhi_first, piece_first,
                     whole_first, 0, 0);
  // the first segment's loads go out before the LDS walk to the next one
  Ids ids_cur = fetch_ids(cur);
  QOp q_cur[G::ksteps], q_nxt[G::ksteps];
  load_q(cur.b, items[0].h0, q_cur);
  // the appended row: loaded a segment ahead, encoded when its segment starts
  AR app_nxt{};
  AE app{};
  // encoded only by a segment that holds it (the encoding divides)
  auto take_app = [&](const AR &a) {
    if (a.blk >= 0) {
      app = encode_append(a, p.k_scale, p.v_scale_w);
      if constexpr (SUB) app.id = (a.id << p.sub_log2) + a.sub;  // pool sub-block id
    } else {
      app.blk = -1;
    }
  };
  if constexpr (APP) take_app(load_app(cur));
  Seg nxt = next_seg(cur);
  if constexpr (APP) app_nxt = load_app(nxt);
  St st[NS];
  load_scales(ids_cur, cur.g);
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(ids_cur, s, s < cur.kn, cur.g, st[s]);
  Ids ids_nxt = fetch_ids(nxt);
  load_q(nxt.valid ? nxt.b : cur.b, nxt.valid ? nxt.h0 : cur.h0, q_nxt);
  reset();
  for (;;) {
    // Units k = 0 .. kn-1 of the segment through NS register stages in turn:
    // while unit k is computed, the loads of units k+1 .. k+NS-1 are in
    // flight; indices from kpad on are the next segment's first units, which
    // land in the stages its own loop starts from. Every load instruction is
    // issued unconditionally (past the end they read nothing), so the
    // compiler's memory-counter waits stay exact: computing a unit waits only
    // for that unit.
    const int kn = cur.kn;
    const int kpad = max(NS, (kn + NS - 1) / NS * NS);
    const int g_cur = cur.g, g_nxt = nxt.valid ? nxt.g : cur.g;
    // the first head row of a KV head writes the appended token back
    const bool writer = appending && cur.h0 % p.group == 0;
    const int jb0 = cur.blo + (cur.w0 + cur.c * kIdsUnits * ND) * NBI;
    const int tok_lim = min(cur.bhi * kBs, cur.n);
    for (int k = 0; k < kpad - NS; k += NS) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int u = k + s + NS - 1;
        issue(ids_cur, u, u < kn, g_cur, st[(s + NS - 1) % NS]);
        if (k + s < kn) {
          compute_unit(jb0 + (k + s) * ND * NBI, tok_lim, q_cur, st[s], app, g_cur, writer,
                       ids_cur, k + s);
          pace();
        }
      }
    }
    // the last step, peeled: it issues this segment's last unit and the
    // next segment's first NS - 1 units (so that the ids of the next
    // segment are read only here, where their load is long done)
    load_scales(ids_nxt, g_nxt);
    {
      const int k = kpad - NS;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s == 0) issue(ids_cur, kpad - 1, kpad - 1 < kn, g_cur, st[NS - 1]);
        else issue(ids_nxt, s - 1, nxt.valid && s - 1 < nxt.kn, g_nxt, st[s - 1]);
        if (k + s < kn) {
          compute_unit(jb0 + (k + s) * ND * NBI, tok_lim, q_cur, st[s], app, g_cur, writer,
                       ids_cur, k + s);
          pace();
        }
      }
    }
    // move to the next segment (copies of loads issued a segment ago, made
    // before the epilogue's stores so that their waits do not cover the
    // next segment's loads already in flight)
    const Seg done = cur;
    cur = nxt;
    ids_cur = ids_nxt;
#pragma unroll
    for (int s = 0; s < G::ksteps; ++s) q_cur[s] = q_nxt[s];
    if (done.last) {
      epilogue(done.b, done.piece, done.whole, done.h0);
      reset();
    }
    if (!cur.valid) break;
    if constexpr (APP) take_app(app_nxt);
    nxt = next_seg(cur);
    if constexpr (APP) app_nxt = load_app(nxt);
    ids_nxt = fetch_ids(nxt);
    load_q(nxt.valid ? nxt.b : cur.b, nxt.valid ? nxt.h0 : cur.h0, q_nxt);
  }

}

template <int QT, int KT, int D, int GH, int NBI, int NS, int NW, bool APP, bool SUB, bool RW,
          bool SC>
__global__ __launch_bounds__(NW * kWave) void decode_kernel(const DecodeParams p) {
  __shared__ Shared<QT, KT, D, GH, NBI, NW> sh;
  const int tid = threadIdx.x;

  Item items[2];
  int n_items = 1;
  // the first range: blocks [first_lo, first_hi) of sequence first_b
  int first_b = 0, first_n = 0, first_lo = 0, first_hi = 0, first_piece = 0;
  bool first_whole = false;
  if (p.mode != kSplitBalanced) {
    // first query head of this workgroup (RW: of this wave, one head row per wave)
    // Fixed split on a one-dimensional grid: workgroup L runs on XCD L % 8;
    // of sequence b, XCD r takes the partitions with partition % 8 ==
    // (r + b) % 8, so that every XCD gets about an eighth of every
    // sequence's partitions whatever the length mix (with a grid indexed by
    // partition, XCD r would take every partition p % 8 == r, and the XCDs
    // of high partition numbers would idle on short sequences). Within a
    // sequence and head-row group, consecutive workgroups take consecutive
    // partitions.
    int part = blockIdx.x, row = blockIdx.y, b = blockIdx.z;
    if (p.swz_rows > 0) {
      const int L = blockIdx.x, r = L & 7, q = L >> 3;
      const int xqn = (p.max_partitions + 7) >> 3;
      const int t = q / xqn;
      row = t % p.swz_rows;
      b = t / p.swz_rows;
      part = 8 * (q % xqn) + ((r + b) & 7);
    }
    const int h0 = RW ? (row * NW + uniform(tid >> 6)) * GH : row * GH;
    const int n = p.context_lens[b];
    if (n <= 0) {
      if (p.mode == kSplitSingle)
        for (int i = RW ? (tid & (kWave - 1)) : tid; i < GH * D; i += (RW ? kWave : NW * kWave))
          store_elem<QT>(p.out, ((size_t)b * p.num_q_heads + h0) * D + i, 0.0f);
      return;
    }
    const int nblk = num_blocks_of(n);
    const int blo = part * p.partition_blocks;
    if (blo >= nblk) return;
    items[0] = Item{h0, h0 / p.group, 0, 0, 0};
    first_b = b;
    first_n = n;
    first_lo = blo;
    first_hi = min(nblk, blo + p.partition_blocks);
    first_piece = part;
    first_whole = nblk <= p.partition_blocks;
  } else {
    // Balanced split: the blocks of all sequences, end to end, cut into
    // num_splits equal shares. First the start block of every sequence
    // (exclusive prefix sum of ceil(n / 16)).
    const int B = p.num_seqs;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    {
      constexpr int PER = kMaxBalancedSeqs / (NW * kWave);
      int cnt[PER];
      int tot = 0;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int bb = PER * tid + k;
        const int n = bb < B ? p.context_lens[bb] : 0;
        if (bb < B) sh.ctx[bb] = n;
        cnt[k] = num_blocks_of(n);
        tot += cnt[k];
      }
      int incl = tot;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      if (lane == kWave - 1) sh.wave_sum[wave] = incl;
      __syncthreads();
      int base = 0, all = 0;
      for (int w = 0; w < NW; ++w) {
        const int ws = sh.wave_sum[w];
        if (w < wave) base += ws;
        all += ws;
      }
      // the first blocks of this workgroup's shares (see below), and the
      // sequences holding them: each thread checks its own sequences
      const int S = min(p.num_splits, all);
      const int s0 = RW ? blockIdx.x : 2 * blockIdx.x;
      const long long f0 = s0 < S ? (long long)s0 * all / S : -1;
      const long long f1 = !RW && s0 + 1 < S ? (long long)(s0 + 1) * all / S : -1;
      int ex = base + incl - tot;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int bb = PER * tid + k;
        if (bb < B) sh.start[bb] = ex;
        if (ex <= f0 && f0 < ex + cnt[k]) sh.first[0] = bb;
        if (ex <= f1 && f1 < ex + cnt[k]) sh.first[1] = bb;
        ex += cnt[k];
      }
      if (tid == (NW * kWave) - 1) sh.start[B] = base + incl;
      __syncthreads();
    }
    const int total = uniform(sh.start[B]);
    // at most one share per block, so that no share is empty
    const int S = min(p.num_splits, total);
    // Workgroup (x, y) takes share 2x of its own head row y and share 2x + 1
    // of the paired row y ^ 1 (the pair's other workgroup takes the other
    // two). The cache rows of neighbouring KV heads sit in different halves
    // of the memory interleave, which the hardware serves at different
    // rates; pairing gives every workgroup the same mix.
    if constexpr (RW) {
      // One wave per head row: workgroup (x, y) reads share x of head rows
      // NW y .. NW y + NW - 1, wave w taking row NW y + w, so every
      // workgroup reads whole cache blocks (all of their KV heads) and has
      // the same mix of heads.
      const int s = blockIdx.x;
      const int h0 = (blockIdx.y * NW + uniform(tid >> 6)) * GH;
      if (s >= S) return;
      items[0] = Item{h0, h0 / p.group, s, (int)((long long)s * total / S),
                      (int)((long long)(s + 1) * total / S)};
      items[1] = items[0];
      n_items = 1;
    } else {
    const int y = blockIdx.y;
    const int y2 = (y ^ 1) < (int)gridDim.y ? (y ^ 1) : y;
    const int s0 = 2 * blockIdx.x;
    if (s0 >= S) return;
    n_items = s0 + 1 < S ? 2 : 1;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int s = min(s0 + k, S - 1);
      const int h0 = (k == 0 ? y : y2) * GH;
      items[k] = Item{h0, h0 / p.group, s, (int)((long long)s * total / S),
                      (int)((long long)(s + 1) * total / S)};
    }
    }
    first_b = uniform(sh.first[0]);
    const int st = uniform(sh.start[first_b]), en = uniform(sh.start[first_b + 1]);
    first_n = uniform(sh.ctx[first_b]);
    first_lo = items[0].lo - st;
    first_hi = min(items[0].hi, en) - st;
    first_piece = items[0].share + first_b;
    first_whole = first_lo == 0 && first_hi == en - st;
  }
  run_ranges<QT, KT, D, GH, NBI, NS, NW, APP, SUB, RW, SC>(p, sh, items, n_items, first_b, first_n, first_lo, first_hi,
                                     first_piece, first_whole);
}

// ---------------------------------------------------------------------------
// kernel selection within a pair
// ---------------------------------------------------------------------------

template <int QT, int KT, int GH>
constexpr int units_of() {
  // blocks per unit: two for fp8 caches with up to 4 heads per workgroup
  // (64 bytes of K and V per lane per block), one otherwise -- two register
  // stages of one unit each stay within 256 VGPRs
  return (ElemBytes<KT>::value == 1 && GH <= 4) ? 2 : 1;
}


// Waves of a balanced-split workgroup: eight (one workgroup per compute
// unit: the hardware serves the workgroups of a compute unit unevenly, the
// waves of one workgroup alike) where two waves per SIMD fit the registers
// without spills, else four.
template <int QT, int KT, int D, int GH, bool APP>
constexpr int balanced_waves() {
  if (GH > 8) return 4;
  if (QT == PA_F32) return D == 64 ? 8 : 4;
  return 8;
}

// SUB: blocks larger than 16 tokens (read as 16-token sub-blocks); the
// 16-token kernels leave the sub-block arithmetic out. kind is a KernelKind:
// fixed partitions, whole sequences (single pass), balanced shares dealt to
// all waves of a workgroup, or balanced shares with one wave per head row
// (built where eight waves fit the registers; {nullptr, 0} otherwise).
template <int QT, int KT, int D, int GH, bool APP, bool SUB, bool SC>
KernelRef kernel_of(int kind) {
  constexpr int NBI = units_of<QT, KT, GH>();
  constexpr int NWB = balanced_waves<QT, KT, D, GH, APP>();
  if (kind == kKindRowWaves) {
    if constexpr (NWB == 8)
      return {reinterpret_cast<const void *>(
                  &decode_kernel<QT, KT, D, GH, NBI, kStages, 8, APP, SUB, true, SC>),
              8 * kWave};
    return {nullptr, 0};
  }
  if (kind == kKindShares)
    return {reinterpret_cast<const void *>(
                &decode_kernel<QT, KT, D, GH, NBI, kStages, NWB, APP, SUB, false, SC>),
            NWB * kWave};
  if (kind == kKindSingle)
    return {reinterpret_cast<const void *>(
                &decode_kernel<QT, KT, D, GH, NBI, kStages, kSingleWaves, APP, SUB, false, SC>),
            kSingleWaves * kWave};
  return {reinterpret_cast<const void *>(
              &decode_kernel<QT, KT, D, GH, NBI, kStages, kFixedWaves, APP, SUB, false, SC>),
          kFixedWaves * kWave};
}

// scaled: kernels for 8-bit caches with scale tables (built without append)
template <int QT, int KT, int D, int GH, bool SUB>
KernelRef with_append(int kind, bool append, bool scaled) {
  if (scaled) {
    if constexpr (ElemBytes<KT>::value == 1)
      if (!append) return kernel_of<QT, KT, D, GH, false, SUB, true>(kind);
    return {nullptr, 0};
  }
  return append ? kernel_of<QT, KT, D, GH, true, SUB, false>(kind)
                : kernel_of<QT, KT, D, GH, false, SUB, false>(kind);
}

template <int QT, int KT, int D, bool SUB>
KernelRef by_gh(int gh, int kind, bool append, bool scaled) {
  switch (gh) {
    case 1: return with_append<QT, KT, D, 1, SUB>(kind, append, scaled);
    case 2: return with_append<QT, KT, D, 2, SUB>(kind, append, scaled);
    case 4: return with_append<QT, KT, D, 4, SUB>(kind, append, scaled);
    case 8: return with_append<QT, KT, D, 8, SUB>(kind, append, scaled);
    case 16: return with_append<QT, KT, D, 16, SUB>(kind, append, scaled);
  }
  return {nullptr, 0};
}

template <int QT, int KT, bool SUB>
KernelRef by_d(int d, int gh, int kind, bool append, bool scaled) {
  switch (d) {
    case 64: return by_gh<QT, KT, 64, SUB>(gh, kind, append, scaled);
    case 128: return by_gh<QT, KT, 128, SUB>(gh, kind, append, scaled);
  }
  return {nullptr, 0};
}
}  // namespace

// The kernels of one element-type pair: the decode kernel for head size d,
// gh query heads per workgroup, a KernelKind, with append or not, with scale
// tables or not; {nullptr, 0} when not built. Each pair has one translation
// unit for 16-token blocks and one (_large) for larger blocks.
KernelRef decode_kernels_f32_f32(int d, int gh, int kind, bool append, bool scaled);
KernelRef decode_kernels_f16_f16(int d, int gh, int kind, bool append, bool scaled);
KernelRef decode_kernels_bf16_bf16(int d, int gh, int kind, bool append, bool scaled);
KernelRef decode_kernels_f16_fp8(int d, int gh, int kind, bool append, bool scaled);
KernelRef decode_kernels_bf16_fp8(int d, int gh, int kind, bool append, bool scaled);
KernelRef decode_kernels_f32_f32_large(int d, int gh, int kind, bool append, bool scaled);
KernelRef decode_kernels_f16_f16_large(int d, int gh, int kind, bool append, bool scaled);
KernelRef decode_kernels_bf16_bf16_large(int d, int gh, int kind, bool append, bool scaled);
KernelRef decode_kernels_f16_fp8_large(int d, int gh, int kind, bool append, bool scaled);
KernelRef decode_kernels_bf16_fp8_large(int d, int gh, int kind, bool append, bool scaled);
KernelRef decode_kernels_f16_int8(int d, int gh, int kind, bool append, bool scaled);
KernelRef decode_kernels_f16_int8_large(int d, int gh, int kind, bool append, bool scaled);
KernelRef decode_kernels_bf16_int8(int d, int gh, int kind, bool append, bool scaled);
KernelRef decode_kernels_bf16_int8_large(int d, int gh, int kind, bool append, bool scaled);

}  // namespace pa
