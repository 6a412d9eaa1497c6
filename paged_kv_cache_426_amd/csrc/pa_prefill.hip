// Paged prefill / chunked prefill attention for gfx950 (CDNA4, wave64).
//
// What is computed. Prefill processes a sequence's input tokens and builds
// their K/V; a long input may be cut into chunks scheduled beside decode
// work ("vLLM inference principles", section on the two phases of one
// generation). For sequence b with n = context_lens[b] cached tokens (the
// chunk's own K/V already written) and a chunk of C query tokens, query row
// i of the chunk sits at position n - C + i and attends causally over cache
// tokens 0 .. n - C + i: out = softmax(q K^T * scale) V ("KV-Cache
// evolution" section 1; query head h reads KV head h / group, section 3A),
// K/V gathered through the block table ("PagedAttention deep dive" section
// 2.1).
//
// Unlike decode, this is a dense contraction: a query tile of many rows
// reuses every K/V tile it loads, so it runs on MFMA.
//
// Work decomposition. A workgroup (4 waves) takes 128 query rows of one
// sequence and one KV head: TQ = 128 / GH consecutive chunk tokens times GH
// query heads of that KV head, rows in token-major order. It walks the keys
// 0 .. (position of its last row) in steps of 32 (two 16-token sub-blocks):
// each step's K and V are loaded once into LDS (double-buffered, the next
// step's global loads in flight while the current step is computed) and used
// by all four waves. Wave w owns rows 32 w .. 32 w + 31 as two 16-row column
// blocks c.
//
// Per step and wave, on 16x16x32 MFMAs with fp32 accumulation:
//   * S^T = K Q^T: A = 16 keys x 32 head elements from the LDS K tile (rows
//     padded by 16 bytes so the 16 rows of a read hit distinct banks), B =
//     the wave's query fragments (registers, loaded once). The result lands
//     with lane l holding query row l % 16 and keys 4 (l / 16) + 0..3 of each
//     16-key tile.
//   * causal mask (select, never a product), online softmax in the exp2
//     domain (running max per row; row reductions across the four lane
//     groups), probabilities rounded to the query's 16-bit type;
//   * O^T += V^T P^T: A = V^T from an LDS tile stored transposed, B = the
//     lane's own eight probabilities -- the MFMA's k index 8 j + e stands for
//     key 4 j + e (e < 4) or 16 + 4 j + e - 4, and V^T is read with the same
//     key order -- so the probabilities never leave registers.
// Rows past the chunk's end are computed on zero queries and not written.
// Keys past the last row's position are masked in S and zeroed in V (stale
// or NaN cache contents never reach the result).

#include <hip/hip_runtime.h>
#include <type_traits>
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPrefillWaves = 4;
constexpr int kPrefillRows = 128;  // query rows (token, head) per workgroup
constexpr int kPrefillKeys = 32;   // keys per step: two 16-token sub-blocks
constexpr float kLog2eP = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct PrefillParams {
  void *out;
  const uint8_t *q;
  const uint8_t *k_cache;
  const uint8_t *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  const int32_t *query_start;
  int num_q_heads;
  int num_kv_heads;
  int max_blocks_per_seq;
  int sub_log2;     // log2(block_size / 16)
  int group;        // query heads per KV head
  int ntiles;       // query tiles per sequence
  int rows_per_seq; // workgroups per sequence and query tile: KV heads x head subgroups
  int num_seqs;
  float scale_log2; // scale * k_scale * log2(e)
  float v_scale;
};

// 8 cache elements (a 16-byte or 8-byte piece) widened exactly to the
// query's 16-bit type, as 4 words.
template <int QT, int KT>
__device__ __forceinline__ u32x4 widen8(const u32x4 &w) {
  if constexpr (ElemBytes<KT>::value == 2) {
    return w;
  } else if constexpr (KT == PA_FP8_E4M3FN) {
    u32x4 r;
    if constexpr (QT == PA_BF16) {
      r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false));
      r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true));
      r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false));
      r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true));
    } else {
      r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, false));
      r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, true));
      r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, false));
      r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, true));
    }
    return r;
  } else {
    // int8 codes are integers of at most 8 significant bits: exact in both
    // 16-bit types
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t src = i < 2 ? w.x : w.y;
      const int sh = (i % 2) * 16;
      const float f0 = (float)((int32_t)(src << (24 - sh)) >> 24);
      const float f1 = (float)((int32_t)(src << (16 - sh)) >> 24);
      if constexpr (QT == PA_BF16)
        o[i] = (f2u(f0) >> 16) | (f2u(f1) & 0xffff0000u);
      else
        o[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f0, f1));
    }
    return u32x4{o[0], o[1], o[2], o[3]};
  }
}

template <int QT>
__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (QT == PA_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// two fp32 values rounded (nearest even) to the query's 16-bit type, packed
template <int QT>
__device__ __forceinline__ uint32_t pack16(float a, float b) {
  if constexpr (QT == PA_BF16) {
    const bf16x2 h = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, h);
  } else {
    const f16x2 h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
  }
}

// four fp32 results rounded (nearest even) to the 16-bit output type
template <int QT>
__device__ __forceinline__ void store4(void *out, size_t idx, const float (&x)[4]) {
  *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(out) + idx) =
      u32x2{pack16<QT>(x[0], x[1]), pack16<QT>(x[2], x[3])};
}

constexpr int kRsrcFlagsP = 0x00020000;  // gfx9 word 3: 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint8_t *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), (short)0, (int)bytes,
                                           kRsrcFlagsP);
}

// 8 cache elements at byte offset off of a sub-block resource
template <int KT>
__device__ __forceinline__ u32x4 load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (ElemBytes<KT>::value == 2) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  } else {
    const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return u32x4{a.x, a.y, 0u, 0u};
  }
}

template <int QT, int KT, int D, int GH>
// three waves per SIMD (168 VGPRs; the few values the compiler then keeps in
// scratch are read only on the rare paths: a new block-id batch, a moving
// softmax maximum, the last step)
__global__ __launch_bounds__(kPrefillWaves * kWave) __attribute__((amdgpu_waves_per_eu(3)))
void prefill_kernel(const PrefillParams p) {
  constexpr int TQ = kPrefillRows / GH;       // chunk tokens per workgroup
  constexpr int KB = ElemBytes<KT>::value;    // cache element bytes
  constexpr int KRS = D * 2 + 16;             // LDS row stride of the K tile (16-bit)
  // V^T tile in LDS: row d (element) holds the step's 32 keys, 16-bit, in a
  // row of 18 dwords; key pair c (keys 2c, 2c + 1) sits at dword c ^ vsw(d),
  // vsw(d) = 8 ((d / 16) & 1). With this stride the 16 rows a half-wave
  // reads (8 bytes each, same columns) fall in distinct banks, and with the
  // swizzle the 32 words a half-wave writes (8 key pairs of 4 element
  // groups, see vkp and vdg) do too.
  constexpr int VRS = kPrefillKeys * 2 + 8;
  constexpr int NST = D / 32;                 // MFMA k-steps over the head dimension
  constexpr int NDT = D / 16;                 // 16-column tiles of the output
  constexpr int DG = D / 8;                   // 8-element pieces of a row
  constexpr int KPIECES = kPrefillKeys * DG / (kPrefillWaves * kWave);  // K pieces per thread
  static_assert(KPIECES >= 1, "unsupported head size");
  __shared__ __attribute__((aligned(16))) uint8_t ksm[2][kPrefillKeys * KRS];
  __shared__ __attribute__((aligned(16))) uint8_t vsm[2][D * VRS];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jq = lane >> 4;  // MFMA lane group
  const int tl = lane & 15;

  // Work index: the launch is one-dimensional, and workgroup x runs on XCD
  // x % 8 (the dispatcher deals workgroups to the XCDs in turn). Work item w
  // goes to x = 8 (w % per) + w / per, so consecutive work items share an
  // XCD; the query tiles of one (sequence, KV head) are consecutive, so they
  // run together on one XCD and re-read their K/V from its L2. Within a
  // (sequence, KV head) the heaviest tiles (latest in the chunk: most keys)
  // come first.
  const int total = p.ntiles * p.rows_per_seq * p.num_seqs;
  const int per = (total + 7) / 8;
  const int w = ((int)blockIdx.x % 8) * per + (int)blockIdx.x / 8;
  if (w >= total) return;
  const int tile = p.ntiles - 1 - w % p.ntiles;
  const int hg = (w / p.ntiles) % p.rows_per_seq;  // (KV head, head subgroup)
  const int b = w / p.ntiles / p.rows_per_seq;
  const int subgroups = p.group / GH;
  const int g = hg / subgroups;
  const int hbase = g * p.group + (hg % subgroups) * GH;
  const int n = p.context_lens[b];
  const int q0 = p.query_start[b];
  const int C = p.query_start[b + 1] - q0;
  const int tok0 = tile * TQ;
  if (tok0 >= C) return;
  const int tokn = min(TQ, C - tok0);
  const int pos0 = n - C + tok0;             // position of the tile's first token
  const int plast = pos0 + tokn - 1;         // position of its last token
  const int nsteps = (plast + kPrefillKeys) / kPrefillKeys;

  // ---- the wave's query rows (two column blocks of 16) ---------------------
  u32x4 qf[2][NST];
  int pos[2];
  bool rowok[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = wave * 32 + c * 16 + tl;
    const int t = r / GH, hh = r % GH;
    rowok[c] = t < tokn;
    pos[c] = pos0 + t;
    const uint8_t *qrow =
        p.q + ((size_t)(q0 + tok0 + (rowok[c] ? t : 0)) * p.num_q_heads + hbase + hh) * D * 2;
#pragma unroll
    for (int s = 0; s < NST; ++s) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(qrow + (32 * s + 8 * jq) * 2);
      qf[c][s] = rowok[c] ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // ---- K/V tile loads --------------------------------------------------------
  const uint32_t rowstride = (uint32_t)p.num_kv_heads * D * KB;  // bytes per token row
  const uint32_t blk_bytes = rowstride * 16;
  const uint32_t span = blk_bytes - (uint32_t)g * D * KB;         // head g's rows to the block end
  // The block-table row, read with vector loads: a scalar load would share
  // its wait counter with the LDS reads of the steps and stall them for a
  // memory round trip.
  const __amdgpu_buffer_rsrc_t trow = rsrc(
      reinterpret_cast<const uint8_t *>(p.block_tables + (size_t)b * p.max_blocks_per_seq),
      (uint32_t)p.max_blocks_per_seq * 4u);
  const int smask = (1 << p.sub_log2) - 1;
  // Physical 16-token sub-block ids, 64 per register: lane i of chunk c
  // holds sub-block 64 c + i (0 past the last one the tile reads; its loads
  // are then of nothing). The next chunk is loaded a chunk (32 steps) ahead,
  // and a step takes its two ids with readlane.
  auto load_chunk = [&](int c) {
    const int j = 64 * c + lane;
    const bool in = j * 16 <= plast;
    const int e = (int)__builtin_amdgcn_raw_buffer_load_b32(
        trow, (uint32_t)(in ? (j >> p.sub_log2) : 0) * 4u, 0, 0);
    return in ? (e << p.sub_log2) + (j & smask) : 0;
  };
  int ch_idx = 0;
  int ch_cur = load_chunk(0);
  int ch_nxt = load_chunk(1);
  auto ids_of = [&](int s, int &id0, int &id1) {  // sub-blocks 2 s and 2 s + 1
    const int j0 = 2 * s;
    const bool next = (j0 >> 6) != ch_idx;
    if (next) {
      ch_cur = ch_nxt;
      ++ch_idx;
    }
    id0 = __builtin_amdgcn_readlane(ch_cur, j0 & 63);
    id1 = __builtin_amdgcn_readlane(ch_cur, (j0 + 1) & 63);
    // the following chunk's load goes out after the ids are taken, so that
    // nothing waits for it
    if (next) ch_nxt = load_chunk(ch_idx + 1);
  };
  auto sub_rsrc = [&](const uint8_t *cache, int j, int id) {
    const uint32_t bytes = j * 16 <= plast ? span : 0u;
    return rsrc(cache + (size_t)id * blk_bytes + (size_t)g * D * KB, bytes);
  };
  // thread roles: K pieces (key, 8-element group); V key pairs (2 keys, 8 elements)
  u32x4 kreg[KPIECES];
  u32x4 vreg[2];
  // V: key pair and element group. Wave w takes the key pairs of half w % 2
  // of the step (8 pairs, fastest over the lanes) and element groups
  // 8 (w / 2) .. 8 (w / 2) + 7.
  const int vkp = 8 * (wave & 1) + (lane & 7);
  const int vdg = 8 * (wave >> 1) + (lane >> 3);
  // (every thread has a V role when the element groups fill the waves)
  const bool vrole = (DG * kPrefillKeys / 2 == kPrefillWaves * kWave) || vdg < DG;
  // The keys a wave loads lie in one 16-key half of the step (64 lanes cover
  // 4 or 8 consecutive keys of K, 8 or 16 of V, aligned), so each load's
  // buffer resource is wave-uniform (a per-lane resource would make the
  // compiler loop over the distinct values).
  auto issue = [&](int s) {
    int id0, id1;
    ids_of(s, id0, id1);
#pragma unroll
    for (int i = 0; i < KPIECES; ++i) {
      const int pc = tid + i * kPrefillWaves * kWave;
      const int key = pc / DG, dg = pc % DG;
      const int half = __builtin_amdgcn_readfirstlane(key / 16);
      const __amdgpu_buffer_rsrc_t r = sub_rsrc(p.k_cache, 2 * s + half, half ? id1 : id0);
      kreg[i] = load8<KT>(r, (uint32_t)(key % 16) * rowstride + dg * 8 * KB);
    }
    if (vrole) {
      const int key = 2 * vkp;
      const int half = __builtin_amdgcn_readfirstlane(key / 16);
      const __amdgpu_buffer_rsrc_t r = sub_rsrc(p.v_cache, 2 * s + half, half ? id1 : id0);
      const uint32_t off = (uint32_t)(key % 16) * rowstride + vdg * 8 * KB;
      vreg[0] = load8<KT>(r, off);
      vreg[1] = load8<KT>(r, off + rowstride);
    }
  };
  // registers -> LDS buffer bf: K rows as they are, V transposed; keys past
  // the last position are zeroed in V
  auto stash = [&](int s, int bf) {
#pragma unroll
    for (int i = 0; i < KPIECES; ++i) {
      const int pc = tid + i * kPrefillWaves * kWave;
      const int key = pc / DG, dg = pc % DG;
      *reinterpret_cast<u32x4 *>(&ksm[bf][key * KRS + dg * 16]) = widen8<QT, KT>(kreg[i]);
    }
    if (vrole) {
      const int key = 2 * vkp;
      const u32x4 a = widen8<QT, KT>(vreg[0]);
      const u32x4 c = widen8<QT, KT>(vreg[1]);
      uint32_t aw[4] = {a.x, a.y, a.z, a.w};
      uint32_t cw[4] = {c.x, c.y, c.z, c.w};
      // only a step that reaches past the last position has keys to zero
      if (kPrefillKeys * s + kPrefillKeys - 1 > plast) {
        const bool ok0 = kPrefillKeys * s + key <= plast;
        const bool ok1 = kPrefillKeys * s + key + 1 <= plast;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          aw[e] = ok0 ? aw[e] : 0u;
          cw[e] = ok1 ? cw[e] : 0u;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // element e of both keys, side by side (low half: the even key)
        const uint32_t sel = (e % 2) ? 0x07060302u : 0x05040100u;
        const uint32_t w = __builtin_amdgcn_perm(cw[e / 2], aw[e / 2], sel);
        const int d = vdg * 8 + e;
        *reinterpret_cast<uint32_t *>(&vsm[bf][d * VRS + 4 * (vkp ^ (8 * ((d >> 4) & 1)))]) = w;
      }
    }
  };

  // ---- online softmax state and accumulators ---------------------------------
  float m[2] = {-INFINITY, -INFINITY};
  float l[2] = {0.0f, 0.0f};  // per-lane partial sums
  f32x4 o[2][NDT];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[c][dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const float sl2 = p.scale_log2;
  const bool pos_scale = sl2 > 0.0f;

  // Step s + 1's K/V are stored to LDS at the end of step s, between its
  // P.V MFMAs (the other buffer was last read in step s - 1, which every
  // wave has finished at step s's barrier), and its loads go out right
  // after that barrier. Past the last step both load nothing (zero-length
  // buffer ranges) and store zeros to the unused buffer, so the step has no
  // branches around them.
  issue(0);
  stash(0, 0);
  for (int s = 0; s < nsteps; ++s) {
    const int bf = s & 1;
    __syncthreads();
    issue(s + 1);
    const int k0 = kPrefillKeys * s;
    // S^T = K Q^T for both 16-key tiles and both column blocks: the four
    // accumulators' chains are interleaved, k step by k step, so that
    // consecutive MFMAs never depend on each other (two chains at a time,
    // tile after tile, measured 3 % slower over the whole kernel)
    f32x4 st[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int c = 0; c < 2; ++c) st[kt][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ss = 0; ss < NST; ++ss) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const u32x4 a =
            *reinterpret_cast<const u32x4 *>(&ksm[bf][(kt * 16 + tl) * KRS + (32 * ss + 8 * jq) * 2]);
#pragma unroll
        for (int c = 0; c < 2; ++c) st[kt][c] = mfma32<QT>(a, qf[c][ss], st[kt][c]);
      }
    }
    // Online softmax of both column blocks. Each row keeps a reference
    // maximum m and the probabilities are exp2(s - m); m moves (and the
    // row's sum and accumulators are rescaled) only when the row's maximum
    // exceeds it by more than 8 (a factor 256), so probabilities stay below
    // 256 and the rescale of the 64 accumulators is rare. The result is the
    // same softmax (every term of a row carries the same factor 2^-m). Keys
    // past a row's position are masked only in steps that reach past the
    // tile's first row.
    const bool diag = k0 + kPrefillKeys - 1 > pos0;
    // V^T operand of output tile dt (rows d = 16 dt + tl; keys 4 jq .. +3
    // and 16 + 4 jq .. +3, in that order in even tiles and swapped in odd
    // ones, whose rows store the two key halves the other way round), read
    // one tile ahead of the P.V MFMAs that use it: holding the whole step's
    // operands (32 VGPRs) would keep the kernel at two waves per SIMD; read
    // per tile it fits three (168 VGPRs), whose waves cover each other's LDS
    // and softmax latency (about 2.5 % faster)
    auto va_of = [&](int dt) {
      const uint8_t *vr = &vsm[bf][(16 * dt + tl) * VRS] + 8 * jq;
      const u32x2 a = *reinterpret_cast<const u32x2 *>(vr);
      const u32x2 b = *reinterpret_cast<const u32x2 *>(vr + 32);
      return u32x4{a.x, a.y, b.x, b.y};
    };
    u32x4 pb[2];
    float alpha[2] = {1.0f, 1.0f};
    float sv[2][8];
    float lm[2];  // this lane's largest scaled logit of the step, per block
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const f32x4 x = st[kt][c];
        sv[c][4 * kt + 0] = x.x;
        sv[c][4 * kt + 1] = x.y;
        sv[c][4 * kt + 2] = x.z;
        sv[c][4 * kt + 3] = x.w;
      }
    // key i of block c is visible to the block's row (always, in a step
    // without the mask: those steps carry no mask arithmetic): its position
    // k0 + 4 jq + 16 (i / 4) + i % 4 is at most the row's, i.e. the
    // constant 16 (i / 4) + i % 4 is at most pos[c] - k0 - 4 jq
    auto visible = [&](auto mask_tag, int c, int i) {
      if constexpr (!decltype(mask_tag)::value) return true;
      else return 16 * (i / 4) + i % 4 <= pos[c] - k0 - 4 * jq;
    };
    auto lane_max = [&](auto mask_tag) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        // the largest scaled logit: the largest raw logit times a positive
        // scale, the smallest times a negative or zero one; masked keys never win
        float e;
        if (pos_scale) {
          e = -INFINITY;
#pragma unroll
          for (int i = 0; i < 8; ++i) e = fmaxf(e, visible(mask_tag, c, i) ? sv[c][i] : -INFINITY);
        } else {
          e = INFINITY;
#pragma unroll
          for (int i = 0; i < 8; ++i) e = fminf(e, visible(mask_tag, c, i) ? sv[c][i] : INFINITY);
        }
        lm[c] = __builtin_isinf(e) ? -INFINITY : e * sl2;
      }
    };
    if (diag) lane_max(std::true_type{});
    else lane_max(std::false_type{});
    // A row's reference maximum m moves only when the row's maximum exceeds
    // it by more than 8: unless some lane's own maximum does, no row moves
    // and the row reductions are skipped (the usual case once every row has
    // seen its first keys).
    const bool any_up = __builtin_amdgcn_ballot_w64(lm[0] > m[0] + 8.0f || lm[1] > m[1] + 8.0f) != 0;
    if (any_up) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float mx = lm[c];
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool up = mx > m[c] + 8.0f;
        const float mn = up ? mx : m[c];
        alpha[c] = up ? __builtin_amdgcn_exp2f(m[c] - mn) : 1.0f;
        m[c] = mn;
        l[c] *= alpha[c];
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[c][dt] *= alpha[c];
    }
    auto probs = [&](auto mask_tag) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        // a row that has seen no key yet keeps m = -inf and gets no weight
        const float mref = m[c] == -INFINITY ? 0.0f : m[c];
        float sum = 0.0f;
        float pr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sv[c][i], sl2, -mref));
          pr[i] = visible(mask_tag, c, i) ? e : 0.0f;
          sum += pr[i];
        }
        l[c] += sum;
        pb[c] = u32x4{pack16<QT>(pr[0], pr[1]), pack16<QT>(pr[2], pr[3]),
                      pack16<QT>(pr[4], pr[5]), pack16<QT>(pr[6], pr[7])};
      }
    };
    if (diag) probs(std::true_type{});
    else probs(std::false_type{});
    // O^T += V^T P^T per 16 output columns, interleaved with the store of
    // step s + 1's K/V. Odd tiles take the probabilities with their two key
    // halves swapped (the same k permutation on both operands leaves the
    // product as it is), so the V operand is used as read, with no register
    // moves between the read and the MFMA (with the read one tile ahead:
    // 955.7 -> 929.8 us).
    u32x4 pbs[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) pbs[c] = u32x4{pb[c].z, pb[c].w, pb[c].x, pb[c].y};
    u32x4 vn = va_of(0);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const u32x4 vc = vn;
      if (dt + 1 < NDT) vn = va_of(dt + 1);
#pragma unroll
      for (int c = 0; c < 2; ++c) o[c][dt] = mfma32<QT>(vc, (dt & 1) ? pbs[c] : pb[c], o[c][dt]);
    }
    stash(s + 1, bf ^ 1);
#pragma unroll
    for (int i = 0; i < 2 * NDT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x006, 2, 0);  // two vector-ALU
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // one LDS write
    }
  }

  // ---- normalise and write: lane holds row (c, tl), elements 16 dt + 4 jq + 0..3
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    float lt = l[c];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (!rowok[c]) continue;
    const int r = wave * 32 + c * 16 + tl;
    const int t = r / GH, hh = r % GH;
    const float inv = p.v_scale / lt;
    const size_t base = ((size_t)(q0 + tok0 + t) * p.num_q_heads + hbase + hh) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const float x[4] = {o[c][dt].x * inv, o[c][dt].y * inv, o[c][dt].z * inv,
                          o[c][dt].w * inv};
      store4<QT>(p.out, base + 16 * dt + 4 * jq, x);
    }
  }
}

// query heads per workgroup: the largest of 8, 4, 2, 1 dividing the group
int prefill_heads(int group) {
  return group % 8 == 0 ? 8 : group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
}

template <int QT, int KT, int D>
const void *prefill_by_gh(int gh) {
  switch (gh) {
    case 1: return reinterpret_cast<const void *>(&prefill_kernel<QT, KT, D, 1>);
    case 2: return reinterpret_cast<const void *>(&prefill_kernel<QT, KT, D, 2>);
    case 4: return reinterpret_cast<const void *>(&prefill_kernel<QT, KT, D, 4>);
    case 8: return reinterpret_cast<const void *>(&prefill_kernel<QT, KT, D, 8>);
  }
  return nullptr;
}

template <int QT, int KT>
const void *prefill_by_d(int d, int gh) {
  return d == 64 ? prefill_by_gh<QT, KT, 64>(gh) : d == 128 ? prefill_by_gh<QT, KT, 128>(gh)
                                                            : nullptr;
}

const void *prefill_kernel_for(int q_dtype, int kv_dtype, int d, int gh) {
  if (q_dtype == PA_BF16) {
    if (kv_dtype == PA_BF16) return prefill_by_d<PA_BF16, PA_BF16>(d, gh);
    if (kv_dtype == PA_FP8_E4M3FN) return prefill_by_d<PA_BF16, PA_FP8_E4M3FN>(d, gh);
    if (kv_dtype == PA_INT8) return prefill_by_d<PA_BF16, PA_INT8>(d, gh);
  } else if (q_dtype == PA_F16) {
    if (kv_dtype == PA_F16) return prefill_by_d<PA_F16, PA_F16>(d, gh);
    if (kv_dtype == PA_FP8_E4M3FN) return prefill_by_d<PA_F16, PA_FP8_E4M3FN>(d, gh);
    if (kv_dtype == PA_INT8) return prefill_by_d<PA_F16, PA_INT8>(d, gh);
  }
  return nullptr;
}

}  // namespace

int prefill_tokens_per_tile(int group) { return kPrefillRows / prefill_heads(group); }

int launch_prefill(const PrefillLaunch &a, void *stream) {
  PrefillParams p;
  p.out = a.out;
  p.q = static_cast<const uint8_t *>(a.q);
  p.k_cache = static_cast<const uint8_t *>(a.k_cache);
  p.v_cache = static_cast<const uint8_t *>(a.v_cache);
  p.block_tables = a.block_tables;
  p.context_lens = a.context_lens;
  p.query_start = a.query_start;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.max_blocks_per_seq = a.max_blocks_per_seq;
  p.sub_log2 = sub_block_log2(a.block_size);
  if (p.sub_log2 < 0) return (int)hipErrorInvalidValue;
  p.group = a.num_q_heads / a.num_kv_heads;
  const bool q8 = a.kv_dtype == PA_FP8_E4M3FN || a.kv_dtype == PA_INT8;
  p.scale_log2 = a.scale * (q8 ? a.k_scale : 1.0f) * kLog2eP;
  p.v_scale = q8 ? a.v_scale : 1.0f;
  const int gh = prefill_heads(p.group);
  const int tq = kPrefillRows / gh;
  p.ntiles = (a.max_query_len + tq - 1) / tq;
  const void *fn = prefill_kernel_for(a.q_dtype, a.kv_dtype, a.head_dim, gh);
  if (!fn) return (int)hipErrorInvalidValue;
  if (p.ntiles == 0) return 0;
  p.rows_per_seq = a.num_kv_heads * (p.group / gh);
  p.num_seqs = a.num_seqs;
  const long long total = (long long)p.ntiles * p.rows_per_seq * a.num_seqs;
  if (total > (1ll << 30)) return (int)hipErrorInvalidValue;
  const dim3 grid((unsigned)(8 * ((total + 7) / 8)));
  void *args[] = {&p};
  hipError_t e = hipLaunchKernel(fn, grid, dim3(kPrefillWaves * kWave), args, 0,
                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return (int)e;
  return (int)hipGetLastError();
}

}  // namespace pa
