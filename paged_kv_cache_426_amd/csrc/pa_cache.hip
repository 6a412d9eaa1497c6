// Cache-writing kernels for gfx950: the slot write of new tokens' K/V rows
// and the copy-on-write block copy.
//
// Slot write: a sequence's newest K/V rows are stored in the slot its host
// block manager assigned -- the current block until it is full, then a fresh
// one ("PagedAttention deep dive" §2.2; "vLLM inference principles", two
// phases: decode extends the cache). With the cache laid out as
// [num_blocks, block_size, Hkv, d], slot s = block * block_size + offset is
// simply row s of a [num_blocks * block_size, Hkv * d] matrix, so one token
// is one contiguous row copy (or quantisation) of Hkv * d elements.
//
// Block copy: a block shared by several sequences is copied before one of
// them writes a different token into it ("PagedAttention deep dive" §2.3;
// "KV-cache sharing article" §3.1). One workgroup copies one block of one
// cache with 16-byte loads and stores.

#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kCopyThreads = 256;

// Scale tables of an 8-bit cache: the scale of (physical block e, KV head
// g) is k[e * block_stride + g * head_stride]; k == nullptr selects the
// per-tensor scales.
struct RcTables {
  const float *k, *v;
  int block_stride, head_stride, block_size, head_dim;
};

// One workgroup per token; each thread moves 16 source bytes per step.
template <int ST, int CT>
__global__ __launch_bounds__(kCopyThreads) void reshape_and_cache_kernel(
    const uint8_t *key, const uint8_t *value, uint8_t *k_cache, uint8_t *v_cache,
    const int64_t *slot_mapping, int row_elems, float k_scale, float v_scale, RcTables tab) {
  constexpr int SB = ElemBytes<ST>::value;
  constexpr int CB = ElemBytes<CT>::value;
  constexpr int VEC = 16 / SB;  // source elements per 16-byte piece
  const int t = blockIdx.x;
  const bool is_v = blockIdx.y == 1;
  const uint8_t *src = (is_v ? value : key) + (size_t)t * row_elems * SB;
  const int pieces = row_elems / VEC;
  if constexpr (ST == CT) {
    // the first piece of the row is loaded together with the slot (one
    // memory round trip instead of two for rows of up to 4 KiB)
    const int i0 = threadIdx.x;
    u32x4 first = {0u, 0u, 0u, 0u};
    if (i0 < pieces) first = reinterpret_cast<const u32x4 *>(src)[i0];
    const int64_t slot = slot_mapping[t];
    if (slot < 0) return;
    uint8_t *dst = (is_v ? v_cache : k_cache) + (size_t)slot * row_elems * CB;
    if (i0 < pieces) reinterpret_cast<u32x4 *>(dst)[i0] = first;
    for (int i = i0 + kCopyThreads; i < pieces; i += kCopyThreads)
      reinterpret_cast<u32x4 *>(dst)[i] = reinterpret_cast<const u32x4 *>(src)[i];
  } else {
    const int64_t slot = slot_mapping[t];
    if (slot < 0) return;
    uint8_t *dst = (is_v ? v_cache : k_cache) + (size_t)slot * row_elems * CB;
    static_assert(CT == PA_FP8_E4M3FN || CT == PA_INT8, "only 8-bit caches convert");
    auto enc = [](float v) { return CT == PA_INT8 ? f32_to_int8(v) : f32_to_e4m3fn(v); };
    const float *table = is_v ? tab.v : tab.k;
    const float tensor_scale = is_v ? v_scale : k_scale;
    // with a table: the scales of this slot's block (a piece never spans two
    // heads: head rows are whole 16-byte pieces of the source, checked on
    // the host)
    const float *row_scales =
        table ? table + (size_t)(slot / tab.block_size) * tab.block_stride : nullptr;
    for (int i = threadIdx.x; i < pieces; i += kCopyThreads) {
      const float scale =
          row_scales ? row_scales[(size_t)(i * VEC / tab.head_dim) * tab.head_stride]
                     : tensor_scale;
      const u32x4 w = reinterpret_cast<const u32x4 *>(src)[i];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
      float x[VEC];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (ST == PA_F32) {
          x[k] = u2f(ws[k]);
        } else if constexpr (ST == PA_BF16) {
          x[2 * k] = bf16_lo(ws[k]);
          x[2 * k + 1] = bf16_hi(ws[k]);
        } else {
          x[2 * k] = f16_lo(ws[k]);
          x[2 * k + 1] = f16_hi(ws[k]);
        }
      }
      uint32_t packed[VEC / 4];
#pragma unroll
      for (int k = 0; k < VEC / 4; ++k) {
        // correctly rounded float32 division (the library is built with
        // -fhip-fp32-correctly-rounded-divide-sqrt and without fast-math)
        packed[k] = enc(x[4 * k] / scale) | (enc(x[4 * k + 1] / scale) << 8) |
                    (enc(x[4 * k + 2] / scale) << 16) | (enc(x[4 * k + 3] / scale) << 24);
      }
      if constexpr (VEC == 8) {
        reinterpret_cast<uint2 *>(dst)[i] = make_uint2(packed[0], packed[1]);
      } else {
        reinterpret_cast<uint32_t *>(dst)[i] = packed[0];
      }
    }
  }
}

// One workgroup per (pair, cache). With per-block scale tables (entries
// scales per block: one, or one per KV head) the block's scales move with
// it: a block's codes mean nothing without them.
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(uint8_t *k_cache,
                                                                   uint8_t *v_cache,
                                                                   const int64_t *block_mapping,
                                                                   size_t block_bytes,
                                                                   float *k_scales,
                                                                   float *v_scales, int entries) {
  const int64_t src = block_mapping[2 * (size_t)blockIdx.x];
  const int64_t dst = block_mapping[2 * (size_t)blockIdx.x + 1];
  uint8_t *base = blockIdx.y == 0 ? k_cache : v_cache;
  const u32x4 *s = reinterpret_cast<const u32x4 *>(base + (size_t)src * block_bytes);
  u32x4 *d = reinterpret_cast<u32x4 *>(base + (size_t)dst * block_bytes);
  const size_t pieces = block_bytes / 16;
  for (size_t i = threadIdx.x; i < pieces; i += kCopyThreads) d[i] = s[i];
  float *tab = blockIdx.y == 0 ? k_scales : v_scales;
  for (int i = threadIdx.x; i < entries; i += kCopyThreads)
    tab[(size_t)dst * entries + i] = tab[(size_t)src * entries + i];
}

template <int ST, int CT>
hipError_t launch_rc(const void *key, const void *value, void *k_cache, void *v_cache,
                     const int64_t *slots, int num_tokens, int row_elems, float ks, float vs,
                     const RcTables &tab, hipStream_t s) {
  hipLaunchKernelGGL((reshape_and_cache_kernel<ST, CT>), dim3(num_tokens, 2),
                     dim3(kCopyThreads), 0, s, static_cast<const uint8_t *>(key),
                     static_cast<const uint8_t *>(value), static_cast<uint8_t *>(k_cache),
                     static_cast<uint8_t *>(v_cache), slots, row_elems, ks, vs, tab);
  return hipGetLastError();
}

}  // namespace

int launch_reshape_and_cache(const void *key, const void *value, void *k_cache, void *v_cache,
                             const int64_t *slot_mapping, int num_tokens, int num_kv_heads,
                             int head_dim, int src_dtype, int cache_dtype, float k_scale,
                             float v_scale, const ScaleTables &tables, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int row = num_kv_heads * head_dim;
  const RcTables tab{tables.k, tables.v, tables.block_stride, tables.head_stride,
                     tables.block_size, head_dim};
  hipError_t e = hipErrorInvalidValue;
#define PA_RC(ST, CT)                                                                     \
  if (src_dtype == ST && cache_dtype == CT)                                               \
    e = launch_rc<ST, CT>(key, value, k_cache, v_cache, slot_mapping, num_tokens, row,    \
                          k_scale, v_scale, tab, s);
  PA_RC(PA_F32, PA_F32)
  PA_RC(PA_F16, PA_F16)
  PA_RC(PA_BF16, PA_BF16)
  PA_RC(PA_F32, PA_FP8_E4M3FN)
  PA_RC(PA_F16, PA_FP8_E4M3FN)
  PA_RC(PA_BF16, PA_FP8_E4M3FN)
  PA_RC(PA_F32, PA_INT8)
  PA_RC(PA_F16, PA_INT8)
  PA_RC(PA_BF16, PA_INT8)
#undef PA_RC
  return (int)e;
}

int launch_copy_blocks(void *k_cache, void *v_cache, const int64_t *block_mapping, int num_pairs,
                       size_t block_bytes, float *k_scales, float *v_scales, int entries,
                       void *stream) {
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, 2), dim3(kCopyThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint8_t *>(k_cache),
                     static_cast<uint8_t *>(v_cache), block_mapping, block_bytes, k_scales,
                     v_scales, entries);
  return (int)hipGetLastError();
}

}  // namespace pa
