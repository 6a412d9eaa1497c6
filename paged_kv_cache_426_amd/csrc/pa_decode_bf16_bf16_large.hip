// Decode kernels for bfloat16 queries and bfloat16 caches, cache blocks of 32 to 256 tokens.

#include "pa_decode_kernel.h"

namespace pa {

KernelRef decode_kernels_bf16_bf16_large(int d, int gh, int kind, bool append, bool scaled) {
  return by_d<PA_BF16, PA_BF16, true>(d, gh, kind, append, scaled);
}

}  // namespace pa
