// Decode kernels for float32 queries and float32 caches, cache blocks of 32 to 256 tokens.

#include "pa_decode_kernel.h"

namespace pa {

KernelRef decode_kernels_f32_f32_large(int d, int gh, int kind, bool append, bool scaled) {
  return by_d<PA_F32, PA_F32, true>(d, gh, kind, append, scaled);
}

}  // namespace pa
