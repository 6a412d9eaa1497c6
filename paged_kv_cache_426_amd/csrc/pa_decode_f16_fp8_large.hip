// Decode kernels for float16 queries and fp8 e4m3fn caches, cache blocks of 32 to 256 tokens.

#include "pa_decode_kernel.h"

namespace pa {

KernelRef decode_kernels_f16_fp8_large(int d, int gh, int kind, bool append, bool scaled) {
  return by_d<PA_F16, PA_FP8_E4M3FN, true>(d, gh, kind, append, scaled);
}

}  // namespace pa
