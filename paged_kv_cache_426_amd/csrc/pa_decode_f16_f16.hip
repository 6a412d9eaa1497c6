// Decode kernels for float16 queries and float16 caches.

#include "pa_decode_kernel.h"

namespace pa {

KernelRef decode_kernels_f16_f16(int d, int gh, int kind, bool append, bool scaled) {
  return by_d<PA_F16, PA_F16, false>(d, gh, kind, append, scaled);
}

}  // namespace pa
