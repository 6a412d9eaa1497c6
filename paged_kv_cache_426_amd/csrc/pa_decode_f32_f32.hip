// Decode kernels for float32 queries and float32 caches.

#include "pa_decode_kernel.h"

namespace pa {

KernelRef decode_kernels_f32_f32(int d, int gh, int kind, bool append, bool scaled) {
  return by_d<PA_F32, PA_F32, false>(d, gh, kind, append, scaled);
}

}  // namespace pa
