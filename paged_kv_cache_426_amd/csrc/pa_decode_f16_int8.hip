// Decode kernels for float16 queries and int8 caches (16-token blocks).

#include "pa_decode_kernel.h"

namespace pa {

KernelRef decode_kernels_f16_int8(int d, int gh, int kind, bool append, bool scaled) {
  return by_d<PA_F16, PA_INT8, false>(d, gh, kind, append, scaled);
}

}  // namespace pa
