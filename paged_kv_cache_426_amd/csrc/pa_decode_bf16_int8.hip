// Decode kernels for bfloat16 queries and int8 caches (16-token blocks).

#include "pa_decode_kernel.h"

namespace pa {

KernelRef decode_kernels_bf16_int8(int d, int gh, int kind, bool append, bool scaled) {
  return by_d<PA_BF16, PA_INT8, false>(d, gh, kind, append, scaled);
}

}  // namespace pa
