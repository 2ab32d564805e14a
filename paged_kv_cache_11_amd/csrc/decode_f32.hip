// decode_f32.hip — decode instantiations for an f32 cache read by f32 queries
// (head size 64: one token row is 16 lanes x 16 bytes).
#include "decode_impl.h"

namespace pa {

hipError_t decode_f32(const DecodeArgs& a) {
  if (a.head_size != 64) return kNotInstantiated;
  return dispatch_block<F32, F32, 64>(a);
}

}  // namespace pa
