// decode_fp8.hip — decode instantiations for an fp8 (E4M3FN) cache read by
// bf16 queries; keys and values are dequantised with per-tensor scales.
#include "decode_impl.h"

namespace pa {

hipError_t decode_fp8(const DecodeArgs& a) {
  switch (a.head_size) {
    case 64: return dispatch_block<FP8, BF16, 64>(a);
    case 128: return dispatch_block<FP8, BF16, 128>(a);
    default: return kNotInstantiated;
  }
}

}  // namespace pa
