// decode_bf16.hip — decode instantiations for a bf16 cache read by bf16 queries.
#include "decode_impl.h"

namespace pa {

hipError_t decode_bf16(const DecodeArgs& a) {
  switch (a.head_size) {
    case 64: return dispatch_block<BF16, BF16, 64>(a);
    case 128: return dispatch_block<BF16, BF16, 128>(a);
    default: return kNotInstantiated;
  }
}

}  // namespace pa
