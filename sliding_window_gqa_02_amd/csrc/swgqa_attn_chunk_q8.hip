// swgqa_attn_chunk_q8.hip -- the MFMA chunk kernel of swgqa_attn_chunk.hpp
// for int8 caches: key rows read as codes (the cache, and a workspace copy
// of the step's new rows in code form), converted to the element type as
// they are staged.
#include "swgqa_attn_chunk.hpp"

namespace swgqa {

hipError_t launch_attn_chunk_q8(int dtype, int D, const AttnArgs& a, hipStream_t st) {
  switch (dtype) {
    case kF32: return launch_t<kF32, kCodeInt8>(D, a, st);
    case kF16: return launch_t<kF16, kCodeInt8>(D, a, st);
    case kBF16: return launch_t<kBF16, kCodeInt8>(D, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace swgqa
