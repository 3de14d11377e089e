// swgqa_attn_decode_rot.hip -- the staged decode kernel of
// swgqa_attn_decode.hpp with rotary embedding of the query and new key rows
// fused in, for the head sizes rotary embedding is used with here (32, 64,
// 128); other shapes rotate in a pass of their own (swgqa_rotary.hip).
#include "swgqa_attn_decode.hpp"

namespace swgqa {

namespace {

template <int DT>
hipError_t launch_rot_t(int D, int nq, const AttnArgs& a, hipStream_t st) {
  switch (D) {
    case 32: return launch_d<DT, 32, true>(nq, a, st);
    case 64: return launch_d<DT, 64, true>(nq, a, st);
    case 128: return launch_d<DT, 128, true>(nq, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_rotary_supports(int dtype, int D, int nq) {
  return (D == 32 || D == 64 || D == 128) && decode_kernel_supports(dtype, D, nq);
}

hipError_t launch_attn_decode_rot(int dtype, int D, int nq, const AttnArgs& a, hipStream_t st) {
  switch (dtype) {
    case kF32: return launch_rot_t<kF32>(D, nq, a, st);
    case kF16: return launch_rot_t<kF16>(D, nq, a, st);
    case kBF16: return launch_rot_t<kBF16>(D, nq, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace swgqa
