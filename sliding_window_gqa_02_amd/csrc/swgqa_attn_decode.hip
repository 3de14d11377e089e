// swgqa_attn_decode.hip -- the staged decode kernel of swgqa_attn_decode.hpp
// without rotary embedding, for every supported head size.
#include "swgqa_attn_decode.hpp"

namespace swgqa {

namespace {

template <int DT>
int stage_rows_t(int D, int nq) {
  switch (D) {
    case 8: return stage_rows<DT, 8>(nq);
    case 16: return stage_rows<DT, 16>(nq);
    case 32: return stage_rows<DT, 32>(nq);
    case 64: return stage_rows<DT, 64>(nq);
    case 128: return stage_rows<DT, 128>(nq);
    default: return 1;
  }
}

template <int DT>
bool ok_t(int D, int nq) {
  switch (D) {
    case 8: return shape_ok<DT, 8>(nq);
    case 16: return shape_ok<DT, 16>(nq);
    case 32: return shape_ok<DT, 32>(nq);
    case 64: return shape_ok<DT, 64>(nq);
    case 128: return shape_ok<DT, 128>(nq);
    default: return false;
  }
}

template <int DT>
hipError_t launch_t(int D, int nq, const AttnArgs& a, hipStream_t st) {
  switch (D) {
    case 8: return launch_d<DT, 8, false>(nq, a, st);
    case 16: return launch_d<DT, 16, false>(nq, a, st);
    case 32: return launch_d<DT, 32, false>(nq, a, st);
    case 64: return launch_d<DT, 64, false>(nq, a, st);
    case 128: return launch_d<DT, 128, false>(nq, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_kernel_supports(int dtype, int D, int nq) {
  switch (dtype) {
    case kF32: return ok_t<kF32>(D, nq);
    case kF16: return ok_t<kF16>(D, nq);
    case kBF16: return ok_t<kBF16>(D, nq);
    default: return false;
  }
}

int decode_stage_rows(int dtype, int D, int nq) {
  switch (dtype) {
    case kF32: return stage_rows_t<kF32>(D, nq);
    case kF16: return stage_rows_t<kF16>(D, nq);
    case kBF16: return stage_rows_t<kBF16>(D, nq);
    default: return 1;
  }
}

hipError_t launch_attn_decode(int dtype, int D, int nq, const AttnArgs& a, hipStream_t st) {
  switch (dtype) {
    case kF32: return launch_t<kF32>(D, nq, a, st);
    case kF16: return launch_t<kF16>(D, nq, a, st);
    case kBF16: return launch_t<kBF16>(D, nq, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace swgqa
