// swgqa_attn_decode_q8.hip -- the staged decode kernel of
// swgqa_attn_decode_q8.hpp for int8 caches, and the shape queries of that
// kernel.
#include "swgqa_attn_decode_q8.hpp"

namespace swgqa {

bool decode_q8_supports(int D, int nq) {
  if (nq != 2 && nq != 4) return false;
  switch (D) {
    case 16: return nq == 2 ? Q8Shape<16, 2>::ok : Q8Shape<16, 4>::ok;
    case 32: return nq == 2 ? Q8Shape<32, 2>::ok : Q8Shape<32, 4>::ok;
    case 64: return nq == 2 ? Q8Shape<64, 2>::ok : Q8Shape<64, 4>::ok;
    case 128: return nq == 2 ? Q8Shape<128, 2>::ok : Q8Shape<128, 4>::ok;
    case 256: return nq == 2 ? Q8Shape<256, 2>::ok : Q8Shape<256, 4>::ok;
    default: return false;
  }
}

int decode_q8_stage_rows(int D, int nq) {
  switch (D) {
    case 16: return q8_stage_rows_d<16>(nq);
    case 32: return q8_stage_rows_d<32>(nq);
    case 64: return q8_stage_rows_d<64>(nq);
    case 128: return q8_stage_rows_d<128>(nq);
    case 256: return q8_stage_rows_d<256>(nq);
    default: return 1;
  }
}

hipError_t launch_attn_decode_q8(int dtype, int D, int nq, const AttnArgs& a, hipStream_t st) {
  return launch_q8_ct<kCodeInt8>(dtype, D, nq, a, st);
}

}  // namespace swgqa
