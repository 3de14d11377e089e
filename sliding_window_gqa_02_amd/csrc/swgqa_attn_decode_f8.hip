// swgqa_attn_decode_f8.hip -- the staged decode kernel of
// swgqa_attn_decode_q8.hpp for fp8 E4M3 caches.
#include "swgqa_attn_decode_q8.hpp"

namespace swgqa {

hipError_t launch_attn_decode_f8(int dtype, int D, int nq, const AttnArgs& a, hipStream_t st) {
  return launch_q8_ct<kCodeFp8>(dtype, D, nq, a, st);
}

}  // namespace swgqa
