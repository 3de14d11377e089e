// swgqa_attn_chunk.hip -- the MFMA chunk kernel of swgqa_attn_chunk.hpp for
// caches in the element type.
#include "swgqa_attn_chunk.hpp"

namespace swgqa {

bool chunk_kernel_supports(int dtype, int D) {
  if (dtype < kF32 || dtype > kBF16) return false;
  const int e = dtype == kF32 ? 4 : 2;
  return D >= 16 && D % 16 == 0 && D <= 256 && D * e <= 512;
}

int chunk_rows_per_workgroup(int waves, int groups) { return 16 * waves / groups; }
int chunk_keys_per_block() { return BN; }
static_assert(BN == kChunkBlockKeys, "key split ranges of the step tail");

bool chunk_kernel_moves_rows(int dtype) {
  switch (dtype) {
    case kF32: return chunk_split_moves<kF32, 0>();
    case kF16: return chunk_split_moves<kF16, 0>();
    case kBF16: return chunk_split_moves<kBF16, 0>();
    default: return false;
  }
}

hipError_t launch_attn_chunk(int dtype, int D, const AttnArgs& a, hipStream_t st) {
  switch (dtype) {
    case kF32: return launch_t<kF32, 0>(D, a, st);
    case kF16: return launch_t<kF16, 0>(D, a, st);
    case kBF16: return launch_t<kBF16, 0>(D, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace swgqa
