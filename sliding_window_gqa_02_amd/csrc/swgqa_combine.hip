// swgqa_combine.hip -- merges the key-split partials of the attention
// kernels: for every query row, m = max_s m_s, l = sum_s l_s 2^(m_s - m),
// out = sum_s acc_s 2^(m_s - m) / l (log2 units, the online-softmax merge),
// rounded to nearest-even in the output type.  Items whose seqlens_k is out
// of range get zero rows, as the attention kernels give them.
#include "swgqa_common.hpp"
#include "swgqa_internal.hpp"

namespace swgqa {

namespace {

// One workgroup of max(D, 64) threads per (item, position, head) row.
template <int DT>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a, int D) {
  const int64_t row = blockIdx.x;  // (b * S + i) * Hq + h
  const int b = (int)(row / ((int64_t)a.S * a.Hq));
  const int d = threadIdx.x;
  if (d >= D) return;
  const ItemPlan pl = plan_item(a.seqlens[b], a.S, a.C, a.gdiv, a.total);
  float o = 0.0f;
  if (pl.ok) {
    float M = -INFINITY;
    for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.ml[(row * a.nsplit + s) * 2]);
    float L = 0.0f, A = 0.0f;
    for (int s = 0; s < a.nsplit; ++s) {
      const float ms = a.ml[(row * a.nsplit + s) * 2];
      const float c = (ms == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
      L += a.ml[(row * a.nsplit + s) * 2 + 1] * c;
      A += a.opart[(row * a.nsplit + s) * D + d] * c;
    }
    o = A / L;
  }
  if constexpr (DT == kF32) ((float*)a.out)[row * D + d] = o;
  else if constexpr (DT == kF16) ((_Float16*)a.out)[row * D + d] = (_Float16)o;
  else ((uint16_t*)a.out)[row * D + d] = f32_to_bf16(o);
}

}  // namespace

hipError_t launch_combine(int dtype, int D, const AttnArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.B * a.S * a.Hq));
  const dim3 block(D < 64 ? 64 : D);
  switch (dtype) {
    case kF32: combine_kernel<kF32><<<grid, block, 0, st>>>(a, D); break;
    case kF16: combine_kernel<kF16><<<grid, block, 0, st>>>(a, D); break;
    case kBF16: combine_kernel<kBF16><<<grid, block, 0, st>>>(a, D); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace swgqa
