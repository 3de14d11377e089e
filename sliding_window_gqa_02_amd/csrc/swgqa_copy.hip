// swgqa_copy.hip -- the planner kernel (resident ranges of every item, for
// tests of the planner) and the workspace fill kernel.
#include "swgqa_common.hpp"
#include "swgqa_internal.hpp"

namespace swgqa {

namespace {

__global__ void plan_kernel(const int32_t* seqlens, int32_t B, int32_t S,
                            int32_t C, int32_t W, GapDiv gdiv, int32_t total, int64_t* out) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const ItemPlan pl = plan_item(seqlens[b], S, C, gdiv, total);
  int64_t* o = out + 8 * (int64_t)b;
  if (!pl.ok) {
    for (int f = 0; f < 8; ++f) o[f] = -1;
    return;
  }
  // hazard: compacting before attention would drop history query 0 reads
  const int64_t need = pl.P < W - 1 ? pl.P : (int64_t)W - 1;
  o[0] = pl.T;
  o[1] = pl.P;
  o[2] = pl.Lb;
  o[3] = pl.La;
  o[4] = pl.kept;
  o[5] = pl.shift;
  o[6] = pl.T - pl.La;
  o[7] = pl.kept < need ? 1 : 0;
}

// int8 codes of the step's new key and value rows (four elements a thread
// and pass), for the chunk kernel over an int8 cache.
template <int DT, int CT>
__global__ void quant_rows_kernel(const void* k, const void* v, uint32_t* kq, uint32_t* vq,
                                  size_t nwords, float ks, float vs) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords;
       i += (size_t)gridDim.x * blockDim.x) {
    uint32_t ck = 0u, cv = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ck |= quant_code_t<CT>(load_one<DT>(k, (int64_t)(4 * i + j)), ks) << (8 * j);
      cv |= quant_code_t<CT>(load_one<DT>(v, (int64_t)(4 * i + j)), vs) << (8 * j);
    }
    kq[i] = ck;
    vq[i] = cv;
  }
}

__global__ void zero_words_kernel(uint32_t* words, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    words[i] = 0u;
}

}  // namespace

hipError_t launch_plan(const int32_t* seqlens, int32_t B, int32_t S, int32_t C,
                       int32_t W, int32_t total, int64_t* out, hipStream_t st) {
  const int threads = 64;
  plan_kernel<<<(B + threads - 1) / threads, threads, 0, st>>>(
      seqlens, B, S, C, W, make_gap_div((uint32_t)(C - W + 1)), total, out);
  return hipGetLastError();
}

namespace {

template <int CT>
hipError_t launch_quant_ct(int dtype, const void* k, const void* v, uint32_t* kq, uint32_t* vq,
                           size_t nwords, float ks, float vs, unsigned blocks, hipStream_t st) {
  switch (dtype) {
    case kF32: quant_rows_kernel<kF32, CT><<<blocks, 256, 0, st>>>(k, v, kq, vq, nwords, ks, vs); break;
    case kF16: quant_rows_kernel<kF16, CT><<<blocks, 256, 0, st>>>(k, v, kq, vq, nwords, ks, vs); break;
    case kBF16: quant_rows_kernel<kBF16, CT><<<blocks, 256, 0, st>>>(k, v, kq, vq, nwords, ks, vs); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_rows(int dtype, int ct, const void* k, const void* v, uint8_t* kq,
                             uint8_t* vq, size_t n, float k_scale, float v_scale, hipStream_t st) {
  const size_t nwords = n / 4;
  if (nwords == 0) return hipSuccess;
  size_t blocks = (nwords + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (ct == kCodeFp8)
    return launch_quant_ct<kCodeFp8>(dtype, k, v, (uint32_t*)kq, (uint32_t*)vq, nwords, k_scale,
                                     v_scale, (unsigned)blocks, st);
  return launch_quant_ct<kCodeInt8>(dtype, k, v, (uint32_t*)kq, (uint32_t*)vq, nwords, k_scale,
                                    v_scale, (unsigned)blocks, st);
}

hipError_t launch_zero_words(uint32_t* words, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  zero_words_kernel<<<(unsigned)blocks, 256, 0, st>>>(words, n);
  return hipGetLastError();
}

}  // namespace swgqa
