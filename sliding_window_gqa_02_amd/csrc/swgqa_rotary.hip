// swgqa_rotary.hip -- rotary embedding of the step's query and new key rows,
// a pass before attention when do_rotary is set.  The rotated rows go to
// workspace scratch, and every later kernel of the step reads them there:
// attention, the append and the write-back (so the cache stores rotated
// keys).
//
// The Investigation Report (onnxruntime/mobius issue #111), sections 1.1 and
// 1.3, names the inputs cos_cache / sin_cache (max_S, D/2) and position_ids
// (B, S) and the attributes do_rotary / rotary_interleaved.  Reading taken
// (the plainest): the pair (a, b) -- elements (k, k + D/2), or (2k, 2k + 1)
// when interleaved -- at position pos becomes (a c - b s, b c + a s), c and s
// from row pos, column k of the caches; each product, sum and difference is
// rounded to binary32 (no fused multiply-add), then the result to the
// element type.  pos = position_ids[b][i], or P + i without them.
//
// An item with a position outside the caches is invalid: the last workgroup
// checks every position and writes the per-item lengths the rest of the step
// reads, with an out-of-range length (-2) for such an item, so every later kernel
// skips it as it skips an out-of-range seqlens_k (zero output, cache
// untouched, status flagged).
#include "swgqa_common.hpp"
#include "swgqa_internal.hpp"

namespace swgqa {

namespace {

constexpr int kRotThreads = 256;

template <int DT>
__device__ __forceinline__ float load_elem(const void* base, int64_t i) {
  return load_one<DT>(base, i);
}

template <int DT>
__device__ __forceinline__ void store_elem(void* base, int64_t i, float x) {
  if constexpr (DT == kF32) ((float*)base)[i] = x;
  else if constexpr (DT == kF16) ((_Float16*)base)[i] = (_Float16)x;
  else ((uint16_t*)base)[i] = f32_to_bf16(x);
}

// (a, b) -> (a c - b s, b c + a s) in binary32 with one rounding per product,
// sum and difference: contraction into fused multiply-adds is off here.
__device__ __forceinline__ void rotate_pair(float a, float b, float c, float s, float& ra,
                                            float& rb) {
#pragma clang fp contract(off)
  const float ac = a * c, bs = b * s, bc = b * c, as = a * s;
  ra = ac - bs;
  rb = bc + as;
}

// Position of query/key row i of item b (plan P = seqlens_k[b] + 1 - S).
__device__ __forceinline__ int64_t rope_position(const RotaryArgs& r, int b, int i) {
  if (r.position_ids) return r.position_ids[(int64_t)b * r.S + i];
  return (int64_t)r.seqlens[b] + 1 - r.S + i;
}

template <int DT>
__global__ __launch_bounds__(kRotThreads) void rotary_kernel(RotaryArgs r) {
  const int half = r.D / 2;
  if (blockIdx.x == gridDim.x - 1) {
    // Per-item validity of every position -> the lengths the step reads.
    // Items go in chunks of kRotThreads; the (item, row) pairs of a chunk are
    // spread over all threads, so neither many short items nor one long item
    // serialises on one thread.
    __shared__ int bad[kRotThreads];
    for (int b0 = 0; b0 < r.B; b0 += kRotThreads) {
      const int nb = r.B - b0 < kRotThreads ? r.B - b0 : kRotThreads;
      bad[threadIdx.x] = 0;
      __syncthreads();
      const int64_t pairs = (int64_t)nb * r.S;
      for (int64_t f = threadIdx.x; f < pairs; f += kRotThreads) {
        const int bl = (int)(f / r.S), i = (int)(f % r.S);
        const int64_t pos = rope_position(r, b0 + bl, i);
        if (pos < 0 || pos >= r.rows) bad[bl] = 1;
      }
      __syncthreads();
      if ((int)threadIdx.x < nb) {
        const int b = b0 + threadIdx.x;
        r.seqlens_out[b] = bad[threadIdx.x] ? -2 : r.seqlens[b];  // -2: T = -1 < S
      }
      __syncthreads();
    }
    return;
  }
  const int64_t heads = r.Hq + r.Hkv;
  const int64_t total = (int64_t)r.B * r.S * heads * half;
  for (int64_t t = (int64_t)blockIdx.x * kRotThreads + threadIdx.x; t < total;
       t += (int64_t)(gridDim.x - 1) * kRotThreads) {
    const int k = (int)(t % half);
    const int64_t rh = t / half;              // ((b * S + i) * heads + h)
    const int h = (int)(rh % heads);
    const int64_t bi = rh / heads;            // b * S + i
    const int b = (int)(bi / r.S), i = (int)(bi % r.S);
    int64_t pos = rope_position(r, b, i);
    pos = pos < 0 ? 0 : (pos >= r.rows ? r.rows - 1 : pos);  // invalid items are skipped
    const bool is_q = h < r.Hq;
    const void* src = is_q ? r.q : r.k;
    void* dst = is_q ? r.q_out : r.k_out;
    const int64_t row = (bi * (is_q ? r.Hq : r.Hkv) + (is_q ? h : h - r.Hq)) * r.D;
    const int64_t ia = row + (r.interleaved ? 2 * k : k);
    const int64_t ib = row + (r.interleaved ? 2 * k + 1 : k + half);
    const float a = load_elem<DT>(src, ia);
    const float bb = load_elem<DT>(src, ib);
    const float c = load_elem<DT>(r.cos_cache, pos * half + k);
    const float s = load_elem<DT>(r.sin_cache, pos * half + k);
    float ra, rb;
    rotate_pair(a, bb, c, s, ra, rb);
    store_elem<DT>(dst, ia, ra);
    store_elem<DT>(dst, ib, rb);
  }
}

}  // namespace

hipError_t launch_rotary(int dtype, const RotaryArgs& r, hipStream_t st) {
  const int64_t work = (int64_t)r.B * r.S * (r.Hq + r.Hkv) * (r.D / 2);
  int64_t blocks = (work + kRotThreads - 1) / kRotThreads;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  const unsigned grid = (unsigned)blocks + 1;  // + the validity workgroup
  switch (dtype) {
    case kF32: rotary_kernel<kF32><<<grid, kRotThreads, 0, st>>>(r); break;
    case kF16: rotary_kernel<kF16><<<grid, kRotThreads, 0, st>>>(r); break;
    case kBF16: rotary_kernel<kBF16><<<grid, kRotThreads, 0, st>>>(r); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace swgqa
