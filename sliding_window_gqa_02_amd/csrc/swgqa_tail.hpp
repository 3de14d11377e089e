// swgqa_tail.hpp -- in-place cache write-back of one (item, KV head) slice
// in the shared-buffer mode: surviving rows [shift, Lb) move to [0, kept),
// then the new rows [max(0, -kept), S) land at kept + i ("Specify
// GroupQueryAttention windowed KV cache layout contract", Description: rows
// [0, L(T)) hold the newest L(T) positions; "[CPU] Add windowed kv cache for
// GQA", block compaction, skipped on drifting steps where the append was
// already done during attention).  Used at the end of an attention
// workgroup that owns the whole slice, after a barrier: no row it overwrites
// is still to be read.  (Cross-workgroup hand-off via device-scope fences was
// measured far slower here -- each release fence writes back L2 -- so other
// launch shapes use a separate write-back kernel.)
#pragma once

#include "swgqa_common.hpp"
#include "swgqa_internal.hpp"

namespace swgqa {

constexpr int kMoveUnroll = 16;  // 16-byte words per thread per pass

// In-place move of one cache slice, rows [shift, shift + kept) -> [0, kept),
// in passes of at most `shift` rows: a pass's destination rows were sources
// only of earlier passes, whose loads completed before the barrier.
__device__ __forceinline__ void move_rows_in_place(u32x4* slice, int64_t w16, int64_t shift,
                                                   int64_t kept, int tid, int nthr) {
  const int64_t cap_rows = (int64_t)nthr * kMoveUnroll / w16;
  const int64_t pass = shift < cap_rows ? shift : (cap_rows > 0 ? cap_rows : 1);
  for (int64_t r0 = 0; r0 < kept; r0 += pass) {
    const int64_t nr = kept - r0 < pass ? kept - r0 : pass;
    const int64_t nw = nr * w16;
    // all loads of the pass first (clamped to a valid word), then the stores
    u32x4 buf[kMoveUnroll];
#pragma unroll
    for (int u = 0; u < kMoveUnroll; ++u) {
      const int64_t idx = tid + (int64_t)u * nthr;
      buf[u] = slice[(shift + r0) * w16 + (idx < nw ? idx : nw - 1)];
    }
#pragma unroll
    for (int u = 0; u < kMoveUnroll; ++u) {
      const int64_t idx = tid + (int64_t)u * nthr;
      if (idx < nw) slice[r0 * w16 + idx] = buf[u];
    }
    __syncthreads();
  }
}

// Cache write-back of slice (b, kvh) for both K and V, shared buffer.
__device__ __forceinline__ void slice_writeback_shared(const AttnArgs& a, const ItemPlan& pl,
                                                       int b, int kvh, int D, int e) {
  const int64_t rowb = (int64_t)D * e;
  const int64_t w16 = rowb / 16;
  const int64_t off = ((int64_t)b * a.Hkv + kvh) * a.C * rowb;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  if (pl.shift > 0) {
    if (pl.kept > 0) {
      move_rows_in_place((u32x4*)((char*)a.present_k + off), w16, pl.shift, pl.kept, tid, nthr);
      move_rows_in_place((u32x4*)((char*)a.present_v + off), w16, pl.shift, pl.kept, tid, nthr);
    }
    // new rows after the move (they may land on rows the move read)
    const int64_t i0 = pl.kept < 0 ? -pl.kept : 0;
    const int64_t nw = (a.S - i0) * w16;
    u32x4* dk = (u32x4*)((char*)a.present_k + off);
    u32x4* dv = (u32x4*)((char*)a.present_v + off);
    for (int64_t idx = tid; idx < nw; idx += nthr) {
      const int64_t i = i0 + idx / w16, w = idx % w16;
      const int64_t src = (((int64_t)b * a.S + i) * a.Hkv + kvh) * rowb;
      dk[(pl.kept + i) * w16 + w] = ((const u32x4*)((const char*)a.k + src))[w];
      dv[(pl.kept + i) * w16 + w] = ((const u32x4*)((const char*)a.v + src))[w];
    }
  }
}

// The end of a step for a workgroup that owns its whole (item, KV head)
// slice (one query tile, one key split): once every wave has finished
// reading, the cache write-back of the slice runs in the same workgroup.
// Other launch shapes merge splits and rewrite the cache in separate kernels.
template <int DT>
__device__ __forceinline__ void slice_tail(const AttnArgs& a, const ItemPlan& pl, int b, int kvh,
                                           int D) {
  if (!a.fuse_writeback || pl.shift == 0) return;  // drifting: appended up front
  __syncthreads();  // all reads of this slice are done
  slice_writeback_shared(a, pl, b, kvh, D, Elem<DT>::bytes);
}

}  // namespace swgqa
