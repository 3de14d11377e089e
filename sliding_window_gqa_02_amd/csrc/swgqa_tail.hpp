// swgqa_tail.hpp -- in-place cache write-back of one (item, KV head) slice
// in the shared-buffer mode: surviving rows [shift, Lb) move to [0, kept),
// then the new rows [max(0, -kept), S) land at kept + i ("Specify
// GroupQueryAttention windowed KV cache layout contract", Description: rows
// [0, L(T)) hold the newest L(T) positions; "[CPU] Add windowed kv cache for
// GQA", block compaction, skipped on drifting steps where the append was
// already done during attention).  Runs at the end of the attention kernel,
// once no row it overwrites is still to be read: after a barrier when one
// workgroup reads the slice; with several query tiles per slice, in the
// tile that arrives last on the slice's counter.  The counter and its
// release/acquire fences are used only on compacting steps (each agent-scope
// release writes back this XCD's L2, measured far too slow to pay on every
// step); drifting steps only append, to rows no tile reads.
#pragma once

#include "swgqa_common.hpp"
#include "swgqa_internal.hpp"

namespace swgqa {

// 16-byte words per thread and tensor that one pass of a move holds in
// registers: kernels whose occupancy is bounded by their attention loop take
// 16; those whose attention loop needs fewer registers than 16 words of K
// and V would take 8 (the move's peak would otherwise set the kernel's
// register count and with it its occupancy).
constexpr int kMoveUnroll = 16;

// In-place move of rows [shift, shift + kept) -> [0, kept) of the K slice and,
// if `v` is not null, of the V slice at the same offsets; rows are `w16`
// 16-byte words apart and words [0, 2^wlog) of each row move (a column part
// of the row when several workgroups share a slice).  Passes take as many
// rows as the workgroup holds in registers: every load of a pass is issued
// (clamped to a valid word), then -- if the pass is longer than `shift`, so
// that its destinations overlap its own sources -- a barrier, then its
// stores, then a barrier before the next pass, whose destinations are this
// pass's sources.
template <int UNROLL = kMoveUnroll>
__device__ __forceinline__ void move_rows_in_place(u32x4* k, u32x4* v, int64_t w16, int wlog,
                                                   int64_t shift, int64_t kept, int tid,
                                                   int nthr) {
  const int64_t cap_rows = ((int64_t)nthr * UNROLL) >> wlog;
  const int64_t pass = cap_rows > 0 ? cap_rows : 1;
  const int64_t wmask = ((int64_t)1 << wlog) - 1;
  for (int64_t r0 = 0; r0 < kept; r0 += pass) {
    const int64_t nr = kept - r0 < pass ? kept - r0 : pass;
    const int64_t nw = nr << wlog;
    u32x4 bk[UNROLL], bv[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t idx = min(tid + (int64_t)u * nthr, nw - 1);
      const int64_t at = (shift + r0 + (idx >> wlog)) * w16 + (idx & wmask);
      bk[u] = k[at];
      if (v) bv[u] = v[at];
    }
    if (nr > shift) __syncthreads();
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t idx = tid + (int64_t)u * nthr;
      if (idx < nw) {
        const int64_t at = (r0 + (idx >> wlog)) * w16 + (idx & wmask);
        k[at] = bk[u];
        if (v) v[at] = bv[u];
      }
    }
    __syncthreads();
  }
}

// Cache write-back of slice (b, kvh) for both K and V, shared buffer; with
// `moved` the surviving rows are already in place and only the new rows land.
template <int UNROLL>
__device__ __forceinline__ void slice_writeback_shared(const AttnArgs& a, const ItemPlan& pl,
                                                       int b, int kvh, int D, int e,
                                                       const u32x4* knew, const u32x4* vnew,
                                                       bool moved) {
  const int64_t rowb = (int64_t)D * e;
  const int64_t w16 = rowb / 16;
  const int64_t off = ((int64_t)b * a.Hkv + kvh) * a.C * rowb;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  if (pl.shift > 0) {
    if (pl.kept > 0 && !moved)
      move_rows_in_place<UNROLL>((u32x4*)((char*)a.present_k + off), (u32x4*)((char*)a.present_v + off),
                         w16, __builtin_ctzll(w16), pl.shift, pl.kept, tid, nthr);
    // new rows after the move (they may land on rows the move read)
    const int64_t i0 = pl.kept < 0 ? -pl.kept : 0;
    const int64_t nw = (a.S - i0) * w16;
    u32x4* dk = (u32x4*)((char*)a.present_k + off);
    u32x4* dv = (u32x4*)((char*)a.present_v + off);
    for (int64_t idx = tid; idx < nw; idx += nthr) {
      const int64_t i = i0 + idx / w16, w = idx % w16;
      const int64_t src = (((int64_t)b * a.S + i) * a.Hkv + kvh) * rowb;
      dk[(pl.kept + i) * w16 + w] = knew ? knew[i * w16 + w]
                                         : ((const u32x4*)((const char*)a.k + src))[w];
      dv[(pl.kept + i) * w16 + w] = vnew ? vnew[i * w16 + w]
                                         : ((const u32x4*)((const char*)a.v + src))[w];
    }
  }
}

// The end of a step for one workgroup of slice (b, kvh).  With one key split
// the write-back runs here: directly when this workgroup is the slice's only
// reader, else in the last of the a.ntiles query tiles to finish.  Each tile
// counts its arrival with an acq_rel read-modify-write at agent scope after a
// barrier, i.e. after all its reads of the slice; the last arrival therefore
// happens after every read of every tile, resets the counter for the next
// call, and rewrites the slice.  Other launch shapes rewrite the cache in a
// separate kernel.
//
// ce is the cache element size in bytes; knew / vnew, if not NULL, hold the
// step's new key / value rows of the slice in cache form (S rows of D * ce /
// 16 words, in LDS) to store in place of a.k's / a.v's.  `moved`: the only
// reader of the slice has already moved the surviving rows while reading
// them.
template <int UNROLL = kMoveUnroll>
__device__ __forceinline__ void slice_tail_rows(const AttnArgs& a, const ItemPlan& pl, int b,
                                                int kvh, int D, int ce, const u32x4* knew,
                                                const u32x4* vnew, bool moved = false) {
  if (!a.fuse_writeback || pl.shift == 0) return;  // drifting: appended by tile 0
  __syncthreads();  // all reads of this slice by this workgroup are done
  if (a.ntiles > 1) {
    __shared__ uint32_t s_last;
    if (threadIdx.x == 0) {
      uint32_t* ctr = a.slice_counters + ((int64_t)b * a.Hkv + kvh);
      const uint32_t seen =
          __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t last = seen + 1u == (uint32_t)a.ntiles ? 1u : 0u;
      if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
  }
  slice_writeback_shared<UNROLL>(a, pl, b, kvh, D, ce, knew, vnew, moved);
}

// Key splits of a slice read as one query tile by the chunk kernel: the band
// [lo, p_last] = [max(P - W + 1, 0), P + S - 1] cut into parts of `per` keys,
// ceil(nkeys / nsplit) rounded up to whole kChunkBlockKeys-key blocks (the
// kernel's split rule); split s reads [lo + s per, min(lo + (s + 1) per,
// p_last + 1)).
struct ChunkSplits {
  int64_t lo, p_last, per;
};
__device__ __forceinline__ ChunkSplits chunk_splits(const ItemPlan& pl, int S, int W, int nsplit,
                                                    const GapDiv& sdiv) {
  ChunkSplits c;
  c.p_last = pl.P + S - 1;
  c.lo = pl.P - W + 1 > 0 ? pl.P - W + 1 : 0;
  const int64_t nkeys = c.p_last - c.lo + 1;
  c.per = ((int64_t)div_gap((uint32_t)(nkeys + nsplit - 1), sdiv) + kChunkBlockKeys - 1) /
          kChunkBlockKeys * kChunkBlockKeys;
  return c;
}

// Whether the key splits of a one-tile chunk step move the surviving rows of
// this item themselves: a compacting step (shift > 0, kept > 0) whose shift
// fits the rows set aside per split, and whose surviving rows -- positions
// P - Lb + shift .. P - 1 -- all lie in the key band (so every one of them is
// read, and stored, by exactly one split).
__device__ __forceinline__ bool chunk_moves_rows(const ItemPlan& pl, int W, int stash_rows) {
  const int64_t lo = pl.P - W + 1 > 0 ? pl.P - W + 1 : 0;
  return pl.shift > 0 && pl.kept > 0 && pl.shift <= stash_rows &&
         pl.P - pl.Lb + pl.shift >= lo;
}

template <int DT>
__device__ __forceinline__ void slice_tail(const AttnArgs& a, const ItemPlan& pl, int b, int kvh,
                                           int D, const u32x4* knew = nullptr,
                                           bool moved = false) {
  slice_tail_rows(a, pl, b, kvh, D, Elem<DT>::bytes, knew, nullptr, moved);
}

}  // namespace swgqa
