// swgqa_step_tail.hip -- the work that follows the attention kernel when it
// does not finish the step itself, in one launch: the merge of key-split
// partials into the output, and the cache write-back (append + block
// compaction).  The two parts touch disjoint memory (partials and output;
// cache rows and new rows) and run side by side in one grid: the first
// workgroups merge, the rest rewrite the cache.
//
// Merge: for every query row, m = max_s m_s, l = sum_s l_s 2^(m_s - m),
// out = sum_s acc_s 2^(m_s - m) / l (log2 units, the online-softmax merge),
// rounded to nearest-even in the output type.  Items whose seqlens_k is out
// of range get zero rows, as the attention kernels give them.
//
// Write-back: after a step, rows [0, La) of present hold the newest La rows
// of the logical concatenation [resident rows | S new rows] ("Specify
// GroupQueryAttention windowed KV cache layout contract", Description).  In
// cache terms ("[CPU] Add windowed kv cache for GQA", key design decisions):
// the old rows [shift, Lb) move to [0, kept) -- only when a gap-sized block is
// reclaimed (shift > 0); on drifting steps nothing moves -- and the new rows
// land after them.  Rows a step of S > C never keeps are dropped.  This runs
// after attention on the same stream, so in the shared-buffer mode (present
// == past) no row a query reads is overwritten early.  In place, the move
// overlaps itself whenever kept > shift; it is done per (item, KV head,
// K|V, column part) with the pass-wise register-staged move of
// swgqa_tail.hpp.  The append waits for the whole move, since new rows may
// land on rows the move still reads.  After a 16-bit chunk step with key
// splits that moved the surviving rows itself, only the rows it set aside
// (those whose new place another split was still to read) are stored here.
#include "swgqa_common.hpp"
#include "swgqa_internal.hpp"
#include "swgqa_tail.hpp"

namespace swgqa {

namespace {

constexpr int kTailThreads = 256;
constexpr int kMergeGroup = 8;  // key splits whose partials are loaded together
constexpr int kCopyUnroll = 4;  // words per thread whose loads are issued together

// Column parts per row: the workgroups of one (item, KV head, K|V) slice
// each move a disjoint set of 16-byte words of every row, so they need no
// ordering between them.
__host__ __device__ inline int writeback_columns(int w16) { return w16 < 4 ? w16 : 4; }

// Merge of query rows: D / 4 threads per row, four outputs each.
template <int DT>
__device__ __forceinline__ void merge_rows(const AttnArgs& a, int D, uint32_t blk) {
  const int tpr = D / 4;
  const int rows_per_block = kTailThreads / tpr;
  const uint32_t nrows = (uint32_t)a.B * a.S * a.Hq;
  const uint32_t row = blk * rows_per_block + threadIdx.x / tpr;
  if (row >= nrows) return;
  const int d = (int)(threadIdx.x % tpr) * 4;
  const int b = (int)(row / (uint32_t)(a.S * a.Hq));
  // Splits in groups of kMergeGroup whose loads (pairs and partials) are all
  // issued before any is used: one memory round trip per group, not per
  // split or per pass -- the first group's before the item's plan, whose
  // seqlens_k read would otherwise come first.  The group's largest m joins
  // the running one, the sums so far are rescaled to it, and the group's
  // terms are added; indices past the last split repeat it and are not
  // summed.
  const int64_t r0 = (int64_t)row * a.nsplit;
  const int ns = a.nsplit;
  const float2* ml2 = (const float2*)a.ml;
  float2 v[kMergeGroup];
  float4 p[kMergeGroup];
  auto load_group = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kMergeGroup; ++j) {
      const int64_t s = r0 + min(s0 + j, ns - 1);
      v[j] = ml2[s];
      p[j] = *(const float4*)(a.opart + s * D + d);
    }
  };
  load_group(0);
  const ItemPlan pl = plan_item(a.seqlens[b], a.S, a.C, a.gdiv, a.total);
  float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (pl.ok) {
    float M = -INFINITY;
    float L = 0.0f;
    float A[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < ns; s0 += kMergeGroup) {
      if (s0 > 0) load_group(s0);
      float Mg = M;
#pragma unroll
      for (int j = 0; j < kMergeGroup; ++j) Mg = fmaxf(Mg, v[j].x);
      if (s0 > 0) {
        const float r = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - Mg);
        L *= r;
#pragma unroll
        for (int i = 0; i < 4; ++i) A[i] *= r;
      }
      M = Mg;
#pragma unroll
      for (int j = 0; j < kMergeGroup; ++j) {
        const bool in = s0 + j < ns;
        const float c = (v[j].x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(v[j].x - M);
        L = in ? L + v[j].y * c : L;
        A[0] = in ? A[0] + p[j].x * c : A[0];
        A[1] = in ? A[1] + p[j].y * c : A[1];
        A[2] = in ? A[2] + p[j].z * c : A[2];
        A[3] = in ? A[3] + p[j].w * c : A[3];
      }
    }
    const float c = fold_sink<DT>(a.sink, a.smooth, (int)(row % (uint32_t)a.Hq), M, L);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = A[i] * c / L;
  }
  const int64_t at = (int64_t)row * D + d;
  if constexpr (DT == kF32) {
    *(float4*)((float*)a.out + at) = make_float4(o[0], o[1], o[2], o[3]);
  } else {
    const uint32_t w0 = pack_word<DT>(o), w1 = pack_word<DT>(o + 2);
    *(uint2*)((uint16_t*)a.out + at) = make_uint2(w0, w1);
  }
}

// Write-back of one (item, KV head, K|V, column part).  With an int8 cache
// the new rows are quantized as they are written (16 codes per word).  `at`
// is the attention launch's arguments (its key splits and stash).
template <int DT>
__device__ __forceinline__ void writeback_part(const CopyArgs& a, const AttnArgs& at,
                                               uint32_t idx) {
  const int64_t rowb = (int64_t)a.D * a.elem_bytes;
  const int64_t w16 = rowb / 16;  // 16-byte words per row (a power of two)
  const int ncol = writeback_columns((int)w16);
  const int kvh = (int)(idx % (uint32_t)a.Hkv);
  const uint32_t rest = idx / (uint32_t)a.Hkv;
  const int b = (int)(rest % (uint32_t)a.B);
  const int z = (int)(rest / (uint32_t)a.B);
  const int which = z / ncol;  // 0: key cache, 1: value cache
  const int col = z % ncol;
  const int64_t wn = w16 / ncol;  // words of each row this workgroup moves
  const int wlog = __builtin_ctzll(wn);
  const ItemPlan pl = plan_item(a.seqlens[b], a.S, a.C, a.gdiv, a.total);
  if (!pl.ok) return;

  const void* past = which ? a.past_v : a.past_k;
  void* present = which ? a.present_v : a.present_k;
  const char* fresh = (const char*)(which ? a.v : a.k);
  const bool shared = present == past;
  if (shared && pl.shift == 0 && a.skip_drifting) return;  // appended by attention

  const int64_t slice = ((int64_t)b * a.Hkv + kvh) * a.C * rowb;
  const u32x4* src = (const u32x4*)((const char*)past + slice) + col * wn;
  u32x4* dst = (u32x4*)((char*)present + slice) + col * wn;
  const int tid = threadIdx.x;

  // 1. Surviving old rows: [shift, shift + kept) -> [0, kept).
  const bool stashed = shared && at.stash && chunk_moves_rows(pl, at.W, at.stash_rows);
  if (stashed) {
    // moved by the chunk kernel's key splits but for the first `shift`
    // positions of every split after the first, set aside in its stash
    // slots (pos - kb); they land on the previous split's rows.  Loads of
    // kCopyUnroll words per thread are issued together.
    const ChunkSplits cs = chunk_splits(pl, a.S, at.W, at.nsplit, at.sdiv);
    const uint32_t rowsz = (uint32_t)pl.shift << wlog;  // words of one split's slots
    const uint32_t nw = (uint32_t)(at.nsplit - 1) * rowsz;
    const int64_t lo_keep = pl.P - pl.Lb + pl.shift;  // first surviving position
    const u32x4* const stash =
        (const u32x4*)at.stash + (((int64_t)b * a.Hkv + kvh) * at.nsplit * 2 + which) *
                                     at.stash_rows * w16 + col * wn;
    for (uint32_t i0 = tid; i0 < nw; i0 += kCopyUnroll * kTailThreads) {
      u32x4 x[kCopyUnroll];
      int64_t to[kCopyUnroll];
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) {
        const uint32_t i = i0 + (uint32_t)u * kTailThreads;
        const uint32_t sm1 = i < nw ? i / rowsz : 0;  // split - 1
        const uint32_t r = (i - sm1 * rowsz) >> wlog;
        const uint32_t w = i & (uint32_t)(wn - 1);
        const int64_t kb = cs.lo + (int64_t)(sm1 + 1) * cs.per;
        const int64_t ke = kb + cs.per < cs.p_last + 1 ? kb + cs.per : cs.p_last + 1;
        const int64_t pos = kb + r;
        const bool ok = i < nw && pos >= lo_keep && pos < ke && pos < pl.P;
        // slot r of split sm1 + 1 (K or V), this column part; word 0 of the
        // first slot when there is nothing to store
        x[u] = stash[ok ? ((int64_t)(sm1 + 1) * 2 * at.stash_rows + r) * w16 + w : 0];
        to[u] = ok ? (pos - lo_keep) * w16 + w : -1;
      }
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u)
        if (to[u] >= 0) dst[to[u]] = x[u];
    }
  } else if (pl.kept > 0 && (!shared || pl.shift > 0)) {
    if (shared) {
      move_rows_in_place(dst, nullptr, w16, wlog, pl.shift, pl.kept, tid, kTailThreads);
    } else {
      // separate buffers: loads of kCopyUnroll words issued together
      const int64_t nw = pl.kept * wn;
      for (int64_t i0 = tid; i0 < nw; i0 += kCopyUnroll * kTailThreads) {
        u32x4 x[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
          const int64_t i = min(i0 + (int64_t)u * kTailThreads, nw - 1);
          x[u] = src[(pl.shift + (i >> wlog)) * w16 + (i & (wn - 1))];
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
          const int64_t i = i0 + (int64_t)u * kTailThreads;
          if (i < nw) dst[(i >> wlog) * w16 + (i & (wn - 1))] = x[u];
        }
      }
    }
  }
  // (stashed rows land below kept, from their own buffer: no wait for them)
  if (!stashed) __syncthreads();

  // 2. New rows i in [max(0, -kept), S) -> row kept + i.
  const int64_t i0 = pl.kept < 0 ? -pl.kept : 0;
  const int64_t nw = (a.S - i0) * wn;
  if (a.quant) {
    const int64_t src_rowb = (int64_t)a.D * a.src_elem_bytes;
    const float scale = which ? a.v_scale : a.k_scale;
    for (int64_t j = tid; j < nw; j += kTailThreads) {
      const int64_t i = i0 + (j >> wlog);
      const int64_t w = j & (wn - 1);
      const char* srow = fresh + (((int64_t)b * a.S + i) * a.Hkv + kvh) * src_rowb;
      dst[(pl.kept + i) * w16 + w] =
          a.quant == kCodeFp8 ? quant_chunk16<DT, kCodeFp8>(srow, (col * wn + w) * 16, scale)
                              : quant_chunk16<DT, kCodeInt8>(srow, (col * wn + w) * 16, scale);
    }
    return;
  }
  for (int64_t j = tid; j < nw; j += kTailThreads) {
    const int64_t i = i0 + (j >> wlog);
    const int64_t w = j & (wn - 1);
    const u32x4* s = (const u32x4*)(fresh + (((int64_t)b * a.S + i) * a.Hkv + kvh) * rowb) + col * wn;
    dst[(pl.kept + i) * w16 + w] = s[w];
  }
}

// Workgroups [0, merge_blocks) merge, the rest write back.
template <int DT>
__global__ __launch_bounds__(kTailThreads) void step_tail_kernel(AttnArgs a, CopyArgs c,
                                                                 uint32_t merge_blocks) {
  if (blockIdx.x < merge_blocks) merge_rows<DT>(a, c.D, blockIdx.x);
  else writeback_part<DT>(c, a, blockIdx.x - merge_blocks);
}

}  // namespace

hipError_t launch_step_tail(int dtype, const AttnArgs& a, const CopyArgs& c, bool merge,
                            bool writeback, hipStream_t st) {
  const int D = c.D;
  const uint32_t rows = (uint32_t)a.B * a.S * a.Hq;
  const uint32_t rows_per_block = kTailThreads / (D / 4);
  const uint32_t merge_blocks = merge ? (rows + rows_per_block - 1) / rows_per_block : 0;
  const uint32_t wb_blocks =
      writeback ? (uint32_t)c.Hkv * c.B * 2 * writeback_columns(D * c.elem_bytes / 16) : 0;
  const uint32_t blocks = merge_blocks + wb_blocks;
  if (blocks == 0) return hipSuccess;
  switch (dtype) {
    case kF32: step_tail_kernel<kF32><<<blocks, kTailThreads, 0, st>>>(a, c, merge_blocks); break;
    case kF16: step_tail_kernel<kF16><<<blocks, kTailThreads, 0, st>>>(a, c, merge_blocks); break;
    case kBF16: step_tail_kernel<kBF16><<<blocks, kTailThreads, 0, st>>>(a, c, merge_blocks); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace swgqa
