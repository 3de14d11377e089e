// swgqa_copy.hip -- cache write-back (append + block compaction), the
// planner kernel and the status-word reset.
//
// After a step, rows [0, La) of present hold the newest La rows of the
// logical concatenation [resident rows | S new rows] ("Specify
// GroupQueryAttention windowed KV cache layout contract", Description).  In
// cache terms ("[CPU] Add windowed kv cache for GQA", key design decisions):
// the old rows [shift, Lb) move to [0, kept) -- only when a gap-sized block is
// reclaimed (shift > 0); on drifting steps nothing moves -- and the new rows
// land after them.  Rows a step of S > C never keeps are dropped.
//
// This kernel runs after attention on the same stream, so in the shared
// buffer mode (present == past) no row a query reads is overwritten early.
// In place, the move [shift, Lb) -> [0, kept) overlaps itself whenever
// kept > shift; it is done by one workgroup per (item, KV head, K|V) with the
// pass-wise register-staged move of swgqa_tail.hpp.  The append waits for
// the whole move, since new rows may land on rows the move still reads.
#include "swgqa_common.hpp"
#include "swgqa_internal.hpp"
#include "swgqa_tail.hpp"

namespace swgqa {

namespace {

constexpr int kCopyThreads = 256;

// Column parts per row: the workgroups of one (item, KV head, K|V) slice
// each move a disjoint set of 16-byte words of every row, so they need no
// ordering between them.
__host__ __device__ inline int writeback_columns(int w16) { return w16 < 4 ? w16 : 4; }

__global__ __launch_bounds__(kCopyThreads) void writeback_kernel(CopyArgs a) {
  const int kvh = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t rowb = (int64_t)a.D * a.elem_bytes;
  const int64_t w16 = rowb / 16;  // 16-byte words per row (a power of two)
  const int ncol = writeback_columns((int)w16);
  const int which = blockIdx.z / ncol;  // 0: key cache, 1: value cache
  const int col = blockIdx.z % ncol;
  const int64_t wn = w16 / ncol;        // words of each row this workgroup moves
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
  if (pl.kept > 0 && (!shared || pl.shift > 0)) {
    if (shared) {
      move_rows_in_place(dst, nullptr, w16, wlog, pl.shift, pl.kept, tid, kCopyThreads);
    } else {
      const int64_t nw = pl.kept * wn;
      for (int64_t idx = tid; idx < nw; idx += kCopyThreads) {
        const int64_t r = idx >> wlog, w = idx & (wn - 1);
        dst[r * w16 + w] = src[(pl.shift + r) * w16 + w];
      }
    }
  }
  __syncthreads();

  // 2. New rows i in [max(0, -kept), S) -> row kept + i.
  const int64_t i0 = pl.kept < 0 ? -pl.kept : 0;
  const int64_t nw = (a.S - i0) * wn;
  for (int64_t idx = tid; idx < nw; idx += kCopyThreads) {
    const int64_t i = i0 + (idx >> wlog);
    const int64_t w = idx & (wn - 1);
    const u32x4* s = (const u32x4*)(fresh + (((int64_t)b * a.S + i) * a.Hkv + kvh) * rowb) + col * wn;
    dst[(pl.kept + i) * w16 + w] = s[w];
  }
}

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

__global__ void zero_words_kernel(uint32_t* words, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    words[i] = 0u;
}

}  // namespace

hipError_t launch_writeback(const CopyArgs& a, hipStream_t st) {
  const dim3 grid(a.Hkv, a.B, 2 * writeback_columns(a.D * a.elem_bytes / 16));
  writeback_kernel<<<grid, kCopyThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_plan(const int32_t* seqlens, int32_t B, int32_t S, int32_t C,
                       int32_t W, int32_t total, int64_t* out, hipStream_t st) {
  const int threads = 64;
  plan_kernel<<<(B + threads - 1) / threads, threads, 0, st>>>(
      seqlens, B, S, C, W, make_gap_div((uint32_t)(C - W + 1)), total, out);
  return hipGetLastError();
}

hipError_t launch_zero_words(uint32_t* words, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  zero_words_kernel<<<(unsigned)blocks, 256, 0, st>>>(words, n);
  return hipGetLastError();
}

}  // namespace swgqa
