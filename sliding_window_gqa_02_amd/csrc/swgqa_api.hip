// swgqa_api.hip -- the C ABI of libswgqa (declared in include/swgqa.h):
// host-side validation, launch planning and kernel dispatch.  No allocation,
// no synchronisation on the forward path.
#include "swgqa.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "swgqa_common.hpp"
#include "swgqa_internal.hpp"

namespace {

using namespace swgqa;

// Workspace: status word at byte 0, per-slice arrival counters from byte
// 256 to kHeaderBytes (zero between calls), then key-split partials.
constexpr size_t kStatusBytes = 256;
constexpr size_t kHeaderBytes = 16384;
constexpr int64_t kMaxSliceCounters = (int64_t)((kHeaderBytes - kStatusBytes) / 4);
#ifndef SWGQA_TARGET_WORKGROUPS
#define SWGQA_TARGET_WORKGROUPS 2048
#endif
#ifndef SWGQA_WHOLE_SLICE_MIN_TILES
#define SWGQA_WHOLE_SLICE_MIN_TILES 128
#endif
#ifndef SWGQA_WHOLE_SLICE_MAX_KEYS
#define SWGQA_WHOLE_SLICE_MAX_KEYS 256
#endif
// With few (item, KV head) slices, the staged decode kernel narrows its
// query tiles until the launch has at least this many workgroups.
#ifndef SWGQA_DECODE_MIN_WORKGROUPS
#define SWGQA_DECODE_MIN_WORKGROUPS 64
#endif
constexpr int kTargetWorkgroups = SWGQA_TARGET_WORKGROUPS;
constexpr int kMinKeysPerSplit = 32;
// Multi-token steps with at least this many query rows per KV head
// ((position, head) pairs) run on the matrix cores.
#ifndef SWGQA_CHUNK_MIN_ROWS
#define SWGQA_CHUNK_MIN_ROWS 32
#endif
#ifndef SWGQA_CHUNK_MIN_WORKGROUPS
#define SWGQA_CHUNK_MIN_WORKGROUPS 256
#endif
constexpr int kChunkMinTokens = 16;       // steps of at least this many tokens use MFMA
constexpr int kChunkMinRows = SWGQA_CHUNK_MIN_ROWS;
#ifndef SWGQA_CHUNK_WIDE_ROWS
#define SWGQA_CHUNK_WIDE_ROWS 128
#endif
constexpr int kChunkWideRows = SWGQA_CHUNK_WIDE_ROWS;
constexpr int64_t kChunkMinWorkgroups = SWGQA_CHUNK_MIN_WORKGROUPS;
#ifndef SWGQA_CHUNK_GROUPS
#define SWGQA_CHUNK_GROUPS 1
#endif
constexpr bool kChunkGroups = SWGQA_CHUNK_GROUPS != 0;
constexpr int64_t kWholeSliceMinTiles = SWGQA_WHOLE_SLICE_MIN_TILES;
constexpr int64_t kWholeSliceMaxKeys = SWGQA_WHOLE_SLICE_MAX_KEYS;
constexpr int64_t kDecodeMinWorkgroups = SWGQA_DECODE_MIN_WORKGROUPS;

size_t elem_bytes(int dt) { return dt == SWGQA_F32 ? 4 : 2; }

swgqa_status validate(const swgqa_params* p) {
  if (!p) return SWGQA_ERR_ARG;
  if (p->batch_size < 0 || p->sequence_length < 1 || p->num_heads < 1 ||
      p->kv_num_heads < 1 || p->head_size < 1 || p->capacity < 1)
    return SWGQA_ERR_ARG;
  if (p->num_heads % p->kv_num_heads != 0) return SWGQA_ERR_ARG;
  if (p->local_window_size < 1 || p->local_window_size > p->capacity) return SWGQA_ERR_ARG;
  if (p->total_sequence_length < 1) return SWGQA_ERR_ARG;
  if (!(p->scale >= 0.0f) || !(p->softcap >= 0.0f)) return SWGQA_ERR_ARG;
  if (p->smooth_softmax != 0 && p->smooth_softmax != 1) return SWGQA_ERR_ARG;
  if (p->do_rotary != 0 && p->do_rotary != 1) return SWGQA_ERR_ARG;
  if (p->rotary_interleaved != 0 && p->rotary_interleaved != 1) return SWGQA_ERR_ARG;
  if (p->do_rotary && (p->rotary_cache_rows < 1 || p->head_size % 2 != 0)) return SWGQA_ERR_ARG;
  if (p->dtype < SWGQA_F32 || p->dtype > SWGQA_BF16) return SWGQA_ERR_UNSUPPORTED;
  if (!head_size_supported(p->head_size)) return SWGQA_ERR_UNSUPPORTED;
  if (p->kv_cache_type < 0 || p->kv_cache_type > 2) return SWGQA_ERR_UNSUPPORTED;
  if (p->kv_cache_type != 0) {
    if (!(p->k_scale > 0.0f && p->v_scale > 0.0f && std::isfinite(p->k_scale) &&
          std::isfinite(p->v_scale)))
      return SWGQA_ERR_ARG;
    // int8 rows of whole 16-byte chunks
    if (p->head_size < 16) return SWGQA_ERR_UNSUPPORTED;
    // steps longer than the 8-bit staged kernel holds need the matrix-core
    // kernel, whose rows are at most 512 bytes (not fp32 at head size 256)
    if (p->sequence_length > kQ8MaxNewRows && !chunk_kernel_supports(p->dtype, p->head_size))
      return SWGQA_ERR_UNSUPPORTED;
  }
  return SWGQA_OK;
}

// Launch geometry of the attention kernels, a pure function of the
// parameters.
enum class Kind { kSplit, kDecode, kChunk, kDecodeQ8 };

struct SplitPlan {
  Kind kind;    // generic split / staged decode / MFMA chunk kernel
  int nq;       // query tile width ((position, head) pairs)
  int ntiles;   // tiles per (item, KV head)
  int nsplit;   // key splits per tile
  int waves;    // waves per workgroup (staged kernel)
  int groups = 1;  // chunk kernel: groups of waves that share the tile's rows
};

SplitPlan plan_split(const swgqa_params* p) {
  SplitPlan s;
  const int group = p->num_heads / p->kv_num_heads;
  const int per_kv = p->sequence_length * group;  // queries per (item, KV head)
  s.waves = 4;
  const bool multi_token = p->sequence_length >= kChunkMinTokens ||
                           (p->sequence_length >= 2 && per_kv >= kChunkMinRows);
  if (p->kv_cache_type != 0 && !(p->sequence_length >= kChunkMinTokens &&
                                 chunk_kernel_supports(p->dtype, p->head_size))) {
    // int8 cache: steps of S < 16 on the int8 staged kernel, tiles of 2 or 4
    // pairs, the same whole-slice / key-split choice as below (longer steps
    // take the matrix-core kernel, with codes)
    s.kind = Kind::kDecodeQ8;
#ifdef SWGQA_Q8_NQ
    s.nq = SWGQA_Q8_NQ;
#else
    s.nq = per_kv > 2 ? 4 : 2;
#endif
    s.ntiles = (per_kv + s.nq - 1) / s.nq;
    const int64_t span = std::min<int64_t>(p->sequence_length, (s.nq + group - 1) / group + 1);
    int64_t nkeys = (int64_t)p->local_window_size + span - 1;
    if (nkeys > p->total_sequence_length) nkeys = p->total_sequence_length;
    const int64_t base = (int64_t)p->batch_size * p->kv_num_heads * s.ntiles;
    if (base >= kWholeSliceMinTiles || nkeys <= kWholeSliceMaxKeys) {
      const int64_t slices = (int64_t)p->batch_size * p->kv_num_heads;
      if (s.nq > 2 && slices * s.ntiles < kDecodeMinWorkgroups) {
        s.nq = 2;
        s.ntiles = (per_kv + s.nq - 1) / s.nq;
      }
      const int sr = decode_q8_stage_rows(p->head_size, s.nq);
      const int64_t stages = (nkeys + sr - 1) / sr;
      s.nsplit = 1;
      s.waves = stages <= 4 ? 4 : 8;
      return s;
    }
    int64_t ns = base > 0 ? (kTargetWorkgroups + base - 1) / base : 1;
    const int64_t ns_max = (nkeys + kMinKeysPerSplit - 1) / kMinKeysPerSplit;
    if (ns > ns_max) ns = ns_max;
    if (ns < 1) ns = 1;
    s.nsplit = (int)ns;
    return s;
  }
  if (multi_token && chunk_kernel_supports(p->dtype, p->head_size) &&
      (p->total_sequence_length >= 8 || p->kv_cache_type != 0)) {
    // multi-token step on the matrix cores (its bias reads take rows of at
    // least 8 entries; an 8-bit cache has no other kernel for steps of 16 or
    // more tokens, and with a shorter total none of their items is valid)
    s.kind = Kind::kChunk;
    // 8-wave workgroups (128 query rows) once a KV head has that many rows:
    // twice the matrix work per staged K/V block
    s.waves = per_kv >= kChunkWideRows ? 8 : 4;
    // at most 32 rows per KV head (short steps: verify, small groups): 8
    // waves in 4 groups of 2 that take turns over the split's blocks
    if (kChunkGroups && per_kv <= 32 && p->dtype != SWGQA_F32 && p->kv_cache_type == 0 &&
        p->head_size * 2 <= 256) {
      s.waves = 8;
      s.groups = 4;
    }
    s.nq = chunk_rows_per_workgroup(s.waves, s.groups);
    s.ntiles = (per_kv + s.nq - 1) / s.nq;
    const int64_t span = std::min<int64_t>(p->sequence_length, (s.nq + group - 1) / group + 1);
    int64_t nkeys = (int64_t)p->local_window_size + span - 1;
    if (nkeys > p->total_sequence_length) nkeys = p->total_sequence_length;
    const int64_t base = (int64_t)p->batch_size * p->kv_num_heads * s.ntiles;
    int64_t ns = base >= kChunkMinWorkgroups ? 1 : (kChunkMinWorkgroups + base - 1) / base;
    const int64_t ns_max = (nkeys + 4 * chunk_keys_per_block() - 1) / (4 * chunk_keys_per_block());
    if (ns > ns_max) ns = ns_max;
    if (ns < 1) ns = 1;
    // splits take whole blocks, ceil(nkeys / ns) rounded up to a block: as
    // many splits as that covers the band with (the rest would be empty
    // workgroups whose partials the merge still reads)
    const int64_t bn = chunk_keys_per_block();
    const int64_t per = ((nkeys + ns - 1) / ns + bn - 1) / bn * bn;
    ns = (nkeys + per - 1) / per;
    s.nsplit = ns < 1 ? 1 : (int)ns;
    return s;
  }
  int nq = 2;
  while (nq < per_kv && nq < 16) nq *= 2;
  // the staged kernel keeps NQ x (elements per 16 bytes) accumulators per lane
  int nq_staged = nq;
  while (nq_staged > 2 && nq_staged * (p->dtype == SWGQA_F32 ? 4 : 8) > 64) nq_staged /= 2;
  s.kind = decode_kernel_supports(p->dtype, p->head_size, nq_staged) ? Kind::kDecode : Kind::kSplit;
  if (s.kind == Kind::kDecode) {
    nq = nq_staged;
  } else {
    while (nq > 2 && nq * p->head_size > kSplitMaxTileElems) nq /= 2;
  }
  s.nq = nq;
  s.ntiles = (per_kv + nq - 1) / nq;
  // key rows a tile can touch: the window of its first position plus the
  // positions it spans
  const int64_t span = std::min<int64_t>(p->sequence_length, (nq + group - 1) / group + 1);
  int64_t nkeys = (int64_t)p->local_window_size + span - 1;
  if (nkeys > p->total_sequence_length) nkeys = p->total_sequence_length;
  const int64_t base = (int64_t)p->batch_size * p->kv_num_heads * s.ntiles;
  if (s.kind == Kind::kDecode && (base >= kWholeSliceMinTiles || nkeys <= kWholeSliceMaxKeys)) {
    // enough tiles to fill the chip with one workgroup each, or a window
    // short enough for one workgroup: no key split, no merge pass, and the
    // in-place write-back stays inside the kernel
    const int64_t slices = (int64_t)p->batch_size * p->kv_num_heads;
    while (s.nq > 2 && slices * s.ntiles < kDecodeMinWorkgroups) {
      // narrower tiles: more workgroups, each with less work per key row
      s.nq /= 2;
      s.ntiles = (per_kv + s.nq - 1) / s.nq;
    }
    const int64_t stages =
        (nkeys + decode_stage_rows(p->dtype, p->head_size, s.nq) - 1) /
        decode_stage_rows(p->dtype, p->head_size, s.nq);
    s.nsplit = 1;
    s.waves = stages <= 4 ? 4 : 8;
    return s;
  }
  int64_t ns = base > 0 ? (kTargetWorkgroups + base - 1) / base : 1;
  const int64_t ns_max = (nkeys + kMinKeysPerSplit - 1) / kMinKeysPerSplit;
  if (ns > ns_max) ns = ns_max;
  if (ns < 1) ns = 1;
  s.nsplit = (int)ns;
  return s;
}

size_t partial_bytes(const swgqa_params* p, const SplitPlan& s) {
  if (s.nsplit <= 1) return 0;
  const size_t rows = (size_t)p->batch_size * p->sequence_length * p->num_heads * s.nsplit;
  return rows * (size_t)p->head_size * 4 + rows * 2 * 4;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Rows per (item, KV head, key split, K|V) that the chunk kernel's key
// splits set aside when they move a compacting step's surviving rows
// themselves (one query tile per slice, a 16-bit cache in the element type):
// the step's largest shift -- a multiple of the gap G = C - W + 1 no larger
// than G - 1 + S, since a step keeps at least W rows once T > C -- capped at
// kStashRows; 0 when no shift fits (every step's move is then the step
// tail's).
int chunk_stash_rows(const swgqa_params* p, const SplitPlan& s) {
  if (s.kind != Kind::kChunk || p->kv_cache_type != 0 || s.ntiles != 1 || s.nsplit <= 1 ||
      !chunk_kernel_moves_rows(p->dtype))
    return 0;
  const int64_t G = (int64_t)p->capacity - p->local_window_size + 1;
  if (G > kStashRows) return 0;
  const int64_t most = (G - 1 + p->sequence_length) / G * G;
  return (int)std::min<int64_t>(most, kStashRows);
}

size_t stash_bytes(const swgqa_params* p, const SplitPlan& s) {
  return (size_t)p->batch_size * p->kv_num_heads * s.nsplit * 2 * chunk_stash_rows(p, s) *
         p->head_size * elem_bytes(p->dtype);
}

// Start of the scratch after the header, the split partials and the stash.
size_t scratch_start(const swgqa_params* p, const SplitPlan& s) {
  return kHeaderBytes + align256(partial_bytes(p, s)) + align256(stash_bytes(p, s));
}

// Rotary scratch (after the partials and the stash): rotated query rows,
// rotated key rows, per-item lengths.
struct RotaryScratch {
  size_t q_off, k_off, seq_off, end;
  size_t kq_off, vq_off;  // int8 codes of the new rows (chunk kernel over an int8 cache)
};

RotaryScratch rotary_scratch(const swgqa_params* p, size_t start, const SplitPlan& s) {
  RotaryScratch r{start, start, start, start, start, start};
  if (p->kv_cache_type != 0 && s.kind == Kind::kChunk) {
    const size_t n = (size_t)p->batch_size * p->sequence_length * p->kv_num_heads * p->head_size;
    r.kq_off = start;
    r.vq_off = r.kq_off + align256(n);
    start = r.vq_off + align256(n);
    r.q_off = r.k_off = r.seq_off = r.end = start;
  }
  if (!p->do_rotary) return r;
  const size_t e = elem_bytes(p->dtype);
  const size_t rows = (size_t)p->batch_size * p->sequence_length;
  r.q_off = start;
  r.k_off = r.q_off + align256(rows * p->num_heads * p->head_size * e);
  r.seq_off = r.k_off + align256(rows * p->kv_num_heads * p->head_size * e);
  r.end = r.seq_off + align256((size_t)p->batch_size * 4);
  return r;
}


bool ranges_partially_overlap(const void* a, const void* b, size_t n) {
  const char* x = (const char*)a;
  const char* y = (const char*)b;
  if (x == y) return false;
  return x < y + n && y < x + n;
}

size_t workspace_bytes_for(const swgqa_params* p) {
  if (validate(p) != SWGQA_OK) return 0;
  const SplitPlan s = plan_split(p);
  return rotary_scratch(p, scratch_start(p, s), s).end;
}

// Workspace of swgqa_forward_noalloc: 32 MiB, enough for every workload
// measured here (the largest, multi-token steps with key splits, needs
// about 22 MB).
constexpr size_t kScratchBytes = (size_t)32 << 20;

}  // namespace

// The workspace of swgqa_forward_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never uses this name as an
// address; it uses what hipGetSymbolAddress returns on each device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// One step with a given workspace; device item errors set bits in
// *status_word (the workspace's first word, or a word of the caller's).
swgqa_status forward_impl(const swgqa_params* p, const void* query, const void* key,
                          const void* value, const void* past_key, const void* past_value,
                          const int32_t* seqlens_k, const void* attention_bias,
                          const void* head_sink, const void* cos_cache, const void* sin_cache,
                          const int64_t* position_ids, void* output, void* present_key,
                          void* present_value, void* workspace, size_t workspace_bytes,
                          uint32_t* status_word, void* stream) {
  const swgqa_status v = validate(p);
  if (v != SWGQA_OK) return v;
  if (p->batch_size == 0) return SWGQA_OK;
  if (!query || !key || !value || !past_key || !past_value || !seqlens_k || !output ||
      !present_key || !present_value || !workspace)
    return SWGQA_ERR_ARG;
  const size_t e = elem_bytes(p->dtype);
  const size_t ce = p->kv_cache_type != 0 ? 1 : e;  // cache element bytes
  const size_t cache_bytes =
      (size_t)p->batch_size * p->kv_num_heads * p->capacity * p->head_size * ce;
  if (ranges_partially_overlap(past_key, present_key, cache_bytes) ||
      ranges_partially_overlap(past_value, present_value, cache_bytes))
    return SWGQA_ERR_ALIAS;
  if (((uintptr_t)workspace & 255u) != 0) return SWGQA_ERR_ARG;
  // every 16-byte row access below needs 16-byte aligned rows
  const uintptr_t align_or = (uintptr_t)query | (uintptr_t)key | (uintptr_t)value |
                             (uintptr_t)past_key | (uintptr_t)past_value |
                             (uintptr_t)present_key | (uintptr_t)present_value |
                             (uintptr_t)output;
  if (align_or & 15u) return SWGQA_ERR_ARG;

  const SplitPlan s = plan_split(p);
  const RotaryScratch rs = rotary_scratch(p, scratch_start(p, s), s);
  if (workspace_bytes < rs.end) return SWGQA_ERR_ARG;
  if (p->do_rotary && (!cos_cache || !sin_cache)) return SWGQA_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  // Rotary embedding runs inside the staged decode kernel where it can (row
  // chunks of 16 bytes, 16-byte aligned tables, the new rows of a slice no
  // more than one per thread), else as a pass of its own before attention.
  const bool rot_fused =
      p->do_rotary && s.kind == Kind::kDecode && p->sequence_length <= 16 &&
      decode_rotary_supports(p->dtype, p->head_size, s.nq) &&
      (size_t)p->sequence_length * (p->head_size * e / 16) <= 256 &&
      (((uintptr_t)cos_cache | (uintptr_t)sin_cache) & 15u) == 0;
  if (p->do_rotary && !rot_fused) {
    // rotated rows and the per-item lengths every later kernel reads
    RotaryArgs r;
    r.q = query;
    r.k = key;
    r.q_out = (char*)workspace + rs.q_off;
    r.k_out = (char*)workspace + rs.k_off;
    r.cos_cache = cos_cache;
    r.sin_cache = sin_cache;
    r.position_ids = position_ids;
    r.seqlens = seqlens_k;
    r.seqlens_out = (int32_t*)((char*)workspace + rs.seq_off);
    r.B = p->batch_size;
    r.S = p->sequence_length;
    r.Hq = p->num_heads;
    r.Hkv = p->kv_num_heads;
    r.D = p->head_size;
    r.rows = p->rotary_cache_rows;
    r.interleaved = p->rotary_interleaved;
    if (launch_rotary(p->dtype, r, st) != hipSuccess) return SWGQA_ERR_HIP;
    query = r.q_out;
    key = r.k_out;
    seqlens_k = r.seqlens_out;
  }
  const bool shared = present_key == past_key && present_value == past_value;
  // int8 cache on the matrix-core kernel: the new rows as codes first
  const bool chunk_q8 = p->kv_cache_type != 0 && s.kind == Kind::kChunk;
  const int ct = p->kv_cache_type == 2 ? kCodeFp8 : kCodeInt8;  // code type, if quantized
  const void* key_rows = key;    // the new rows as the element type (rotated)
  const void* value_rows = value;
  if (chunk_q8) {
    uint8_t* kq = (uint8_t*)workspace + rs.kq_off;
    uint8_t* vq = (uint8_t*)workspace + rs.vq_off;
    const size_t n = (size_t)p->batch_size * p->sequence_length * p->kv_num_heads * p->head_size;
    if (launch_quant_rows(p->dtype, ct, key, value, kq, vq, n, p->k_scale, p->v_scale, st) !=
        hipSuccess)
      return SWGQA_ERR_HIP;
    key = kq;
    value = vq;
  }

  AttnArgs a;
  a.q = query;
  a.k = key;
  a.v = value;
  a.past_k = past_key;
  a.past_v = past_value;
  a.seqlens = seqlens_k;
  a.bias = attention_bias;
  a.sink = head_sink;
  a.smooth = p->smooth_softmax;
  a.out = output;
  a.status = status_word;
  a.slice_counters = (uint32_t*)((char*)workspace + kStatusBytes);
  float* part = (float*)((char*)workspace + kHeaderBytes);
  a.opart = part;
  a.ml = part + (size_t)p->batch_size * p->sequence_length * p->num_heads * s.nsplit *
                    p->head_size;
  a.present_k = shared ? present_key : nullptr;
  a.present_v = shared ? present_value : nullptr;
  a.stash_rows = shared ? chunk_stash_rows(p, s) : 0;
  a.stash = a.stash_rows > 0 ? (char*)workspace + kHeaderBytes + align256(partial_bytes(p, s))
                             : nullptr;
  a.B = p->batch_size;
  a.S = p->sequence_length;
  a.Hq = p->num_heads;
  a.Hkv = p->kv_num_heads;
  a.C = p->capacity;
  a.W = p->local_window_size;
  a.total = p->total_sequence_length;
  a.group = p->num_heads / p->kv_num_heads;
  a.gdiv = make_gap_div((uint32_t)(p->capacity - p->local_window_size + 1));
  a.ntiles = s.ntiles;
  a.nsplit = s.nsplit;
  a.tdiv = make_gap_div((uint32_t)(s.ntiles * s.nsplit));
  a.hdiv = make_gap_div((uint32_t)p->kv_num_heads);
  a.sdiv = make_gap_div((uint32_t)s.nsplit);
  a.qdiv = make_gap_div((uint32_t)(p->num_heads / p->kv_num_heads));
  a.scale = p->scale > 0.0f ? p->scale : 1.0f / sqrtf((float)p->head_size);
  a.softcap = p->softcap;
  a.inv_softcap = p->softcap > 0.0f ? 1.0f / p->softcap : 0.0f;
  a.bias_b = p->bias_dim0_is_batch ? 1 : 0;
  a.bias_h = p->bias_dim1_is_heads ? 1 : 0;
  // in-kernel write-back: one workgroup per slice, or (staged decode) the
  // last query tile of each slice, tracked by a counter
  const bool counted = (s.kind == Kind::kDecode || s.kind == Kind::kDecodeQ8) &&
                       (int64_t)p->batch_size * p->kv_num_heads <= kMaxSliceCounters;
  a.fuse_writeback = (shared && s.nsplit == 1 && (s.ntiles == 1 || counted)) ? 1 : 0;
  a.waves = s.waves;
  a.chunk_groups = s.groups;
  // long-gap compactions on the staged kernel, one 8-wave workgroup per
  // slice (every shift at least one round of the 8 waves' stages); the 8-bit
  // kernel keeps the move after attention (measured no faster with it fused)
  {
    const int64_t gap = (int64_t)p->capacity - p->local_window_size + 1;
    const bool staged = s.kind == Kind::kDecode && !rot_fused;
    const int sr = staged ? decode_stage_rows(p->dtype, p->head_size, s.nq) : 0;
    a.fused_move = (staged && a.fuse_writeback && s.ntiles == 1 && s.nsplit == 1 &&
                    s.waves == 8 && sr > 0 && gap >= 8 * (int64_t)sr)
                       ? 1 : 0;
  }
  // What the attention kernel does not finish -- the merge of key splits, the
  // write-back when it is not done in the attention kernel -- runs in one
  // more launch, after every read.
  const bool merge = s.nsplit > 1;
  const bool writeback = !a.fuse_writeback;
  a.k_scale = p->k_scale;
  a.v_scale = p->v_scale;
  a.rot_cos = a.rot_sin = nullptr;
  a.rot_pos = nullptr;
  a.rot_rows = a.rot_interleaved = 0;
  a.k_rot = nullptr;
  a.seqlens_out = nullptr;
  if (rot_fused) {
    a.rot_cos = cos_cache;
    a.rot_sin = sin_cache;
    a.rot_pos = position_ids;
    a.rot_rows = p->rotary_cache_rows;
    a.rot_interleaved = p->rotary_interleaved;
    if (writeback) a.k_rot = (char*)workspace + rs.k_off;
    if (merge || writeback) a.seqlens_out = (int32_t*)((char*)workspace + rs.seq_off);
  }

  const hipError_t ea =
      s.kind == Kind::kChunk
          ? (!chunk_q8          ? launch_attn_chunk(p->dtype, p->head_size, a, st)
             : ct == kCodeFp8   ? launch_attn_chunk_f8(p->dtype, p->head_size, a, st)
                                : launch_attn_chunk_q8(p->dtype, p->head_size, a, st))
      : s.kind == Kind::kDecodeQ8
          ? (ct == kCodeFp8 ? launch_attn_decode_f8(p->dtype, p->head_size, s.nq, a, st)
                            : launch_attn_decode_q8(p->dtype, p->head_size, s.nq, a, st))
      : s.kind == Kind::kDecode
          ? (rot_fused ? launch_attn_decode_rot(p->dtype, p->head_size, s.nq, a, st)
                       : launch_attn_decode(p->dtype, p->head_size, s.nq, a, st))
                                : launch_attn_split(p->dtype, p->head_size, s.nq, a, st);
  if (ea != hipSuccess) return SWGQA_ERR_HIP;
  if (!merge && !writeback) return SWGQA_OK;
  // with fused rotary the tail reads the rotated keys and the lengths with
  // the position verdict that the attention kernel wrote
  AttnArgs at = a;
  if (rot_fused) at.seqlens = a.seqlens_out;

  CopyArgs c;
  c.past_k = past_key;
  c.past_v = past_value;
  c.k = rot_fused ? a.k_rot : key_rows;  // element-type rows (quantized as written)
  c.v = value_rows;
  c.present_k = present_key;
  c.present_v = present_value;
  c.seqlens = rot_fused ? a.seqlens_out : seqlens_k;
  c.B = p->batch_size;
  c.S = p->sequence_length;
  c.Hkv = p->kv_num_heads;
  c.C = p->capacity;
  c.W = p->local_window_size;
  c.total = p->total_sequence_length;
  c.gdiv = a.gdiv;
  c.D = p->head_size;
  c.elem_bytes = (int32_t)ce;
  c.quant = p->kv_cache_type != 0 ? ct : 0;
  c.src_elem_bytes = (int32_t)e;
  c.dtype = p->dtype;
  c.k_scale = p->k_scale;
  c.v_scale = p->v_scale;
  c.skip_drifting = shared ? 1 : 0;  // drifting appends were done by attention
  if (launch_step_tail(p->dtype, at, c, merge, writeback, st) != hipSuccess) return SWGQA_ERR_HIP;
  return SWGQA_OK;
}

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// The current device's scratch address; on its first use on a device the
// header (status word and slice counters, which must start at zero) is
// cleared with a fill kernel on `st`.
hipError_t device_scratch(void** out, hipStream_t st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr || ((uintptr_t)ptr & 255u) != 0) return hipErrorInvalidSymbol;
    e = launch_zero_words((uint32_t*)ptr, kHeaderBytes / 4, st);
    if (e != hipSuccess) return e;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t swgqa_workspace_size(const swgqa_params* p) { return workspace_bytes_for(p); }

swgqa_status swgqa_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes < kHeaderBytes) return SWGQA_ERR_ARG;
  if (launch_zero_words((uint32_t*)workspace, workspace_bytes / 4, (hipStream_t)stream) !=
      hipSuccess)
    return SWGQA_ERR_HIP;
  return SWGQA_OK;
}

swgqa_status swgqa_forward(const swgqa_params* p, const void* query, const void* key,
                           const void* value, const void* past_key,
                           const void* past_value, const int32_t* seqlens_k,
                           const void* attention_bias, const void* head_sink,
                           const void* cos_cache, const void* sin_cache,
                           const int64_t* position_ids, void* output,
                           void* present_key, void* present_value, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return forward_impl(p, query, key, value, past_key, past_value, seqlens_k, attention_bias,
                      head_sink, cos_cache, sin_cache, position_ids, output, present_key,
                      present_value, workspace, workspace_bytes, (uint32_t*)workspace, stream);
}

swgqa_status swgqa_forward_noalloc(const swgqa_params* p, const void* query, const void* key,
                                   const void* value, const void* past_key,
                                   const void* past_value, const int32_t* seqlens_k,
                                   const void* attention_bias, const void* head_sink,
                                   const void* cos_cache, const void* sin_cache,
                                   const int64_t* position_ids, void* output,
                                   void* present_key, void* present_value,
                                   uint32_t* device_status, void* stream) {
  const swgqa_status v = validate(p);
  if (v != SWGQA_OK) return v;
  if (p->batch_size == 0) return SWGQA_OK;
  const size_t need = workspace_bytes_for(p);
  if (need > kScratchBytes) return SWGQA_ERR_SCRATCH;
  if (((uintptr_t)device_status & 3u) != 0) return SWGQA_ERR_ARG;
  void* ws = nullptr;
  if (device_scratch(&ws, (hipStream_t)stream) != hipSuccess) return SWGQA_ERR_HIP;
  return forward_impl(p, query, key, value, past_key, past_value, seqlens_k, attention_bias,
                      head_sink, cos_cache, sin_cache, position_ids, output, present_key,
                      present_value, ws, kScratchBytes,
                      device_status ? device_status : (uint32_t*)ws, stream);
}

swgqa_status swgqa_plan(const swgqa_params* p, const int32_t* seqlens_k,
                        swgqa_plan_entry* plan_out, void* stream) {
  const swgqa_status v = validate(p);
  if (v != SWGQA_OK) return v;
  if (p->batch_size == 0) return SWGQA_OK;
  if (!seqlens_k || !plan_out) return SWGQA_ERR_ARG;
  if (launch_plan(seqlens_k, p->batch_size, p->sequence_length, p->capacity,
                  p->local_window_size, p->total_sequence_length, (int64_t*)plan_out,
                  (hipStream_t)stream) != hipSuccess)
    return SWGQA_ERR_HIP;
  return SWGQA_OK;
}

int64_t swgqa_resident_length(int64_t T, int64_t C, int64_t W) {
  if (W < 1 || C < W || T < 0) return -1;
  // the kernels' form (multiply-shift division by the gap) wherever it
  // applies, so host tests exercise it
  if (T <= ((int64_t)1 << 31) && C < ((int64_t)1 << 31))
    return resident_len_step(T, (int32_t)C, make_gap_div((uint32_t)(C - W + 1)));
  return resident_len(T, C, W);
}

int swgqa_rollback_exact(int64_t T, int64_t k, int64_t C, int64_t W) {
  if (W < 1 || C < W || T < 0 || k < 0 || k > T) return 0;
  return resident_len(T - k, C, W) == resident_len(T, C, W) - k ? 1 : 0;
}

swgqa_status swgqa_device_status(const void* workspace, int clear, void* stream) {
  if (!workspace) return SWGQA_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  uint32_t word = 0;
  if (hipMemcpyAsync(&word, workspace, sizeof word, hipMemcpyDeviceToHost, st) != hipSuccess)
    return SWGQA_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return SWGQA_ERR_HIP;
  if (clear) {
    if (launch_zero_words((uint32_t*)workspace, 1, st) != hipSuccess) return SWGQA_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return SWGQA_ERR_HIP;
  }
  return (word & kStatusBadItem) ? SWGQA_ERR_DEVICE_INPUT : SWGQA_OK;
}

const char* swgqa_status_string(swgqa_status s) {
  switch (s) {
    case SWGQA_OK: return "ok";
    case SWGQA_ERR_ARG: return "invalid argument";
    case SWGQA_ERR_UNSUPPORTED: return "unsupported head size or element type";
    case SWGQA_ERR_ALIAS: return "past and present buffers overlap partially";
    case SWGQA_ERR_DEVICE_INPUT: return "seqlens_k out of range for some item";
    case SWGQA_ERR_HIP: return "HIP runtime error";
    case SWGQA_ERR_SCRATCH: return "step needs more workspace than the library's static scratch";
  }
  return "unknown status";
}

}  // extern "C"
