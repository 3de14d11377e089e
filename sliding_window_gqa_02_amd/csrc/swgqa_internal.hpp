// swgqa_internal.hpp -- launch interface between the C ABI (swgqa_api.hip)
// and the kernels.  Internal to libswgqa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swgqa_common.hpp"

namespace swgqa {

// Arguments shared by the attention kernels.  Pointers are device pointers;
// layouts as in include/swgqa.h.
struct AttnArgs {
  const void* q;
  const void* k;        // new rows (B, S, Hkv*D)
  const void* v;
  const void* past_k;   // (B, Hkv, C, D)
  const void* past_v;
  const int32_t* seqlens;
  const void* bias;     // NULL or (B|1, Hq|1, S, total)
  void* out;            // (B, S, Hq*D)
  float* opart;         // split partial accumulators (rows of D floats)
  float* ml;            // split partial (max, sum) pairs, log2 domain
  uint32_t* status;
  // per-slice arrival counters for the in-kernel write-back of multi-tile
  // launches (zero between calls)
  uint32_t* slice_counters;
  // fused append on drifting steps (shared buffer only; may be NULL)
  void* present_k;
  void* present_v;
  int32_t B, S, Hq, Hkv, C, W, total, group;
  GapDiv gdiv;  // division by the gap C - W + 1
  GapDiv tdiv;  // division by ntiles * nsplit (work items per slice)
  GapDiv hdiv;  // division by Hkv
  GapDiv sdiv;  // division by nsplit
  GapDiv qdiv;  // division by group (query heads per KV head)
  int32_t ntiles, nsplit;
  float scale, softcap;
  float inv_softcap;  // 1 / softcap (binary32 quotient), or 0 without softcap
  int32_t bias_b, bias_h;
  // softmax sink: head_sink (Hq elements) or, with smooth != 0 and no
  // head_sink, a logit of 0; it joins the denominator with a zero value row
  const void* sink;
  int32_t smooth;
  int32_t fuse_writeback;  // shared buffer, one key split: write-back in the kernel
  int32_t waves;           // waves per workgroup of the staged kernel
  int32_t chunk_groups;    // chunk kernel: groups of waves that share a tile's rows (1 or 4)
  // staged decode kernel, 8 waves, one workgroup per slice: the variant that
  // moves a compacting slice's surviving rows as it reads them
  int32_t fused_move;
  // rotary embedding fused into the staged decode kernel (rot_cos non-NULL):
  // tables (rot_rows, D/2), 16-byte aligned; positions (B, S) or NULL (P + i)
  const void* rot_cos;
  const void* rot_sin;
  const int64_t* rot_pos;
  int32_t rot_rows, rot_interleaved;
  void* k_rot;             // rotated new keys (B, S, Hkv*D) for the step tail, or NULL
  int32_t* seqlens_out;    // per-item lengths for the step tail (-2: bad position), or NULL
  // int8 cache (the int8 decode kernel): element = code * scale
  float k_scale, v_scale;
  // 16-bit chunk kernel, key splits over one query tile per slice, shared
  // buffer (else NULL): on compacting steps whose surviving rows all lie in
  // the key band and whose shift is at most stash_rows, the split that reads
  // a surviving row stores it at its new place -- except rows whose new place
  // lies in an earlier split's part, which go here, (item, KV head, split,
  // K|V, stash_rows rows), for the step tail to store
  void* stash;
  int32_t stash_rows;
};

// Keys per LDS block of the chunk kernel.
constexpr int kChunkBlockKeys = 32;
// Largest stash_rows (rows set aside per item, KV head, key split and K|V).
constexpr int kStashRows = 64;

struct CopyArgs {
  const void* past_k;
  const void* past_v;
  const void* k;
  const void* v;
  void* present_k;
  void* present_v;
  const int32_t* seqlens;
  int32_t B, S, Hkv, C, W, total, D;
  GapDiv gdiv;
  int32_t elem_bytes;     // cache element bytes (1 for int8 codes)
  int32_t skip_drifting;  // shared buffer and the append already fused
  // quantized cache: new rows (element type, src_elem_bytes each) are
  // quantized with k_scale / v_scale as they are written; quant is the code
  // type (kCodeInt8, kCodeFp8) or 0
  int32_t quant;
  int32_t src_elem_bytes;
  int32_t dtype;
  float k_scale, v_scale;
};

// Rotary pass (swgqa_rotary.hip): rotates q (B,S,Hq,D) and k (B,S,Hkv,D)
// into q_out / k_out and writes the per-item lengths the step reads.
struct RotaryArgs {
  const void* q;
  const void* k;
  void* q_out;
  void* k_out;
  const void* cos_cache;
  const void* sin_cache;
  const int64_t* position_ids;  // (B, S) or NULL (then P + i)
  const int32_t* seqlens;
  int32_t* seqlens_out;         // seqlens, or -2 for items with bad positions
  int32_t B, S, Hq, Hkv, D, rows, interleaved;
};
hipError_t launch_rotary(int dtype, const RotaryArgs& r, hipStream_t stream);

// Split-K attention for short steps; returns hipSuccess or the launch error.
hipError_t launch_attn_split(int dtype, int D, int nq, const AttnArgs& a,
                             hipStream_t stream);
// MFMA kernel for multi-token steps (swgqa_attn_chunk.hip): 16 query rows
// per wave, 4 or 8 waves per workgroup, keys in blocks of 32.
bool chunk_kernel_supports(int dtype, int D);
int chunk_rows_per_workgroup(int waves, int groups);  // 4 or 8 waves, 1 or 4 groups
int chunk_keys_per_block();
// Whether the kernel (cache in the element type) honours AttnArgs::stash.
bool chunk_kernel_moves_rows(int dtype);
hipError_t launch_attn_chunk(int dtype, int D, const AttnArgs& a, hipStream_t stream);
// The same kernel over an int8 / fp8 E4M3 cache (swgqa_attn_chunk_q8.hip,
// swgqa_attn_chunk_f8.hip); a.k / a.v hold the step's new rows as codes
// (launch_quant_rows).
hipError_t launch_attn_chunk_q8(int dtype, int D, const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_chunk_f8(int dtype, int D, const AttnArgs& a, hipStream_t stream);
// Codes (code type ct: kCodeInt8 / kCodeFp8) of n elements of k and v
// (element type dtype), n % 4 == 0.
hipError_t launch_quant_rows(int dtype, int ct, const void* k, const void* v, uint8_t* kq,
                             uint8_t* vq, size_t n, float k_scale, float v_scale,
                             hipStream_t stream);
// Staged decode kernel (swgqa_attn_decode.hip): supports row sizes up to
// 256 bytes and NQ * (16 / element bytes) <= 64.
bool decode_kernel_supports(int dtype, int D, int nq);
// Key rows one wave of the staged decode kernel takes per stage.
int decode_stage_rows(int dtype, int D, int nq);
hipError_t launch_attn_decode(int dtype, int D, int nq, const AttnArgs& a,
                              hipStream_t stream);
// Staged decode kernel for an int8 cache (swgqa_attn_decode_q8.hip): head
// sizes 16..256, query tiles of 2 or 4 pairs, S < 16.
bool decode_q8_supports(int D, int nq);
// New rows per step the 8-bit staged kernel holds in LDS: the quantized new
// rows of a step of at most this many tokens.
constexpr int kQ8MaxNewRows = 16;
int decode_q8_stage_rows(int D, int nq);
hipError_t launch_attn_decode_q8(int dtype, int D, int nq, const AttnArgs& a,
                                 hipStream_t stream);
// The same kernel for fp8 E4M3 caches (swgqa_attn_decode_f8.hip).
hipError_t launch_attn_decode_f8(int dtype, int D, int nq, const AttnArgs& a,
                                 hipStream_t stream);
// The same kernel with rotary embedding fused in (head sizes 32, 64, 128).
bool decode_rotary_supports(int dtype, int D, int nq);
hipError_t launch_attn_decode_rot(int dtype, int D, int nq, const AttnArgs& a,
                                  hipStream_t stream);
// Split merge and/or cache write-back after the attention kernel, one launch.
hipError_t launch_step_tail(int dtype, const AttnArgs& a, const CopyArgs& c, bool merge,
                            bool writeback, hipStream_t stream);
hipError_t launch_plan(const int32_t* seqlens, int32_t B, int32_t S, int32_t C,
                       int32_t W, int32_t total, int64_t* out, hipStream_t stream);
hipError_t launch_zero_words(uint32_t* words, size_t n, hipStream_t stream);

// Supported head sizes of every kernel.
bool head_size_supported(int D);

// The split kernel's query tile holds NQ (position, head) pairs, NQ in
// {2, 4, 8, 16}, with NQ * D <= kSplitMaxTileElems.
constexpr int kSplitMaxTileElems = 2048;

}  // namespace swgqa
