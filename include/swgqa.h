/*
 * swgqa.h -- C ABI of libswgqa: one GroupQueryAttention step over a windowed
 * (sliding-window) KV cache on an AMD Instinct MI355X (gfx950).
 *
 * The operation is the one the pages define:
 *  - "Specify GroupQueryAttention windowed KV cache layout contract"
 *    (onnxruntime PR #32419), Description: with capacity C (dimension 2 of
 *    past_key), window W = local_window_size, total length T and gap
 *    G = C - W + 1, the resident length is L(T) = T for T <= C and
 *    T - G*ceil((T - C)/G) otherwise.  After a step, present row i of a
 *    slice, 0 <= i < L(T), holds absolute position T - L(T) + i; the content
 *    of rows L(T) .. C-1 is not defined.  S may be any value >= 1 (S > C
 *    too), and the last dimension of attention_bias (total_sequence_length)
 *    indexes absolute key positions.
 *  - "[CPU] Add windowed kv cache for GQA" (onnxruntime PR #31142), key design
 *    decisions: block (gap-sized) eviction, compaction skipped on drifting
 *    steps, staging of multi-token steps that would evict history their
 *    first query reads.  Results equal those of a full-length cache.
 *  - "GQA In-Place KV Cache: Investigation Report" (onnxruntime/mobius issue
 *    #111), sections 1.1-1.3: inputs query/key/value, past/present in BNSH,
 *    seqlens_k = total length - 1 per item, total_sequence_length, the
 *    shared-buffer and separate-buffer modes, attributes num_heads,
 *    kv_num_heads, scale (default 1/sqrt(head_size)), local_window_size,
 *    softcap, smooth_softmax, and the optional input head_sink (one value
 *    per query head).
 *  - "Fix CPU Attention causal mask for q_len=1 with past_key and kv_len > 1"
 *    (onnxruntime PR #34226), Description: query i sees key j iff
 *    j <= i + past_sequence_length.
 *
 * Semantics of one step, item b (P = seqlens_k[b] + 1 - S):
 *  - query i (absolute position p = P + i) attends to keys at absolute
 *    positions j with p - W < j <= p (W keys including itself), over the
 *    logical concatenation of the resident rows and the S new rows;
 *  - score = scale * q.k, then softcap*tanh(score/softcap) when softcap > 0,
 *    then + attention_bias[b|0][h|0][i][j]; softmax; weighted sum of V;
 *  - rotary embedding (do_rotary): before attention and before they are
 *    stored, query and new key rows are rotated pairwise -- elements
 *    (k, k + D/2), or (2k, 2k + 1) with rotary_interleaved -- the pair (a, b)
 *    at position pos becoming (a c - b s, b c + a s) with c, s =
 *    cos_cache[pos][k], sin_cache[pos][k]; each product, sum and difference
 *    is rounded to binary32, then the result to the element type (the
 *    Investigation Report, sections 1.1 and 1.3, names these inputs and
 *    attributes only; this is the plainest reading).  pos = position_ids[b][i],
 *    or P + i without them; an item with a position outside the caches is
 *    skipped like an item with out-of-range seqlens_k;
 *  - softmax sink: with head_sink given, one more logit head_sink[h] (used
 *    as given: not scaled, capped or biased) joins the softmax denominator
 *    with a zero value row -- out = sum_j e^{s_j} v_j / (e^{sink} +
 *    sum_j e^{s_j}); with smooth_softmax != 0 and no head_sink that logit
 *    is 0 (the Investigation Report, sections 1.1 and 1.3, names head_sink
 *    and smooth_softmax without defining them; this is the plainest reading);
 *  - quantized cache (kv_cache_type 1: int8, 2: fp8 E4M3): past/present
 *    hold 8-bit codes, one scale per tensor (k_scale for keys, v_scale for
 *    values); a cache element stands for value(code) * scale, and a new
 *    element x (after rotary) is stored as the code of the binary32 quotient
 *    x / scale -- int8: rounded to an integer with ties to even, saturated to
 *    [-128, 127], NaN to -128; fp8: OCP E4M3 ("FN": bias 7, no infinities,
 *    0x7F NaN), the nearest value with ties to the even code, magnitudes of
 *    448 or more saturated to 448, NaN to 0x7F, zero results coded +0; the
 *    step attends to every key and value row in that dequantized form, new
 *    rows included (the Investigation Report, section 1.1, names k_scale /
 *    v_scale and a cache type only; this is the plainest reading).  Head
 *    sizes below 16 return SWGQA_ERR_UNSUPPORTED with these caches, and so
 *    do steps of more than 16 tokens with fp32 at head size 256;
 *  - query head h reads KV head h / (num_heads / kv_num_heads);
 *  - present rows [0, L(T)) receive the newest L(T) rows of that
 *    concatenation (byte copies); rows [L(T), C) are unspecified.
 *
 * Ownership and execution: every buffer is allocated by the caller in
 * device memory (seqlens_k too).  The library allocates nothing, never
 * synchronises inside swgqa_forward / swgqa_plan, and enqueues its kernels
 * on `stream` (a hipStream_t passed as void*; NULL = the null stream).
 * Calls on one stream are ordered; calls that share a workspace must not
 * run concurrently.
 *
 * Errors found on the host return a status before anything is enqueued.
 * Errors that depend on device data (seqlens_k[b] + 1 < S, or
 * > total_sequence_length) cannot be returned synchronously: the item is
 * skipped (its output rows are zero-filled, its present rows untouched) and
 * a sticky bit is set in the workspace status word, read with
 * swgqa_device_status.
 */
#ifndef SWGQA_H
#define SWGQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SWGQA_F32 = 0,
  SWGQA_F16 = 1,
  SWGQA_BF16 = 2
} swgqa_dtype;

typedef enum {
  SWGQA_OK = 0,
  SWGQA_ERR_ARG = 1,          /* null pointer, bad size or shape */
  SWGQA_ERR_UNSUPPORTED = 2,  /* valid but not built: head_size, dtype */
  SWGQA_ERR_ALIAS = 3,        /* past and present overlap partially */
  SWGQA_ERR_DEVICE_INPUT = 4, /* some seqlens_k[b] out of range (device) */
  SWGQA_ERR_HIP = 5,          /* a HIP runtime call failed */
  SWGQA_ERR_SCRATCH = 6       /* swgqa_forward_noalloc: the step needs more
                                 workspace than the static scratch holds */
} swgqa_status;

/* Step parameters.  All sizes are element counts. */
typedef struct {
  int32_t batch_size;            /* B >= 0 (0: nothing to do) */
  int32_t sequence_length;       /* S >= 1 new tokens per item */
  int32_t num_heads;             /* Hq >= 1 */
  int32_t kv_num_heads;          /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_size;             /* D: 8, 16, 32, 64, 128 or 256 */
  int32_t capacity;              /* C: dimension 2 of past/present */
  int32_t local_window_size;     /* W: 1 <= W <= C (-1 is rejected) */
  int32_t total_sequence_length; /* >= max_b(seqlens_k[b]+1); bias row stride */
  float scale;                   /* 0 -> 1/sqrt(D) */
  float softcap;                 /* 0 -> disabled, else > 0 */
  int32_t dtype;                 /* swgqa_dtype of every tensor below */
  int32_t bias_dim0_is_batch;    /* bias dim 0: B (1) or 1 (0) */
  int32_t bias_dim1_is_heads;    /* bias dim 1: Hq (1) or 1 (0) */
  int32_t smooth_softmax;        /* 0 or 1: a sink logit of 0 when head_sink is NULL */
  int32_t do_rotary;             /* 0 or 1 */
  int32_t rotary_interleaved;    /* 0: pairs (k, k + D/2); 1: pairs (2k, 2k + 1) */
  int32_t rotary_cache_rows;     /* rows of cos_cache / sin_cache (>= 1 with do_rotary) */
  int32_t kv_cache_type;         /* 0: caches in dtype; 1: int8; 2: fp8 E4M3 codes (see above) */
  float k_scale;                 /* kv_cache_type 1: key element = code * k_scale (> 0) */
  float v_scale;                 /* kv_cache_type 1: value element = code * v_scale (> 0) */
} swgqa_params;

/* Plan record of one item, all int64: T, P, Lb = L(P), La = L(T),
 * kept = La - S (old rows that survive), shift = Lb + S - La (rows evicted
 * this step; 0 on a drifting step), first = T - La (absolute position of
 * row 0 after the step), hazard (1 if compacting before attention would drop
 * history the first query reads; such steps are staged).  Invalid items:
 * all fields -1.  The per-item planner of PR #31142's review thread. */
typedef struct {
  int64_t T, P, Lb, La, kept, shift, first, hazard;
} swgqa_plan_entry;

/* Bytes of device workspace swgqa_forward needs for these parameters: the
 * status word in bytes [0, 4), per-(item, KV head) arrival counters in bytes
 * [256, 16384) that every call leaves at zero, then key-split partials, the
 * rows that multi-token 16-bit steps with key splits set aside while they
 * compact the cache, and, with do_rotary, the rotated query and key rows and
 * the per-item lengths (scratch).  0 if the parameters are invalid.  Pure host function.  A
 * workspace of at least this size serves any parameter set whose own size is
 * not larger. */
size_t swgqa_workspace_size(const swgqa_params* params);

/* Zeroes the first workspace_bytes of the workspace, status word and
 * counters included (enqueued on `stream`; a small kernel, no memset node).
 * Call once on a fresh workspace, before its first swgqa_forward. */
swgqa_status swgqa_workspace_init(void* workspace, size_t workspace_bytes,
                                  void* stream);

/* One windowed GQA step.  Device pointers, row-major, innermost last:
 *   query          (B, S, Hq*D)
 *   key, value     (B, S, Hkv*D)         the S new rows of every item
 *   past_key/value (B, Hkv, C, D)        rows [0, L(P_b)) valid on entry;
 *                                        dtype elements, or 8-bit codes with
 *                                        kv_cache_type 1 / 2
 *   seqlens_k      int32 (B)             total length T_b = seqlens_k[b]+1
 *   attention_bias NULL or (B|1, Hq|1, S, total_sequence_length)
 *   head_sink      NULL or (Hq)          per-head sink logit
 *   cos_cache, sin_cache (rotary_cache_rows, D/2), required with do_rotary
 *   position_ids   NULL or int64 (B, S)  rotary positions (default P + i)
 *   output         (B, S, Hq*D)
 *   present_key/value (B, Hkv, C, D)     == past (shared buffer, in place)
 *                                        or disjoint from it
 *   workspace      >= swgqa_workspace_size(params) bytes, 256-B aligned
 * Returns SWGQA_OK once the work is enqueued. */
swgqa_status swgqa_forward(const swgqa_params* params, const void* query,
                           const void* key, const void* value,
                           const void* past_key, const void* past_value,
                           const int32_t* seqlens_k,
                           const void* attention_bias, const void* head_sink,
                           const void* cos_cache, const void* sin_cache,
                           const int64_t* position_ids, void* output,
                           void* present_key, void* present_value,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/* swgqa_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same step, same kernels, same results
 * as swgqa_forward; its workspace is a static 32 MiB device array inside the
 * library, one per GPU, held until the process ends.  Nothing is allocated.
 *  - Parameters whose swgqa_workspace_size exceeds 32 MiB return
 *    SWGQA_ERR_SCRATCH before anything is enqueued (every workload here
 *    needs at most about 22 MB).
 *  - device_status: NULL, or a 4-byte aligned device word of the caller's
 *    into which device-detected item errors OR the bit that
 *    swgqa_device_status reports (sticky: the caller clears it); with NULL
 *    such errors are visible only as zero-filled outputs.
 *  - The first call on a device looks up the array's address and clears its
 *    counters with a fill kernel on `stream`; make that first call outside
 *    graph capture.
 *  - All calls on one GPU share its array: calls that overlap in time on one
 *    GPU (other streams, other threads) race and must not be issued. */
swgqa_status swgqa_forward_noalloc(const swgqa_params* params, const void* query,
                                   const void* key, const void* value,
                                   const void* past_key, const void* past_value,
                                   const int32_t* seqlens_k,
                                   const void* attention_bias, const void* head_sink,
                                   const void* cos_cache, const void* sin_cache,
                                   const int64_t* position_ids, void* output,
                                   void* present_key, void* present_value,
                                   uint32_t* device_status, void* stream);

/* Enqueues the planner alone: writes B plan records to device memory
 * `plan_out` (B * 64 bytes).  For tests of the resident-range planner. */
swgqa_status swgqa_plan(const swgqa_params* params, const int32_t* seqlens_k,
                        swgqa_plan_entry* plan_out, void* stream);

/* L(T) on the host (PR #32419 Description); -1 if C < W or W < 1 or T < 0. */
int64_t swgqa_resident_length(int64_t T, int64_t C, int64_t W);

/* 1 if rejecting the last k of T tokens needs no cache edit, i.e.
 * L(T-k) == L(T) - k (PR #32419 Description, rollback); else 0. */
int swgqa_rollback_exact(int64_t T, int64_t k, int64_t C, int64_t W);

/* Synchronises `stream`, reads the workspace status word, clears it if
 * `clear` is nonzero.  Returns SWGQA_OK, SWGQA_ERR_DEVICE_INPUT if an
 * invalid item was seen since the last clear, or SWGQA_ERR_HIP. */
swgqa_status swgqa_device_status(const void* workspace, int clear,
                                 void* stream);

/* Static description of a status code. */
const char* swgqa_status_string(swgqa_status status);

#ifdef __cplusplus
}
#endif

#endif /* SWGQA_H */
