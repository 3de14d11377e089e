// swgqa_attn_decode.hpp -- split-K grouped-query attention for short steps
// (decode and small verify steps) over a windowed KV cache, tuned for
// CDNA4's wave64 / LDS / HBM balance.  Instantiated without rotary
// embedding in swgqa_attn_decode.hip and with it in
// swgqa_attn_decode_rot.hip.
//
// Same contract as the generic split kernel (swgqa_attn_split.hip): query i
// of item b at absolute position p = P + i attends to keys p - W < j <= p of
// [resident rows | S new rows], keys below P read from cache row
// j - (P - Lb), the rest from the new rows (no staging copy).
//
// Work of one wave is organised in stages of SR consecutive key rows:
//  A. K rows arrive as 16-byte chunks, LPR lanes per row (coalesced: one load
//     instruction covers RPW whole rows).  Each lane forms partial dot
//     products of its chunk with the NQ queries of the tile (packed dot2 for
//     fp16/bf16) and stores them to LDS -- no cross-lane shuffles.
//  B. One lane per (row, query) pair sums the LPR partials, applies scale,
//     softcap, bias and the causal/window mask once (no redundant
//     transcendental work), takes the stage maximum per query across lanes,
//     and writes p = 2^(s - m) and the rescale factor to LDS.
//  C. The V rows (same lane layout as K) are accumulated with p read back
//     from LDS as a broadcast.
// K and V of the next DEPTH - 1 stages are loaded into further register sets
// before stage n is computed, so their loads are in flight while it is
// (DEPTH = 3: triple buffering).
// LDS traffic is private to the wave and in program order, so phases only
// need compiler ordering fences, not barriers.
//
// With rotary embedding (ROT) the kernel also rotates its inputs (the
// Investigation Report, sections 1.1 and 1.3, name cos_cache / sin_cache,
// position_ids, do_rotary and rotary_interleaved; the pair (a, b) at position
// pos becomes (a c - b s, b c + a s) with c, s from row pos of the tables,
// each product, sum and difference rounded to binary32, the result rounded
// to the element type):
//  - the query tile in registers, the partner half of a pair fetched from the
//    lane holding it;
//  - the S new key rows of the slice, once per workgroup, into LDS; stages
//    that reach new rows take their K chunks from there, and so do the
//    append and the compaction;
//  - an item with a position outside the tables is skipped like an
//    out-of-range seqlens_k.
#pragma once

#include "swgqa_common.hpp"
#include "swgqa_internal.hpp"
#include "swgqa_tail.hpp"

#include <math.h>

namespace swgqa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Stages of K/V loads in flight per wave (2: double, 3: triple buffering).
#ifndef SWGQA_DEC_DEPTH
#define SWGQA_DEC_DEPTH 3
#endif
// K/V rows are read once per step: streaming (non-temporal) loads, measured
// ~10% faster on the 32-item serving decode.
#ifndef SWGQA_DEC_NT
#define SWGQA_DEC_NT 1
#endif



template <int DT, int D, int NQ>
struct DecShape {
  static constexpr int e = Elem<DT>::bytes;
  static constexpr int EPL = 16 / e;                    // elements per lane per row
  static constexpr int LPR = D / EPL;                   // lanes per row
  static constexpr int RPW = kWave / (LPR > 0 ? LPR : 1);  // rows per load instruction
  static constexpr int U = (LPR / NQ) >= 1 ? (LPR / NQ) : 1;  // loads per stage
  static constexpr int SR = RPW * U;                    // rows per wave stage
  static constexpr int PAIRS = SR * NQ;                 // (row, query) pairs per stage
  static constexpr int PPL = PAIRS / kWave;             // pairs per lane
  static constexpr int NW = 4;                          // 32-bit words per chunk
  static constexpr bool ok = D % EPL == 0 && LPR >= 1 && LPR <= 16 &&
                             NQ * EPL <= 64 && PAIRS % kWave == 0 && NQ <= kWave;
};

// Wave-private ordering point for LDS traffic between the phases: LDS
// instructions of one wave execute in order, so only the compiler must not
// move accesses across this point.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Max / sum over the lanes that share (lane % NQ): xor offsets NQ..32.
// Offsets below 16 use DPP inside a 16-lane row (quad_perm for 1 and 2,
// row rotations by 4 and 8, which cover the same lane classes), 16 and 32
// row swaps between two copies (v_permlane16_swap / v_permlane32_swap).
template <int NQ, bool MAX>
__device__ __forceinline__ float allreduce_q(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  if constexpr (NQ <= 1) x = op(x, dpp_f<0xB1>(x));    // quad_perm [1,0,3,2]
  if constexpr (NQ <= 2) x = op(x, dpp_f<0x4E>(x));    // quad_perm [2,3,0,1]
  if constexpr (NQ <= 4) x = op(x, dpp_f<0x124>(x));   // row_ror:4
  if constexpr (NQ <= 8) x = op(x, dpp_f<0x128>(x));   // row_ror:8
  if constexpr (NQ <= 16) x = reduce_xor16(x, op);
  if constexpr (NQ <= 32) x = reduce_xor32(x, op);
  return x;
}

// dot of one 16-byte chunk of Q (held as words) with one chunk of K
template <int DT>
__device__ __forceinline__ float chunk_dot(const uint32_t* q, const uint32_t* k, float acc) {
  if constexpr (DT == kF32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(q[i]), __uint_as_float(k[i]), acc);
  } else if constexpr (DT == kBF16) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, q[i]),
                                            __builtin_bit_cast(bf2, k[i]), acc, false);
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, q[i]), __builtin_bit_cast(h2, k[i]),
                                   acc, false);
  }
  return acc;
}

// Table columns used by 16-byte chunk w of a row: EPC values from column
// (w * EPC) mod (D / 2) for pairs (k, k + D / 2) (one 16-byte load), EPC / 2
// values from column w * EPC / 2 for interleaved pairs (one 8-byte load).
// pos is already clamped to the table.
template <int DT, int D>
__device__ __forceinline__ void load_rot_cols(const void* table, int64_t pos, int w, bool ilv,
                                              uint32_t (&out)[4]) {
  constexpr int e = Elem<DT>::bytes, EPC = 16 / e;
  static_assert((D / 2) * e % 16 == 0, "table rows must hold whole 16-byte chunks");
  const char* row = (const char*)table + pos * (int64_t)(D / 2) * e;
  if (!ilv) {
    typedef const u32x4 __attribute__((address_space(1)))* gp;
    const u32x4 v = *(gp)(row + ((w * EPC) & (D / 2 - 1)) * e);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  } else {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    typedef const u32x2 __attribute__((address_space(1)))* gp;
    const u32x2 v = *(gp)(row + (w * EPC / 2) * e);
    out[0] = v[0]; out[1] = v[1]; out[2] = 0u; out[3] = 0u;
  }
}

// Rotates chunk w of a row (words f) given the partner chunk (words g: chunk
// w ^ (chunks per row / 2), holding the other element of each pair when the
// pairs are (k, k + D / 2)) and the table words of load_rot_cols.  Written
// as x c + y s' per element, x the element, y its partner, s' = -s where x
// is the pair's first element: the same products, sum and difference as
// (a c - b s, b c + a s), each rounded once (negation is exact).
template <int DT, int D>
__device__ __forceinline__ void rotate_chunk(uint32_t (&f)[4], const uint32_t (&g)[4],
                                             const uint32_t (&cw)[4], const uint32_t (&sw)[4],
                                             int w, bool ilv) {
#pragma clang fp contract(off)
  constexpr int e = Elem<DT>::bytes, EPC = 16 / e, EPW = EPC / 4;
  float x[EPC], y[EPC], c[EPC], s[EPC], r[EPC];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    unpack_word<DT>(f[i], x + i * EPW);
    unpack_word<DT>(g[i], y + i * EPW);
    unpack_word<DT>(cw[i], c + i * EPW);
    unpack_word<DT>(sw[i], s + i * EPW);
  }
  if (!ilv) {
    const float sg = w * EPC < D / 2 ? -1.0f : 1.0f;  // x holds the pairs' first elements
#pragma unroll
    for (int j = 0; j < EPC; ++j) {
      const float xc = x[j] * c[j], ys = y[j] * (sg * s[j]);
      r[j] = xc + ys;
    }
  } else {
#pragma unroll
    for (int m = 0; m < EPC / 2; ++m) {
      const float a = x[2 * m], b = x[2 * m + 1];
      const float ac = a * c[m], bs = b * s[m], bc = b * c[m], as = a * s[m];
      r[2 * m] = ac - bs;
      r[2 * m + 1] = bc + as;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = pack_word<DT>(r + i * EPW);
}

// Word v of lane l ^ M (M < 16; lanes in rows of 16 as DPP sees them):
// quad permutes for 1 and 2, a row rotation by 8 for 8, and for 4 a row
// rotation by 12 (lanes with bit 2 clear, reading lane + 4) or by 4 (the
// others, reading lane - 4); a row rotation right by n reads lane - n.
template <int M>
__device__ __forceinline__ uint32_t xor_lanes(uint32_t v) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8, "lane distance within a DPP row");
  if constexpr (M == 1) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
  } else if constexpr (M == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
  } else if constexpr (M == 4) {
    const uint32_t up = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x12C, 0xF, 0xF, false);
    const uint32_t dn = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false);
    return (__lane_id() & 4) ? dn : up;
  } else {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);
  }
}

// Rows of new keys the rotary variant holds in LDS (S < 16 on this path).
constexpr int kRotMaxRows = 16;

template <int DT, int D, int NQ, int kWaves, int DEPTH, bool ROT, bool FM = false>
__global__ __launch_bounds__(kWaves * kWave)
__attribute__((amdgpu_waves_per_eu((kWaves + 3) / 4, 8))) void attn_decode_kernel(AttnArgs a) {
  constexpr int kThreads = kWaves * kWave;
  using Sh = DecShape<DT, D, NQ>;
  constexpr int e = Sh::e, EPL = Sh::EPL, LPR = Sh::LPR, RPW = Sh::RPW, U = Sh::U;
  constexpr int SR = Sh::SR, PAIRS = Sh::PAIRS, PPL = Sh::PPL;
  static_assert(Sh::ok, "unsupported decode shape");

  // work item P of the launch: slice P / T, item (tile, split) P % T
  const uint32_t T = gridDim.x;  // ntiles * nsplit
  const uint32_t P = xcd_contiguous(blockIdx.x + T * (blockIdx.y + gridDim.y * blockIdx.z),
                                    T * gridDim.y * gridDim.z);
  const uint32_t slice = div_gap(P, a.tdiv);
  const uint32_t t = P - slice * T;
  const int b = (int)div_gap(slice, a.hdiv);
  const int kvh = (int)slice - b * a.Hkv;
  // seqlens_k first: the plan and every K/V address wait on it
  const int32_t seqlen = load_seqlen(a.seqlens, b);
  const int tile = a.nsplit == 1 ? (int)t : (int)div_gap(t, a.sdiv);
  const int split = (int)t - tile * a.nsplit;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int rslot = lane / LPR;
  const int sub = lane % LPR;

  __shared__ float s_part[kWaves][NQ * SR * LPR];   // [q][row][sub]
  __shared__ float s_p[kWaves][PAIRS];              // [row][q]
  __shared__ float s_corr[kWaves][NQ];
  __shared__ float s_m[kWaves][NQ];
  __shared__ float s_l[kWaves][NQ];
  __shared__ float s_acc[kWaves][NQ][D];
  __shared__ u32x4 s_knew[ROT ? kRotMaxRows * (D * e / 16) : 1];  // rotated new keys
  __shared__ u32x4 s_knew1[ROT ? kWaves : 1][ROT ? D * e / 16 : 1];  // per wave, S == 1

  // New rows of a drifting step are appended by tile 0 of split 0 (shared
  // buffer only): rows [Lb, Lb + S) lie beyond every row this step reads, so
  // they can be written as soon as Lb is known.  The sources do not depend on
  // the plan and are loaded first.
  constexpr int W16 = D * e / 16;
  const bool appender = a.present_k != nullptr && tile == 0 && split == 0;
  const bool early_append = appender && a.S * W16 <= kThreads;
  u32x4 app_k = {0u, 0u, 0u, 0u}, app_v = {0u, 0u, 0u, 0u};
  // ROT: chunk k_w of new row k_row per thread (clamped; S * W16 <= threads
  // on this path), and the positions of the item's rows in lanes 0 .. S - 1
  const int nkc = a.S * W16;
  const int kc_t = a.S == 1 ? lane : tid;  // S == 1: the row's chunks in every wave
  const int kc = kc_t < nkc ? kc_t : nkc - 1;
  const int k_row = kc / W16, k_w = kc % W16;
  int64_t pos_lane = 0;
  if constexpr (ROT) {
    const int64_t src = ((int64_t)(b * a.S + k_row) * a.Hkv + kvh) * D * e + k_w * 16;
    app_k = *(const u32x4*)((const char*)a.k + src);
    if (early_append) app_v = *(const u32x4*)((const char*)a.v + src);
    if (a.rot_pos) pos_lane = a.rot_pos[(int64_t)b * a.S + (lane < a.S ? lane : a.S - 1)];
  } else if (early_append && tid < a.S * W16) {
    const int64_t src = ((int64_t)(b * a.S + tid / W16) * a.Hkv + kvh) * D * e + (tid % W16) * 16;
    app_k = *(const u32x4*)((const char*)a.k + src);
    app_v = *(const u32x4*)((const char*)a.v + src);
  }

  const int nq_item = a.S * a.group;
  const int q0 = tile * NQ;
  // Query tile: (position, head) pairs q0 .. q0 + NQ - 1, position-major,
  // walked with a carry (pairs past the item's last repeat it).  Loaded
  // before the plan: their addresses do not depend on seqlens_k.
  const int i_first = (int)div_gap((uint32_t)q0, a.qdiv);
  int i_last = i_first;
  uint32_t qw[NQ][4];
  int q_row[NQ];  // position index i of each pair (ROT)
  {
    int h = q0 - i_first * a.group;
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      q_row[t] = i_last;
      const int64_t row = ((int64_t)b * a.S + i_last) * a.Hq + kvh * a.group + h;
      const uint4 v = *(const uint4*)((const char*)a.q + (row * D + sub * EPL) * e);
      qw[t][0] = v.x; qw[t][1] = v.y; qw[t][2] = v.z; qw[t][3] = v.w;
      if (t + 1 < NQ && q0 + t + 1 < nq_item && ++h == a.group) {
        h = 0;
        ++i_last;
      }
    }
  }
  ItemPlan pl = plan_item(seqlen, a.S, a.C, a.gdiv, a.total);
  if constexpr (ROT) {
    // every position inside the tables, else the item is skipped; the step
    // tail (a later launch) reads the verdict as an out-of-range length
    bool rot_ok;
    if (a.rot_pos)
      rot_ok = !__any(lane < a.S && (pos_lane < 0 || pos_lane >= (int64_t)a.rot_rows));
    else
      rot_ok = pl.P + a.S - 1 < (int64_t)a.rot_rows;  // P >= 0 when the plan is valid
    if (a.seqlens_out && tid == 0 && tile == 0 && split == 0 && kvh == 0)
      a.seqlens_out[b] = rot_ok ? seqlen : -2;
    pl.ok = pl.ok && rot_ok;
  } else if (early_append && pl.ok && pl.shift == 0 && tid < a.S * W16) {
    const int64_t dst = ((int64_t)(b * a.Hkv + kvh) * a.C + pl.Lb + tid / W16) * D * e +
                        (tid % W16) * 16;
    *(u32x4*)((char*)a.present_k + dst) = app_k;
    *(u32x4*)((char*)a.present_v + dst) = app_v;
  }

  if (!pl.ok) {
    if (tid == 0 && tile == 0 && split == 0 && kvh == 0) flag_status(a.status, kStatusBadItem);
    for (int idx = tid; idx < NQ * D; idx += kThreads) {
      const int t = idx / D, d = idx % D;
      const int qi = q0 + t;
      if (qi >= nq_item) continue;
      const int i = (int)div_gap((uint32_t)qi, a.qdiv), h = kvh * a.group + qi - i * a.group;
      const int64_t row = ((int64_t)b * a.S + i) * a.Hq + h;
      if (a.nsplit == 1) {
        if constexpr (DT == kF32) ((float*)a.out)[row * D + d] = 0.0f;
        else ((uint16_t*)a.out)[row * D + d] = 0;
      } else {
        a.opart[(row * a.nsplit + split) * D + d] = 0.0f;
        if (d == 0) {
          a.ml[(row * a.nsplit + split) * 2 + 0] = -INFINITY;
          a.ml[(row * a.nsplit + split) * 2 + 1] = 0.0f;
        }
      }
    }
    return;
  }

  // the query this lane scores in phase B (same for all its pairs)
  const int my_q = lane % NQ;
  const int my_qi = q0 + my_q;
  const bool my_q_ok = my_qi < nq_item;
  const int my_qd = (int)div_gap((uint32_t)my_qi, a.qdiv);  // (divisions by invariants)
  const int my_i = my_q_ok ? my_qd : i_last;
  const int my_h = kvh * a.group + (my_q_ok ? my_qi - my_qd * a.group : 0);
  const int64_t my_pos = pl.P + my_i;

  // Union key range of the tile, split evenly (n < 2^31: keys are positions
  // below total_sequence_length).
  const int64_t p_first = pl.P + i_first;
  const int64_t p_last = pl.P + i_last;
  const int64_t lo = p_first - a.W + 1 > 0 ? p_first - a.W + 1 : 0;
  const int64_t n = p_last - lo + 1;
  const int64_t chunk =
      a.nsplit == 1 ? n : (int64_t)div_gap((uint32_t)n + (uint32_t)a.nsplit - 1u, a.sdiv);
  const int64_t kb = lo + split * chunk;
  const int64_t ke = kb + chunk < p_last + 1 ? kb + chunk : p_last + 1;
  const int32_t nk = ke > kb ? (int32_t)(ke - kb) : 0;  // keys kb + jr, 0 <= jr < nk
  const int nst = (nk + SR - 1) / SR;
  // keys with jr < ncache are resident cache rows, the others new rows
  const int32_t ncache = (int32_t)(pl.P - kb < 0 ? 0 : (pl.P - kb < nk ? pl.P - kb : nk));
  const int knew0 = (int)(kb - pl.P);  // new row of key jr >= ncache: knew0 + jr

  // visibility of key kb + jr for this lane's query, as 32-bit bounds on jr
  const int64_t vlo = my_pos - a.W + 1 - kb;
  const int64_t vhi = (my_pos < ke - 1 ? my_pos : ke - 1) - kb;
  const int32_t vis_lo = my_q_ok ? (int32_t)(vlo < -(int64_t)0x7fffffff ? -0x7fffffff : vlo) : 1;
  const int32_t vis_hi = my_q_ok ? (int32_t)vhi : 0;

  // Byte addresses of key jr for this lane's 16-byte chunk: cache row
  // kb + jr - (P - Lb) of the slice, or new row kb + jr - P of the step.
  constexpr int kRowBytes = D * e;
  constexpr int kRowShift = __builtin_ctz(kRowBytes);
  static_assert((kRowBytes & (kRowBytes - 1)) == 0, "row bytes must be a power of two");
  const int64_t slice_row0 = (int64_t)(b * a.Hkv + kvh) * a.C + (kb - (pl.P - pl.Lb));
  const uint64_t ck_lane = (uint64_t)a.past_k + (uint64_t)(slice_row0 * kRowBytes) + sub * 16;
  const uint64_t cv_lane = (uint64_t)a.past_v + (uint64_t)(slice_row0 * kRowBytes) + sub * 16;
  const int64_t new_stride = (int64_t)a.Hkv * kRowBytes;  // bytes between new rows
  const int64_t new_row0 = (int64_t)b * a.S + (kb + ncache - pl.P);  // new row of jr = ncache
  const uint64_t nk_lane = (uint64_t)a.k + (uint64_t)((new_row0 * a.Hkv + kvh) * kRowBytes) + sub * 16;
  const uint64_t nv_lane = (uint64_t)a.v + (uint64_t)((new_row0 * a.Hkv + kvh) * kRowBytes) + sub * 16;
  const uint64_t dv_cache = cv_lane - ck_lane;
  const uint64_t dv_new = nv_lane - nk_lane;

  // FM: a compacting step whose slice this workgroup reads alone (one query
  // tile, one key split, shared buffer): the surviving rows, stage rows jr in
  // [ncache - kept, ncache), all of them read here, are stored `shift` rows
  // down while their stage is computed, rather than read a second time after
  // attention.  Stage st belongs to round st / kWaves; a destination lies
  // `shift` rows, at least fm_every = 2^k <= shift / (kWaves * SR) rounds,
  // below its source, so after a barrier that every wave passes once it has
  // computed every fm_every-th round (its loads of those rounds returned), all
  // destinations of the next fm_every rounds are rows no wave still reads.
  // Rows below the read range (evicted) are read by nobody.
  constexpr int kRoundRows = kWaves * SR;
  const bool fmove = FM && !ROT && a.fuse_writeback && a.ntiles == 1 && a.nsplit == 1 &&
                     pl.shift >= kRoundRows && pl.kept > 0 && pl.kept <= ncache;
  const int nrounds = (nst + kWaves - 1) / kWaves;
  int fm_mask = 0;
  if (fmove) {
    const int64_t q = pl.shift / kRoundRows;  // >= 1
    const int lg = 63 - __builtin_clzll((uint64_t)q);
    fm_mask = (1 << (lg < 20 ? lg : 20)) - 1;
  }
  const int32_t fm_lo = ncache - (int32_t)(fmove ? pl.kept : 0);
  const uint64_t fm_k =
      (uint64_t)a.present_k + (uint64_t)((slice_row0 - pl.shift) * kRowBytes) + sub * 16;
  const uint64_t fm_dv = (uint64_t)a.present_v - (uint64_t)a.present_k;

  const bool has_cap = a.softcap > 0.0f;
  const float cap = a.softcap;
  const float inv_cap = a.inv_softcap;  // (made on the host)
  const bool has_bias = a.bias != nullptr;
  const int64_t bias_row = has_bias
      ? ((((a.bias_b ? (int64_t)b : 0) * (a.bias_h ? a.Hq : 1) + (a.bias_h ? my_h : 0)) * a.S + my_i) *
         (int64_t)a.total)
      : 0;

  float m_run = -INFINITY;  // running max (log2 units) of query my_q; wave-uniform per query
  float l_run = 0.0f;       // this lane's share of the running sum
  float acc[NQ][EPL];
#pragma unroll
  for (int t = 0; t < NQ; ++t)
#pragma unroll
    for (int k = 0; k < EPL; ++k) acc[t][k] = 0.0f;

  const bool ilv = ROT && a.rot_interleaved != 0;
  // rotated new key rows: the workgroup's copy, or with S == 1 this wave's
  // own copy of the one row (no barrier needed)
  const u32x4* knew_lds = (ROT && a.S == 1) ? &s_knew1[wave][0] : &s_knew[0];

  float* part = s_part[wave];
  float* pbuf = s_p[wave];
  float* cbuf = s_corr[wave];

  // Loads of one stage, issued unconditionally: rows past the split's end
  // are clamped to its last key (finite data whose scores the mask removes),
  // so the compiler can count the loads in flight and wait only for the
  // stage being computed.
  auto load_stage = [&](int st, uint32_t (&kr)[U][4], uint32_t (&vr)[U][4]) __attribute__((always_inline)) {
    const uint32_t s0 = (uint32_t)min(st, nst) * SR;  // no overflow: nst * SR < 2^31 + SR
    const uint32_t last = (uint32_t)(nk - 1);
    uint64_t ka[U], va[U];
    if (s0 + SR <= (uint32_t)ncache) {  // uniform: a whole stage of cache rows, no clamp
      // (ncache <= nk; the rows' offsets from the stage's first are constants)
      const uint64_t k0 = ck_lane + ((uint64_t)(s0 + rslot) << kRowShift);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        ka[u] = k0 + ((uint64_t)(u * RPW) << kRowShift);
        va[u] = ka[u] + dv_cache;
      }
    } else if (min(s0 + SR, (uint32_t)nk) <= (uint32_t)ncache) {  // uniform: only cache rows
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t off = (uint64_t)min(s0 + u * RPW + rslot, last) << kRowShift;
        ka[u] = ck_lane + off;
        va[u] = cv_lane + off;
      }
    } else {
      // branch-free mask select: a plain select between these bases is
      // turned into a private-memory lookup table by the compiler
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t jr = min(s0 + u * RPW + rslot, last);
        const uint64_t msk = 0ull - (uint64_t)(jr < (uint32_t)ncache);
        ka[u] = ((ck_lane + ((uint64_t)jr << kRowShift)) & msk) |
                ((nk_lane + (uint64_t)(((int64_t)jr - ncache) * new_stride)) & ~msk);
        va[u] = ka[u] + ((dv_cache & msk) | (dv_new & ~msk));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x4 kk = load16_global<SWGQA_DEC_NT>(ka[u]);
      const u32x4 vv = load16_global<SWGQA_DEC_NT>(va[u]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        kr[u][w] = kk[w];
        vr[u][w] = vv[w];
      }
    }
  };

  auto compute_stage = [&](int st, uint32_t (&kr)[U][4], const uint32_t (&vr)[U][4]) __attribute__((always_inline)) {
    if constexpr (ROT) {
      // new rows take their rotated chunks from LDS (uniform test)
      const uint32_t s0 = (uint32_t)st * SR;
      if (s0 + SR > (uint32_t)ncache) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t jr = min(s0 + u * RPW + rslot, (uint32_t)(nk - 1));
          if (jr >= (uint32_t)ncache) {
            const u32x4 r = knew_lds[(knew0 + (int)jr) * W16 + sub];
#pragma unroll
            for (int w = 0; w < 4; ++w) kr[u][w] = r[w];
          }
        }
      }
    }
    // A. partial dots -> LDS [q][row][sub]
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = u * RPW + rslot;
#pragma unroll
      for (int t = 0; t < NQ; ++t) part[(t * SR + row) * LPR + sub] = chunk_dot<DT>(qw[t], kr[u], 0.0f);
    }
    uint32_t tok = 0u;
    if constexpr (FM && !ROT) {
      if (fmove) {  // the moved rows' K words
        const int32_t s0 = st * SR;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int32_t jr = s0 + u * RPW + rslot;
          if (jr >= fm_lo && jr < ncache)
            store16_global<SWGQA_FM_NT>(fm_k + ((uint64_t)(uint32_t)jr << kRowShift),
                           u32x4{kr[u][0], kr[u][1], kr[u][2], kr[u][3]});
#pragma unroll
          for (int w = 0; w < 4; ++w) tok ^= kr[u][w];
        }
      }
    }
    wave_lds_fence();
    // B. scores, stage max, probabilities
    float s[PPL];
    float smax = -INFINITY;
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      const int pid = lane + k * kWave;
      const int row = pid / NQ;
      const float* pp = part + (my_q * SR + row) * LPR;
      float x = 0.0f;
      if constexpr (LPR % 4 == 0) {
#pragma unroll
        for (int w = 0; w < LPR; w += 4) {
          const float4 v4 = *(const float4*)(pp + w);
          x += (v4.x + v4.y) + (v4.z + v4.w);
        }
      } else {
#pragma unroll
        for (int w = 0; w < LPR; ++w) x += pp[w];
      }
      x *= a.scale;
      const int32_t jr = st * SR + row;
      const bool vis = jr >= vis_lo && jr <= vis_hi;
      if (has_cap) {
        const float y = x * inv_cap;
        if constexpr (DT == kF32) {
          x = cap * tanhf(y);
        } else {
          // tanh|y| = 1 - 2 / (e^{2|y|} + 1): one exp and one reciprocal;
          // its absolute error (~1e-7) is far inside fp16/bf16 outputs
          const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(
                                     __builtin_amdgcn_exp2f(2.0f * kLog2e * fabsf(y)) + 1.0f);
          x = cap * copysignf(t, y);
        }
      }
      if (has_bias && vis) x += load_one<DT>(a.bias, bias_row + kb + jr);
      s[k] = vis ? x * kLog2e : -INFINITY;
      smax = fmaxf(smax, s[k]);
    }
    smax = allreduce_q<NQ, true>(smax);
    const float m_new = fmaxf(m_run, smax);
    const float corr = (m_run == m_new) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.0f;
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      const float p = (s[k] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(s[k] - m_new);
      pbuf[lane + k * kWave] = p;
      psum += p;
    }
    l_run = l_run * corr + psum;
    m_run = m_new;
    if (lane < NQ) cbuf[lane] = corr;
    wave_lds_fence();
    // C. rescale and accumulate V
    float cr[NQ];
    bool rescale = false;
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      cr[t] = cbuf[t];
      rescale |= cr[t] != 1.0f;
    }
    if (rescale) {  // the same in every lane: skipped once the maxima settle
#pragma unroll
      for (int t = 0; t < NQ; ++t)
#pragma unroll
        for (int k = 0; k < EPL; ++k) acc[t][k] *= cr[t];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = u * RPW + rslot;
      float pr[NQ];
#pragma unroll
      for (int t = 0; t < NQ; ++t) pr[t] = pbuf[row * NQ + t];
      float vf[EPL];
#pragma unroll
      for (int w = 0; w < 4; ++w) unpack_word<DT>(vr[u][w], &vf[w * (EPL / 4)]);
#pragma unroll
      for (int t = 0; t < NQ; ++t)
#pragma unroll
        for (int k = 0; k < EPL; ++k) acc[t][k] = fmaf(pr[t], vf[k], acc[t][k]);
    }
    wave_lds_fence();
    if constexpr (FM && !ROT) {
      if (fmove) {  // the moved rows' V words, and the round's barrier
        const int32_t s0 = st * SR;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int32_t jr = s0 + u * RPW + rslot;
          if (jr >= fm_lo && jr < ncache)
            store16_global<SWGQA_FM_NT>(fm_k + fm_dv + ((uint64_t)(uint32_t)jr << kRowShift),
                           u32x4{vr[u][0], vr[u][1], vr[u][2], vr[u][3]});
#pragma unroll
          for (int w = 0; w < 4; ++w) tok ^= vr[u][w];
        }
        const int m = st / kWaves;
        if (m + 1 < nrounds && ((m + 1) & fm_mask) == 0) barrier_after(tok);
      }
    }
  };

  // ROT: rotation of the query tile and of the slice's new key chunks, once
  // the first stage loads are issued (the table loads queue behind them);
  // the rotated keys go to LDS, to the appended rows and, for a step tail
  // that rewrites the cache, to a.k_rot; then a barrier.
  // S == 1: the tables' chunk `sub` at the step's one position, loaded ahead
  // of the stage loads so that it has arrived when rot_prep runs
  uint32_t rc1[4] = {0u, 0u, 0u, 0u}, rs1[4] = {0u, 0u, 0u, 0u};
  if constexpr (ROT) {
    if (a.S == 1) {
      int64_t r = a.rot_pos ? pos_lane : pl.P;  // lanes hold position 0 (S == 1)
      r = r < 0 ? 0 : (r >= a.rot_rows ? (int64_t)a.rot_rows - 1 : r);
      load_rot_cols<DT, D>(a.rot_cos, r, sub, ilv, rc1);
      load_rot_cols<DT, D>(a.rot_sin, r, sub, ilv, rs1);
    }
  }
  auto rot_prep = [&]() __attribute__((always_inline)) {
    if constexpr (ROT) {
      const int64_t top = (int64_t)a.rot_rows - 1;
      auto table_row = [&](int i) -> int64_t {
        const int64_t p = a.rot_pos ? (int64_t)__shfl((long long)pos_lane, i, kWave) : pl.P + i;
        return p < 0 ? 0 : (p > top ? top : p);
      };
      if (a.S == 1) {
        // One position for the whole step: one cos / sin chunk per lane
        // (chunk `sub`, which is also chunk k_w of the new row in the lanes
        // lane < W16 that hold it, in every wave); each wave rotates the row
        // into its own LDS copy, so no barrier is needed.
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
          uint32_t g[4];
#pragma unroll
          for (int w = 0; w < 4; ++w) g[w] = xor_lanes<LPR / 2>(qw[t][w]);
          rotate_chunk<DT, D>(qw[t], g, rc1, rs1, sub, ilv);
        }
        uint32_t f[4], g[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          f[w] = app_k[w];
          g[w] = xor_lanes<W16 / 2>(f[w]);
        }
        rotate_chunk<DT, D>(f, g, rc1, rs1, sub, ilv);
        const u32x4 rk = {f[0], f[1], f[2], f[3]};
        if (lane < W16) s_knew1[wave][lane] = rk;
        wave_lds_fence();
        if (tid < nkc) {
          if (early_append && pl.shift == 0) {
            const int64_t dst = ((int64_t)(b * a.Hkv + kvh) * a.C + pl.Lb) * D * e + k_w * 16;
            *(u32x4*)((char*)a.present_k + dst) = rk;
            *(u32x4*)((char*)a.present_v + dst) = app_v;
          }
          if (a.k_rot && tile == 0 && split == 0) {
            const int64_t at = ((int64_t)b * a.Hkv + kvh) * D * e + k_w * 16;
            *(u32x4*)((char*)a.k_rot + at) = rk;
          }
        }
        return;
      }
      uint32_t qc[NQ][4], qs[NQ][4], kcw[4], ksw[4];
#pragma unroll
      for (int t = 0; t < NQ; ++t) {
        const int64_t r = table_row(q_row[t]);
        load_rot_cols<DT, D>(a.rot_cos, r, sub, ilv, qc[t]);
        load_rot_cols<DT, D>(a.rot_sin, r, sub, ilv, qs[t]);
      }
      const int64_t kr_row = table_row(k_row);
      load_rot_cols<DT, D>(a.rot_cos, kr_row, k_w, ilv, kcw);
      load_rot_cols<DT, D>(a.rot_sin, kr_row, k_w, ilv, ksw);
#pragma unroll
      for (int t = 0; t < NQ; ++t) {
        uint32_t g[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) g[w] = xor_lanes<LPR / 2>(qw[t][w]);
        rotate_chunk<DT, D>(qw[t], g, qc[t], qs[t], sub, ilv);
      }
      uint32_t f[4], g[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        f[w] = app_k[w];
        g[w] = xor_lanes<W16 / 2>(f[w]);
      }
      rotate_chunk<DT, D>(f, g, kcw, ksw, k_w, ilv);
      const u32x4 rk = {f[0], f[1], f[2], f[3]};
      if (tid < nkc) {
        s_knew[tid] = rk;  // row k_row, chunk k_w
        if (early_append && pl.shift == 0) {
          const int64_t dst = ((int64_t)(b * a.Hkv + kvh) * a.C + pl.Lb + k_row) * D * e + k_w * 16;
          *(u32x4*)((char*)a.present_k + dst) = rk;
          *(u32x4*)((char*)a.present_v + dst) = app_v;
        }
        if (a.k_rot && tile == 0 && split == 0) {
          const int64_t at = ((int64_t)(b * a.S + k_row) * a.Hkv + kvh) * D * e + k_w * 16;
          *(u32x4*)((char*)a.k_rot + at) = rk;
        }
      }
      __syncthreads();
    }
  };

  // Stages of this wave: wave, wave + kWaves, ...; the loads of the next
  // DEPTH - 1 stages are in flight while one stage is computed.
  uint32_t k0[U][4], v0[U][4], k1[U][4], v1[U][4];
  int st = wave;
  if (nk == 0) {
    // empty split: nothing to read
    rot_prep();
  } else if (nst <= kWaves) {
    // at most one stage per wave: nothing to overlap
    if constexpr (ROT) {
      if (wave < nst) load_stage(wave, k0, v0);
      rot_prep();
      if (wave < nst) compute_stage(wave, k0, v0);
    } else if (wave < nst) {
      load_stage(wave, k0, v0);
      compute_stage(wave, k0, v0);
    }
  } else if constexpr (DEPTH == 3) {
    load_stage(st, k0, v0);
    uint32_t k2[U][4], v2[U][4];
    rot_prep();  // between the first two stages' loads: fewer registers live
    load_stage(st + kWaves, k1, v1);
    while (st < nst) {
      load_stage(st + 2 * kWaves, k2, v2);
      compute_stage(st, k0, v0);
      st += kWaves;
      if (st >= nst) break;
      load_stage(st + 2 * kWaves, k0, v0);
      compute_stage(st, k1, v1);
      st += kWaves;
      if (st >= nst) break;
      load_stage(st + 2 * kWaves, k1, v1);
      compute_stage(st, k2, v2);
      st += kWaves;
    }
  } else {
    load_stage(st, k0, v0);
    rot_prep();
    while (st < nst) {
      load_stage(st + kWaves, k1, v1);
      compute_stage(st, k0, v0);
      st += kWaves;
      if (st >= nst) break;
      load_stage(st + kWaves, k0, v0);
      compute_stage(st, k1, v1);
      st += kWaves;
    }
  }

  // the barriers of rounds this wave had no stage in
  if (FM && fmove) {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int done = nst > wv ? (nst - wv + kWaves - 1) / kWaves : 0;
    for (int m = done; m + 1 < nrounds; ++m)
      if (((m + 1) & fm_mask) == 0) barrier_after(0u);
  }

  // Wave result: acc summed over row slots, l over the lanes of each query.
  const float l_tot = allreduce_q<NQ, false>(l_run);
  // (sum over the lanes that share lane % LPR: the row slots)
#pragma unroll
  for (int t = 0; t < NQ; ++t)
#pragma unroll
    for (int k = 0; k < EPL; ++k) acc[t][k] = allreduce_q<LPR, false>(acc[t][k]);
  if (rslot == 0) {
#pragma unroll
    for (int t = 0; t < NQ; ++t)
#pragma unroll
      for (int k = 0; k < EPL; ++k) s_acc[wave][t][sub * EPL + k] = acc[t][k];
  }
  if (lane < NQ) {
    s_m[wave][lane] = m_run;
    s_l[wave][lane] = l_tot;
  }
  __syncthreads();

  // Merge the waves; write the output or this split's partial.
  for (int idx = tid; idx < NQ * D; idx += kThreads) {
    const int t = idx / D, d = idx % D;
    const int qi = q0 + t;
    if (qi >= nq_item) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][t]);
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float c = (s_m[w][t] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(s_m[w][t] - M);
      L += s_l[w][t] * c;
      A += s_acc[w][t][d] * c;
    }
    const int i = (int)div_gap((uint32_t)qi, a.qdiv), h = kvh * a.group + qi - i * a.group;
    const int64_t row = ((int64_t)b * a.S + i) * a.Hq + h;
    if (a.nsplit == 1) {
      const float c = fold_sink<DT>(a.sink, a.smooth, h, M, L);
      const float o = A * c / L;
      if constexpr (DT == kF32) ((float*)a.out)[row * D + d] = o;
      else if constexpr (DT == kF16) ((_Float16*)a.out)[row * D + d] = (_Float16)o;
      else ((uint16_t*)a.out)[row * D + d] = f32_to_bf16(o);
    } else {
      a.opart[(row * a.nsplit + split) * D + d] = A;
      if (d == 0) {
        a.ml[(row * a.nsplit + split) * 2 + 0] = M;
        a.ml[(row * a.nsplit + split) * 2 + 1] = L;
      }
    }
  }
  // Appends of more rows than threads, after attention (never with ROT,
  // whose S * W16 new chunks fit the workgroup).
  if (!ROT && appender && !early_append && pl.shift == 0) {
    char* pk = (char*)a.present_k + ((int64_t)(b * a.Hkv + kvh) * a.C) * D * e;
    char* pv = (char*)a.present_v + ((int64_t)(b * a.Hkv + kvh) * a.C) * D * e;
    for (int idx = tid; idx < a.S * W16; idx += kThreads) {
      const int i = idx / W16, w = idx % W16;
      const int64_t src = ((int64_t)(b * a.S + i) * a.Hkv + kvh) * D * e + w * 16;
      const int64_t dst = (pl.Lb + i) * (int64_t)D * e + w * 16;
      *(uint4*)(pk + dst) = *(const uint4*)((const char*)a.k + src);
      *(uint4*)(pv + dst) = *(const uint4*)((const char*)a.v + src);
    }
  }

  slice_tail<DT>(a, pl, b, kvh, D, ROT ? (a.S == 1 ? &s_knew1[0][0] : &s_knew[0]) : nullptr,
                 fmove);
}

template <int DT, int D, int NQ, bool ROT>
hipError_t launch_nq(const AttnArgs& a, hipStream_t st) {
  if constexpr (DecShape<DT, D, NQ>::ok) {
    const dim3 grid(a.ntiles * a.nsplit, a.Hkv, a.B);
    // with rotary, 8-wave workgroups (at most 256 registers a lane) keep two
    // stages in flight: a third spills
    // the variant that moves surviving rows while reading them (compacting
    // steps of long windows; see the kernel) where the host asks for it, in
    // shapes whose three register sets leave room for it (no spills)
    using Sh = DecShape<DT, D, NQ>;
    constexpr bool kFm = SWGQA_FUSED_MOVE && !ROT && Sh::U <= 4 && Sh::PPL <= 2;
    if (kFm && a.waves == 8 && a.fused_move)
      attn_decode_kernel<DT, D, NQ, 8, SWGQA_DEC_DEPTH, false, kFm><<<grid, 8 * kWave, 0, st>>>(a);
    else if (a.waves == 8)
      attn_decode_kernel<DT, D, NQ, 8, ROT ? 2 : SWGQA_DEC_DEPTH, ROT><<<grid, 8 * kWave, 0, st>>>(a);
    else
      attn_decode_kernel<DT, D, NQ, 4, SWGQA_DEC_DEPTH, ROT><<<grid, 4 * kWave, 0, st>>>(a);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <int DT, int D>
int stage_rows(int nq) {
  switch (nq) {
    case 2: return DecShape<DT, D, 2>::SR;
    case 4: return DecShape<DT, D, 4>::SR;
    case 8: return DecShape<DT, D, 8>::SR;
    case 16: return DecShape<DT, D, 16>::SR;
    default: return 1;
  }
}

template <int DT, int D>
bool shape_ok(int nq) {
  switch (nq) {
    case 2: return DecShape<DT, D, 2>::ok;
    case 4: return DecShape<DT, D, 4>::ok;
    case 8: return DecShape<DT, D, 8>::ok;
    case 16: return DecShape<DT, D, 16>::ok;
    default: return false;
  }
}

template <int DT, int D, bool ROT>
hipError_t launch_d(int nq, const AttnArgs& a, hipStream_t st) {
  switch (nq) {
    case 2: return launch_nq<DT, D, 2, ROT>(a, st);
    case 4: return launch_nq<DT, D, 4, ROT>(a, st);
    case 8: return launch_nq<DT, D, 8, ROT>(a, st);
    case 16: return launch_nq<DT, D, 16, ROT>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

}  // namespace swgqa
