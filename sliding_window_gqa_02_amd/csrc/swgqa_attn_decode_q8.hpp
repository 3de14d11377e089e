// swgqa_attn_decode_q8.hpp -- staged grouped-query attention for short steps
// (S < 16) over a windowed KV cache held as 8-bit codes: int8
// (swgqa_attn_decode_q8.hip) or fp8 E4M3 (swgqa_attn_decode_f8.hip).
//
// The Investigation Report (onnxruntime/mobius issue #111), section 1.1,
// names the inputs k_scale / v_scale ("KV cache quantization scale") and a
// cache type apart from the element type.  Reading taken: one scale per
// tensor, a cache element stands for code * scale, and a new element x is
// stored as the binary32 quotient x / scale rounded to an integer (ties to
// even) and saturated to [-128, 127]; the step attends to every key and value
// row in that dequantized form, new rows included.  With fp8 E4M3 codes the
// same holds with the quotient rounded to the nearest E4M3 value (ties to the
// even code, saturated at 448).
//
// Same contract and work split as the staged decode kernel
// (swgqa_attn_decode.hpp): one workgroup per (item, KV head, query tile,
// key split), query i of item b at p = P + i attends keys p - W < j <= p of
// [resident rows | S new rows].  What differs:
//  - scores are scale * k_scale * sum(q * code), the value sum is taken over
//    codes and multiplied by v_scale once, at the end; codes enter the
//    products as exact 16-bit values (integers of at most 8 bits and E4M3
//    values are exact in fp16 and bf16);
//  - 16-bit queries in 4-query tiles with D >= 64 (the serving shape) take
//    both products on the matrix cores, a 16-row stage at a time: scores as
//    K . Q^T (16 x 16 x 32 in the query type, the 4 queries repeated over the
//    16 columns), value sums as P . V (16 x 16 x 16 in fp16, P rounded to
//    fp16 once and the normaliser summing the rounded values);
//  - other shapes use the vector units: a lane's 16-byte chunk holds 16
//    codes, so a row of D codes takes D / 16 lanes, dotted with the query
//    tile held in registers (packed 16-bit pairs for fp16 / bf16); with
//    16-bit outputs P is rounded to fp16 and the value sum taken two rows at
//    a time as packed fp16 dot products;
//  - the S new rows of the slice are quantized once per workgroup into LDS
//    (K and V codes); stages that reach them take their chunks from there
//    (their global loads are clamped to a resident row), and so do the
//    append and the in-place compaction.
#pragma once

#include "swgqa_common.hpp"
#include "swgqa_internal.hpp"
#include "swgqa_tail.hpp"

#include <math.h>

namespace swgqa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Stages of K/V loads in flight per wave.
#ifndef SWGQA_Q8_DEPTH
#define SWGQA_Q8_DEPTH 3
#endif

#ifndef SWGQA_Q8_PV16
#define SWGQA_Q8_PV16 1
#endif

#ifndef SWGQA_Q8_UMUL
#define SWGQA_Q8_UMUL 1
#endif

// Key scores of 16-bit queries on the matrix cores (tiles of 4 queries).
#ifndef SWGQA_Q8_MFMA
#define SWGQA_Q8_MFMA 1
#endif

typedef float q8f4 __attribute__((ext_vector_type(4)));
typedef _Float16 q8h4 __attribute__((ext_vector_type(4)));

// VB bytes (4, 8 or 16) at a global address, non-temporal, in the first
// VB / 4 words.
template <int VB>
__device__ __forceinline__ u32x4 load_codes_global(uint64_t addr) {
  u32x4 r = {0u, 0u, 0u, 0u};
  if constexpr (VB == 16) {
    r = load16_global<1>(addr);
  } else if constexpr (VB == 8) {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const u2 v = __builtin_nontemporal_load((const u2 __attribute__((address_space(1)))*)addr);
    r[0] = v[0];
    r[1] = v[1];
  } else {
    r[0] = __builtin_nontemporal_load((const uint32_t __attribute__((address_space(1)))*)addr);
  }
  return r;
}

template <int D, int NQ>
struct Q8Shape {
  static constexpr int EPL = 16;                           // codes per lane per row
  static constexpr int LPR = D / 16;                       // lanes per row
  static constexpr int RPW = kWave / (LPR > 0 ? LPR : 1);  // rows per load instruction
  // loads per stage: SWGQA_Q8_UMUL x (LPR / NQ), so that a stage's fixed
  // cost (the softmax step) is spread over more rows than a 16-bit stage
  static constexpr int U = (SWGQA_Q8_UMUL * LPR / NQ) >= 1 ? (SWGQA_Q8_UMUL * LPR / NQ) : 1;
  static constexpr int SR = RPW * U;                       // rows per wave stage
  static constexpr int PAIRS = SR * NQ;                    // (row, query) pairs per stage
  static constexpr int PPL = PAIRS / kWave;                // pairs per lane
  static constexpr bool ok = D % 16 == 0 && LPR >= 1 && LPR <= 16 && NQ * EPL <= 64 &&
                             PAIRS % kWave == 0;
};

__device__ __forceinline__ void wave_lds_fence_q8() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int CTRL>
__device__ __forceinline__ float dpp_q8(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Max / sum over the lanes that share (lane % NQ).
template <int NQ, bool MAX>
__device__ __forceinline__ float allreduce_q8(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  if constexpr (NQ <= 1) x = op(x, dpp_q8<0xB1>(x));    // quad_perm [1,0,3,2]
  if constexpr (NQ <= 2) x = op(x, dpp_q8<0x4E>(x));    // quad_perm [2,3,0,1]
  if constexpr (NQ <= 4) x = op(x, dpp_q8<0x124>(x));   // row_ror:4
  if constexpr (NQ <= 8) x = op(x, dpp_q8<0x128>(x));   // row_ror:8
  if constexpr (NQ <= 16) x = reduce_xor16(x, op);
  if constexpr (NQ <= 32) x = reduce_xor32(x, op);
  return x;
}

// Two codes (exact as floats) as one packed pair of the 16-bit type: the
// upper half of each float for bf16 (one byte permute), a conversion for fp16
// (integers of at most 8 bits and E4M3 values are exact in both).
template <int DT>
__device__ __forceinline__ uint32_t pack_pair16(float lo, float hi) {
  if constexpr (DT == kBF16) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
}

// One 16 x 16 x 32 product of the 16-bit type on the matrix cores: lane l
// supplies row l % 16 of A and column l % 16 of B, with 8 elements each of
// the 32-element reduction; the result holds column l % 16 and rows
// 4 (l / 16) + [0, 4).
template <int DT>
__device__ __forceinline__ q8f4 mfma16x32(const u32x4& a, const u32x4& b, q8f4 c) {
  if constexpr (DT == kBF16) {
    typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, a),
                                                   __builtin_bit_cast(bf8, b), c, 0, 0, 0);
  } else {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a),
                                                  __builtin_bit_cast(h8, b), c, 0, 0, 0);
  }
}

// Packed dot of two 16-bit pairs, accumulated in fp32.
template <int DT>
__device__ __forceinline__ float dot2_16(uint32_t a, uint32_t b, float acc) {
  if constexpr (DT == kBF16) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, a), __builtin_bit_cast(bf2, b),
                                           acc, false);
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), acc,
                                  false);
  }
}

template <int DT, int D, int NQ, int kWaves, int CT>
__global__ __launch_bounds__(kWaves * kWave)
__attribute__((amdgpu_waves_per_eu((kWaves + 3) / 4, 8))) void attn_decode_q8_kernel(AttnArgs a) {
  constexpr int kThreads = kWaves * kWave;
  using Sh = Q8Shape<D, NQ>;
  constexpr int EPL = Sh::EPL, LPR = Sh::LPR, RPW = Sh::RPW, U = Sh::U;
  constexpr int SR = Sh::SR, PAIRS = Sh::PAIRS, PPL = Sh::PPL;
  constexpr int e = Elem<DT>::bytes;
  constexpr int W16 = D / 16;  // 16-byte chunks per cache row
  static_assert(Sh::ok, "unsupported int8 decode shape");
  // value sums as packed fp16 dot products over row pairs (16-bit outputs)
  constexpr bool PV16 = DT != kF32 && U % 2 == 0 && SWGQA_Q8_PV16;
  // Key scores on the matrix cores: a stage's 16 rows against the tile's 4
  // queries (each repeated in 4 of the 16 columns), D / 32 products of
  // 32 elements.  Lane l loads row l % 16, chunks (l / 16) % 4 + 4 u of it,
  // and keeps the score of row l / 4 and query l % 4.
  constexpr bool MK = DT != kF32 && NQ == 4 && D >= 64 && SR == 16 && SWGQA_Q8_MFMA;
  constexpr int KM = D / 32;
  static_assert(!MK || (U == D / 64 && PPL == 1), "matrix-core key path shape");
  // Value sums on the matrix cores (with the key path): O[q][d] +=
  // P[q][16 rows] . V[16 rows][d] as D / 16 products of 16 x 16 x 16 in
  // fp16 -- A holds P (query l % 4 in row l % 16), B the codes.  Lane l
  // loads rows 4 (l / 16) + [0, 4), bytes [VB (l % 16), VB (l % 16) + VB)
  // of each; product t takes byte t, so the lane's result column is
  // element VB (l % 16) + t, and every lane group holds all 4 queries.
  // P is rounded to fp16 once and the normaliser sums the rounded values.
  constexpr bool MV = MK;
  constexpr int VB = D / 16;              // code bytes per lane and row
  constexpr int UV = MV ? 4 : U;          // value loads per lane and stage
  constexpr bool PROUND = MV || PV16;     // P rounded to fp16

  const uint32_t T = gridDim.x;  // ntiles * nsplit
  const uint32_t P = xcd_contiguous(blockIdx.x + T * (blockIdx.y + gridDim.y * blockIdx.z),
                                    T * gridDim.y * gridDim.z);
  const uint32_t slice = div_gap(P, a.tdiv);
  const uint32_t t = P - slice * T;
  const int b = (int)div_gap(slice, a.hdiv);
  const int kvh = (int)slice - b * a.Hkv;
  const int32_t seqlen = load_seqlen(a.seqlens, b);
  const int tile = a.nsplit == 1 ? (int)t : (int)div_gap(t, a.sdiv);
  const int split = (int)t - tile * a.nsplit;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int rslot = lane / LPR;
  const int sub = lane % LPR;

  __shared__ float s_part[kWaves][MK ? 1 : NQ * SR * LPR];   // [q][row][sub]
  __shared__ __attribute__((aligned(16))) float s_p[kWaves][PAIRS];  // [row][q] ([q][row] on the matrix-core path)
  __shared__ float s_corr[kWaves][NQ];
  __shared__ float s_m[kWaves][NQ];
  __shared__ float s_l[kWaves][NQ];
  __shared__ float s_acc[kWaves][NQ][D];
  __shared__ u32x4 s_knew[kQ8MaxNewRows * W16];     // codes of the new rows
  __shared__ u32x4 s_vnew[kQ8MaxNewRows * W16];

  const int nq_item = a.S * a.group;
  const int q0 = tile * NQ;
  // Query tile: elements [sub * 16, sub * 16 + 16) of each pair, as 16
  // words (fp32) or 8 packed pairs (fp16 / bf16); pairs walked
  // position-major with a carry.
  const int i_first = (int)div_gap((uint32_t)q0, a.qdiv);
  int i_last = i_first;
  constexpr int QW = EPL * e / 4;  // words of a query chunk
  uint32_t qw[MK ? 1 : NQ][QW];
  // matrix-core path: operand m holds elements 16 ((l / 16) % 4 + 4 (m / 2))
  // + 8 (m % 2) + [0, 8) of query l % 4
  u32x4 qb[MK ? KM : 1];
  {
    int h = q0 - i_first * a.group;
    int64_t my_row = 0;
#pragma unroll
    for (int tq = 0; tq < NQ; ++tq) {
      const int64_t row = ((int64_t)b * a.S + i_last) * a.Hq + kvh * a.group + h;
      if constexpr (MK) {
        if ((lane & 3) == tq) my_row = row;
      } else {
        const char* qp = (const char*)a.q + (row * D + sub * EPL) * e;
#pragma unroll
        for (int i = 0; i < QW / 4; ++i) {
          const u32x4 v = *(const u32x4*)(qp + i * 16);
#pragma unroll
          for (int w = 0; w < 4; ++w) qw[tq][4 * i + w] = v[w];
        }
      }
      if (tq + 1 < NQ && q0 + tq + 1 < nq_item && ++h == a.group) {
        h = 0;
        ++i_last;
      }
    }
    if constexpr (MK) {
      const char* qp = (const char*)a.q + (my_row * D + ((lane >> 4) & 3) * 16) * e;
#pragma unroll
      for (int m = 0; m < KM; ++m) qb[m] = *(const u32x4*)(qp + ((m >> 1) * 64 + (m & 1) * 8) * e);
    }
  }
  // The S new K and V rows, one element per thread and pass (their loads
  // do not depend on the plan), quantized into the LDS rows.
  {
    uint8_t* kn8 = (uint8_t*)s_knew;
    uint8_t* vn8 = (uint8_t*)s_vnew;
    const int nel = a.S * D;
    for (int f = tid; f < 2 * nel; f += kThreads) {
      const bool is_v = f >= nel;
      const int r = is_v ? f - nel : f;
      const int i = r / D, d = r % D;
      const int64_t at = ((int64_t)(b * a.S + i) * a.Hkv + kvh) * D + d;
      const float x = load_one<DT>(is_v ? a.v : a.k, at);
      (is_v ? vn8 : kn8)[r] = (uint8_t)quant_code_t<CT>(x, is_v ? a.v_scale : a.k_scale);
    }
  }
  const ItemPlan pl = plan_item(seqlen, a.S, a.C, a.gdiv, a.total);

  if (!pl.ok) {
    if (tid == 0 && tile == 0 && split == 0 && kvh == 0) flag_status(a.status, kStatusBadItem);
    for (int idx = tid; idx < NQ * D; idx += kThreads) {
      const int tq = idx / D, d = idx % D;
      const int qi = q0 + tq;
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

  __syncthreads();  // the new rows' codes are in LDS
  // Appended by tile 0 of split 0 on drifting steps (shared buffer): rows
  // [Lb, Lb + S) lie beyond every row this step reads.
  const bool appender = a.present_k != nullptr && tile == 0 && split == 0;
  if (appender && pl.shift == 0) {
    for (int c = tid; c < a.S * W16; c += kThreads) {
      const int64_t dst = ((int64_t)(b * a.Hkv + kvh) * a.C + pl.Lb + c / W16) * D + (c % W16) * 16;
      *(u32x4*)((char*)a.present_k + dst) = s_knew[c];
      *(u32x4*)((char*)a.present_v + dst) = s_vnew[c];
    }
  }

  const int my_q = lane % NQ;
  const int my_qi = q0 + my_q;
  const bool my_q_ok = my_qi < nq_item;
  const int my_qd = (int)div_gap((uint32_t)my_qi, a.qdiv);  // (divisions by invariants)
  const int my_i = my_q_ok ? my_qd : i_last;
  const int my_h = kvh * a.group + (my_q_ok ? my_qi - my_qd * a.group : 0);
  const int64_t my_pos = pl.P + my_i;

  // Union key range of the tile, split evenly.
  const int64_t p_first = pl.P + i_first;
  const int64_t p_last = pl.P + i_last;
  const int64_t lo = p_first - a.W + 1 > 0 ? p_first - a.W + 1 : 0;
  const int64_t n = p_last - lo + 1;
  const int64_t chunk =
      a.nsplit == 1 ? n : (int64_t)(((uint32_t)n + (uint32_t)a.nsplit - 1u) / (uint32_t)a.nsplit);
  const int64_t kb = lo + split * chunk;
  const int64_t ke = kb + chunk < p_last + 1 ? kb + chunk : p_last + 1;
  const int32_t nk = ke > kb ? (int32_t)(ke - kb) : 0;  // keys kb + jr, 0 <= jr < nk
  const int nst = (nk + SR - 1) / SR;
  const int32_t ncache = (int32_t)(pl.P - kb < 0 ? 0 : (pl.P - kb < nk ? pl.P - kb : nk));
  const int knew0 = (int)(kb - pl.P);  // new row of key jr >= ncache: knew0 + jr

  const int64_t vlo = my_pos - a.W + 1 - kb;
  const int64_t vhi = (my_pos < ke - 1 ? my_pos : ke - 1) - kb;
  const int32_t vis_lo = my_q_ok ? (int32_t)(vlo < -(int64_t)0x7fffffff ? -0x7fffffff : vlo) : 1;
  const int32_t vis_hi = my_q_ok ? (int32_t)vhi : 0;

  // Cache row of key jr < ncache: kb + jr - (P - Lb).  Keys of new rows load
  // a resident row instead (row min(jr, ncache - 1), or row 0 of the slice
  // when no key of the range is resident) and take their codes from LDS.
  constexpr int kRowShift = __builtin_ctz(D);
  const int64_t slice_base = (int64_t)(b * a.Hkv + kvh) * a.C;
  const int64_t first_row = ncache > 0 ? kb - (pl.P - pl.Lb) : 0;
  const uint32_t last_res = ncache > 0 ? (uint32_t)(ncache - 1) : 0u;
  const uint64_t ck_base = (uint64_t)a.past_k + (uint64_t)((slice_base + first_row) << kRowShift);
  const uint64_t ck_lane = ck_base + sub * 16;
  const uint64_t dv = (uint64_t)a.past_v - (uint64_t)a.past_k;
  // matrix-core path: K row lane % 16, chunks (lane / 16) % 4 + 4 u
  const int krow = lane & 15;
  const int kchunk = (lane >> 4) & 3;
  const uint64_t ckm_lane = ck_base + kchunk * 16;

  const bool has_cap = a.softcap > 0.0f;
  const float cap = a.softcap;
  const float inv_cap = a.inv_softcap;  // (made on the host)
  const bool has_bias = a.bias != nullptr;
  const int64_t bias_row = has_bias
      ? ((((a.bias_b ? (int64_t)b : 0) * (a.bias_h ? a.Hq : 1) + (a.bias_h ? my_h : 0)) * a.S + my_i) *
         (int64_t)a.total)
      : 0;
  const float qk_scale = a.scale * a.k_scale;

  float m_run = -INFINITY;
  float l_run = 0.0f;
  float acc[MV ? 1 : NQ][EPL];
#pragma unroll
  for (int tq = 0; tq < (MV ? 1 : NQ); ++tq)
#pragma unroll
    for (int k = 0; k < EPL; ++k) acc[tq][k] = 0.0f;
  q8f4 o[MV ? VB : 1];  // matrix-core value sums: [t][query]
#pragma unroll
  for (int t = 0; t < (MV ? VB : 1); ++t) o[t] = q8f4{0.0f, 0.0f, 0.0f, 0.0f};
  // matrix-core value path: rows 4 (lane / 16) + r, bytes from VB (lane % 16)
  const int vg = lane >> 4;
  const int vc = lane & 15;

  float* part = s_part[wave];
  float* pbuf = s_p[wave];
  float* cbuf = s_corr[wave];

  // Loads of one stage, issued unconditionally at clamped resident rows.
  auto load_stage = [&](int st, u32x4 (&kr)[U], u32x4 (&vr)[UV]) __attribute__((always_inline)) {
    const uint32_t s0 = (uint32_t)min(st, nst) * SR;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t jr = min(s0 + u * RPW + rslot, last_res);
      const uint64_t ka = ck_lane + ((uint64_t)jr << kRowShift);
      if constexpr (MK) {
        const uint32_t jk = min(s0 + krow, last_res);
        kr[u] = load16_global<1>(ckm_lane + ((uint64_t)jk << kRowShift) + u * 64);
      } else {
        kr[u] = load16_global<1>(ka);
      }
      if constexpr (!MV) vr[u] = load16_global<1>(ka + dv);
    }
    if constexpr (MV) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t jv = min(s0 + 4 * vg + r, last_res);
        vr[r] = load_codes_global<VB>(ck_base + dv + ((uint64_t)jv << kRowShift) + VB * vc);
      }
    }
  };

  auto compute_stage = [&](int st, u32x4 (&kr)[U], u32x4 (&vr)[UV]) __attribute__((always_inline)) {
    const uint32_t s0 = (uint32_t)st * SR;
    if (s0 + SR > (uint32_t)ncache) {  // uniform: the stage reaches new rows
      // branch-free per lane: every lane reads LDS (a clamped row) and
      // selects, so no register with a load in flight is overwritten
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t jr = min(s0 + u * RPW + rslot, (uint32_t)(nk - 1));
        const bool is_new = jr >= (uint32_t)ncache;
        const int r = is_new ? knew0 + (int)jr : 0;
        if constexpr (!MV) {
          const u32x4 vn = s_vnew[r * W16 + sub];
#pragma unroll
          for (int w = 0; w < 4; ++w) vr[u][w] = is_new ? vn[w] : vr[u][w];
        }
        if constexpr (MK) {
          const uint32_t jk = min(s0 + krow, (uint32_t)(nk - 1));
          const bool k_new = jk >= (uint32_t)ncache;
          const int rk = k_new ? knew0 + (int)jk : 0;
          const u32x4 kn = s_knew[rk * W16 + kchunk + 4 * u];
#pragma unroll
          for (int w = 0; w < 4; ++w) kr[u][w] = k_new ? kn[w] : kr[u][w];
        } else {
          const u32x4 kn = s_knew[r * W16 + sub];
#pragma unroll
          for (int w = 0; w < 4; ++w) kr[u][w] = is_new ? kn[w] : kr[u][w];
        }
      }
      if constexpr (MV) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t jv = min(s0 + 4 * vg + r, (uint32_t)(nk - 1));
          const bool v_new = jv >= (uint32_t)ncache;
          const int rv = v_new ? knew0 + (int)jv : 0;
          const uint32_t* vn = (const uint32_t*)s_vnew + (rv * D + VB * vc) / 4;
#pragma unroll
          for (int w = 0; w < VB / 4; ++w) vr[r][w] = v_new ? vn[w] : vr[r][w];
        }
      }
    }
    // A. scores: matrix-core products, or partial dots over 16 codes -> LDS
    // [q][row][sub]
    q8f4 sacc = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (MK) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float kf[EPL];
#pragma unroll
        for (int w = 0; w < 4; ++w) codes4_t<CT>(kr[u][w], kf + 4 * w);
        u32x4 lo, hi;  // codes 0..7 and 8..15 of the chunk as 16-bit pairs
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lo[j] = pack_pair16<DT>(kf[2 * j], kf[2 * j + 1]);
          hi[j] = pack_pair16<DT>(kf[8 + 2 * j], kf[9 + 2 * j]);
        }
        sacc = mfma16x32<DT>(lo, qb[2 * u], sacc);
        sacc = mfma16x32<DT>(hi, qb[2 * u + 1], sacc);
      }
    } else {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = u * RPW + rslot;
      float kf[EPL];
#pragma unroll
      for (int w = 0; w < 4; ++w) codes4_t<CT>(kr[u][w], kf + 4 * w);
      if constexpr (DT == kF32) {
#pragma unroll
        for (int tq = 0; tq < NQ; ++tq) {
          float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
          for (int k = 0; k < EPL; k += 2) {
            d0 = fmaf(__uint_as_float(qw[tq][k]), kf[k], d0);
            d1 = fmaf(__uint_as_float(qw[tq][k + 1]), kf[k + 1], d1);
          }
          part[(tq * SR + row) * LPR + sub] = d0 + d1;
        }
      } else {
        uint32_t kp[EPL / 2];  // the codes as packed 16-bit pairs (exact)
#pragma unroll
        for (int j = 0; j < EPL / 2; ++j) kp[j] = pack_pair16<DT>(kf[2 * j], kf[2 * j + 1]);
#pragma unroll
        for (int tq = 0; tq < NQ; ++tq) {
          float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
          for (int j = 0; j < EPL / 2; j += 2) {
            d0 = dot2_16<DT>(qw[tq][j], kp[j], d0);
            d1 = dot2_16<DT>(qw[tq][j + 1], kp[j + 1], d1);
          }
          part[(tq * SR + row) * LPR + sub] = d0 + d1;
        }
      }
    }
    wave_lds_fence_q8();
    }
    // B. scores, stage max, probabilities
    float s[PPL];
    float smax = -INFINITY;
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      const int pid = lane + k * kWave;
      const int row = pid / NQ;
      float x = 0.0f;
      if constexpr (MK) {
        const int rs = (lane >> 2) & 3;  // row lane / 4 of the product
        x = rs == 0 ? sacc[0] : rs == 1 ? sacc[1] : rs == 2 ? sacc[2] : sacc[3];
      } else {
        const float* pp = part + (my_q * SR + row) * LPR;
#pragma unroll
        for (int w = 0; w < LPR; ++w) x += pp[w];
      }
      x *= qk_scale;
      const int32_t jr = st * SR + row;
      const bool vis = jr >= vis_lo && jr <= vis_hi;
      if (has_cap) {
        const float y = x * inv_cap;
        if constexpr (DT == kF32) {
          x = cap * tanhf(y);
        } else {
          const float tt = 1.0f - 2.0f * __builtin_amdgcn_rcpf(
                                      __builtin_amdgcn_exp2f(2.0f * kLog2e * fabsf(y)) + 1.0f);
          x = cap * copysignf(tt, y);
        }
      }
      if (has_bias && vis) x += load_one<DT>(a.bias, bias_row + kb + jr);
      s[k] = vis ? x * kLog2e : -INFINITY;
      smax = fmaxf(smax, s[k]);
    }
    smax = allreduce_q8<NQ, true>(smax);
    const float m_new = fmaxf(m_run, smax);
    const float corr = (m_run == m_new) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.0f;
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      float p = (s[k] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(s[k] - m_new);
      // PV16: P enters the value sum rounded to fp16 and the normaliser sums
      // the rounded P, so the output stays an exact weighted mean
      if constexpr (PROUND) p = (float)(_Float16)p;
      if constexpr (MV) pbuf[(lane & 3) * 16 + (lane >> 2)] = p;  // [q][row]
      else pbuf[lane + k * kWave] = p;
      psum += p;
    }
    l_run = l_run * corr + psum;
    m_run = m_new;
    if (lane < NQ) cbuf[lane] = corr;
    wave_lds_fence_q8();
    // C. rescale and accumulate the value codes
    float cr[NQ];
    bool rescale = false;
#pragma unroll
    for (int tq = 0; tq < NQ; ++tq) {
      cr[tq] = cbuf[tq];
      rescale |= cr[tq] != 1.0f;
    }
    if constexpr (MV) {
      if (rescale) {
#pragma unroll
        for (int t = 0; t < VB; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[t][r] *= cr[r];
      }
      // A: P of query lane % 4 at rows 4 (lane / 16) + [0, 4)
      const q8f4 pv = *(const q8f4*)(pbuf + (lane & 3) * 16 + 4 * vg);
      const uint2 pa = make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pv[0], pv[1])),
                                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pv[2], pv[3])));
      float vf[4][VB];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int w = 0; w < VB / 4; ++w) codes4_t<CT>(vr[r][w], vf[r] + 4 * w);
#pragma unroll
      for (int t = 0; t < VB; ++t) {
        const uint2 vb = make_uint2(
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(vf[0][t], vf[1][t])),
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(vf[2][t], vf[3][t])));
        o[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(q8h4, pa),
                                                      __builtin_bit_cast(q8h4, vb), o[t], 0, 0, 0);
      }
    } else {
    if (rescale) {
#pragma unroll
      for (int tq = 0; tq < NQ; ++tq)
#pragma unroll
        for (int k = 0; k < EPL; ++k) acc[tq][k] *= cr[tq];
    }
    if constexpr (PV16) {
      // two rows at a time: (p_a, p_b) . (v_a[k], v_b[k]) as one packed fp16
      // dot product per query and element (codes are exact in fp16)
#pragma unroll
      for (int u = 0; u < U; u += 2) {
        const int ra = u * RPW + rslot, rb = ra + RPW;
        uint32_t pp[NQ];
#pragma unroll
        for (int tq = 0; tq < NQ; ++tq)
          pp[tq] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pbuf[ra * NQ + tq],
                                                                           pbuf[rb * NQ + tq]));
        float va[EPL], vb[EPL];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          codes4_t<CT>(vr[u][w], va + 4 * w);
          codes4_t<CT>(vr[u + 1][w], vb + 4 * w);
        }
#pragma unroll
        for (int k = 0; k < EPL; ++k) {
          const uint32_t vp = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(va[k], vb[k]));
#pragma unroll
          for (int tq = 0; tq < NQ; ++tq) acc[tq][k] = dot2_16<kF16>(pp[tq], vp, acc[tq][k]);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = u * RPW + rslot;
        float pr[NQ];
#pragma unroll
        for (int tq = 0; tq < NQ; ++tq) pr[tq] = pbuf[row * NQ + tq];
        float vf[EPL];
#pragma unroll
        for (int w = 0; w < 4; ++w) codes4_t<CT>(vr[u][w], vf + 4 * w);
#pragma unroll
        for (int tq = 0; tq < NQ; ++tq)
#pragma unroll
          for (int k = 0; k < EPL; ++k) acc[tq][k] = fmaf(pr[tq], vf[k], acc[tq][k]);
      }
    }
    }
    wave_lds_fence_q8();
  };

  // Stages of this wave: wave, wave + kWaves, ...; the loads of the next
  // DEPTH - 1 stages are in flight while one is computed.
  u32x4 k0[U], v0[UV], k1[U], v1[UV];
  int st = wave;
  if (nk == 0) {
    // empty split
  } else if (nst <= kWaves) {
    if (wave < nst) {
      load_stage(wave, k0, v0);
      compute_stage(wave, k0, v0);
    }
  } else if constexpr (SWGQA_Q8_DEPTH == 3) {
    // whole groups of three stages, no exit between them (a stage past the
    // end loads clamped rows and is not computed)
    u32x4 k2[U], v2[UV];
    load_stage(st, k0, v0);
    load_stage(st + kWaves, k1, v1);
    const int groups = (nst - wave + 3 * kWaves - 1) / (3 * kWaves);
    for (int g = 0; g < groups; ++g) {
      load_stage(st + 2 * kWaves, k2, v2);
      compute_stage(st, k0, v0);
      st += kWaves;
      load_stage(st + 2 * kWaves, k0, v0);
      if (st < nst) compute_stage(st, k1, v1);
      st += kWaves;
      load_stage(st + 2 * kWaves, k1, v1);
      if (st < nst) compute_stage(st, k2, v2);
      st += kWaves;
    }
  } else {
    load_stage(st, k0, v0);
    const int groups = (nst - wave + 2 * kWaves - 1) / (2 * kWaves);
    for (int g = 0; g < groups; ++g) {
      load_stage(st + kWaves, k1, v1);
      compute_stage(st, k0, v0);
      st += kWaves;
      load_stage(st + kWaves, k0, v0);
      if (st < nst) compute_stage(st, k1, v1);
      st += kWaves;
    }
  }

  // Wave result, then the merge of the waves.
  const float l_tot = allreduce_q8<NQ, false>(l_run);
  if constexpr (MV) {
    if (lane < 16) {  // lane group 0 holds the 4 queries' sums
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < VB; ++t) s_acc[wave][r][VB * lane + t] = o[t][r];
    }
  } else {
  // (sum over the lanes that share lane % LPR: the row slots)
#pragma unroll
  for (int tq = 0; tq < NQ; ++tq)
#pragma unroll
    for (int k = 0; k < EPL; ++k) acc[tq][k] = allreduce_q8<LPR, false>(acc[tq][k]);
  if (rslot == 0) {
#pragma unroll
    for (int tq = 0; tq < NQ; ++tq)
#pragma unroll
      for (int k = 0; k < EPL; ++k) s_acc[wave][tq][sub * EPL + k] = acc[tq][k];
  }
  }
  if (lane < NQ) {
    s_m[wave][lane] = m_run;
    s_l[wave][lane] = l_tot;
  }
  __syncthreads();

  for (int idx = tid; idx < NQ * D; idx += kThreads) {
    const int tq = idx / D, d = idx % D;
    const int qi = q0 + tq;
    if (qi >= nq_item) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][tq]);
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float c = (s_m[w][tq] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(s_m[w][tq] - M);
      L += s_l[w][tq] * c;
      A += s_acc[w][tq][d] * c;
    }
    A *= a.v_scale;  // the value sum was taken over codes
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

  slice_tail_rows(a, pl, b, kvh, D, 1, s_knew, s_vnew);
}

template <int DT, int D, int NQ, int CT>
hipError_t launch_q8_nq(const AttnArgs& a, hipStream_t st) {
  if constexpr (Q8Shape<D, NQ>::ok) {
    // the new rows' codes live in LDS arrays of kQ8MaxNewRows rows
    if (a.S < 1 || a.S > kQ8MaxNewRows) return hipErrorInvalidValue;
    const dim3 grid(a.ntiles * a.nsplit, a.Hkv, a.B);
    if (a.waves == 8)
      attn_decode_q8_kernel<DT, D, NQ, 8, CT><<<grid, 8 * kWave, 0, st>>>(a);
    else
      attn_decode_q8_kernel<DT, D, NQ, 4, CT><<<grid, 4 * kWave, 0, st>>>(a);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <int DT, int D, int CT>
hipError_t launch_q8_d(int nq, const AttnArgs& a, hipStream_t st) {
  switch (nq) {
    case 2: return launch_q8_nq<DT, D, 2, CT>(a, st);
    case 4: return launch_q8_nq<DT, D, 4, CT>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int CT>
hipError_t launch_q8_t(int D, int nq, const AttnArgs& a, hipStream_t st) {
  switch (D) {
    case 16: return launch_q8_d<DT, 16, CT>(nq, a, st);
    case 32: return launch_q8_d<DT, 32, CT>(nq, a, st);
    case 64: return launch_q8_d<DT, 64, CT>(nq, a, st);
    case 128: return launch_q8_d<DT, 128, CT>(nq, a, st);
    case 256: return launch_q8_d<DT, 256, CT>(nq, a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int CT>
hipError_t launch_q8_ct(int dtype, int D, int nq, const AttnArgs& a, hipStream_t st) {
  switch (dtype) {
    case kF32: return launch_q8_t<kF32, CT>(D, nq, a, st);
    case kF16: return launch_q8_t<kF16, CT>(D, nq, a, st);
    case kBF16: return launch_q8_t<kBF16, CT>(D, nq, a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
int q8_stage_rows_d(int nq) {
  switch (nq) {
    case 2: return Q8Shape<D, 2>::SR;
    case 4: return Q8Shape<D, 4>::SR;
    default: return 1;
  }
}

}  // namespace

}  // namespace swgqa
