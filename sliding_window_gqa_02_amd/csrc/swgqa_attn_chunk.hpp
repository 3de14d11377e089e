// swgqa_attn_chunk.hpp -- grouped-query attention for multi-token steps
// (prefill, chunked prefill, S >= 16) over a windowed KV cache, on the CDNA4
// matrix cores.  Instantiated for element-type caches in
// swgqa_attn_chunk.hip and for int8 caches in swgqa_attn_chunk_q8.hip.
//
// Same contract as the decode kernels: query i of item b at absolute
// position p = P + i attends to keys p - W < j <= p of [resident rows | S
// new rows] ("Specify GroupQueryAttention windowed KV cache layout
// contract", Description; causal rule of "Fix CPU Attention causal mask
// ..."), keys below P read from cache row j - (P - Lb), the rest straight
// from the new rows, so a step that evicts history it still reads needs no
// staging copy ("[CPU] Add windowed kv cache for GQA", staging).
//
// A workgroup (4 or 8 waves, 16 query rows each; or 8 waves in 4 groups of
// 2 that share 32 rows, see GRP) owns consecutive (position, head) query rows
// of one KV head's group and walks the key band [p_first - W + 1, p_last] in
// blocks of 32 keys staged in LDS -- every K/V row staged is used by all the
// heads of the group.  Per block each wave (16 query rows):
//   S^T = K . Q^T   16 keys x 16 queries per MFMA (Q^T is the B operand, held
//                   in registers for the whole band);
//   softmax         each lane owns one query column, so max / sum need only
//                   in-lane work plus two cross-lane steps, and every
//                   (query, key) score is transformed exactly once;
//   O^T += V^T . P^T  the S^T accumulator registers are the P^T operand as
//                   they stand (keys on the reduction axis), and O^T keeps
//                   the same one-query-per-lane-column layout as the softmax
//                   state, so rescaling needs no shuffles.
// fp32 uses v_mfma_f32_16x16x4_f32 (full fp32 products); fp16 / bf16 use the
// 16x16x16 forms.  P enters the PV product rounded to fp16 (the normaliser
// sums the rounded P, so the result is an exact weighted mean of V), or for
// bf16 as a hi + lo pair of bf16 values (8 significant bits alone would move
// a mean of few keys by ~2^-9).
// The next block's K/V are loaded into registers while the current block is
// computed.
//
// With an int8 cache (Q8; the Investigation Report, section 1.1, names
// k_scale / v_scale; reading: element = code * scale, new elements quantized
// with ties to even and saturation) every key row is read as codes -- the
// cache rows, and the step's new rows from a workspace copy the quantization
// pass wrote -- 16 / e codes where an element-type row has 16 bytes; the
// codes enter LDS converted to the element type (integers of at most 8 bits
// are exact in fp32, fp16 and bf16), k_scale joins the score scale and
// v_scale the output.
#pragma once

#include "swgqa_common.hpp"
#include "swgqa_internal.hpp"
#include "swgqa_tail.hpp"

#include <math.h>
#include <stdint.h>
#include <type_traits>

namespace swgqa {

namespace {

// A workgroup of NW waves (4 or 8) owns 16 NW query rows (16 NW / GRP with
// wave groups).
constexpr int BN = 32;   // keys per block
constexpr float kLog2e = 1.4426950408889634f;

typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

// C += A B over a reduction of 32 (gfx950's 16x16x32 products, twice the
// work per instruction of the 16x16x16 ones): lane i + 16 g holds row i of A
// and column i of B, each at reduction elements 8 g .. 8 g + 7 in its 8
// halves, so any assignment of reduction indices to (g, element) that A and
// B share gives the same sum.
template <int DT>
__device__ __forceinline__ f4 mfma_x32(const uint4& a, const uint4& b, const f4& c) {
  if constexpr (DT == kF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a),
                                                  __builtin_bit_cast(h8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a),
                                                   __builtin_bit_cast(b8, b), c, 0, 0, 0);
}

template <int DT, int D, int NW>
struct ChunkShape {
  static constexpr int kThreads = NW * kWave;
  static constexpr int e = Elem<DT>::bytes;
  // LDS row strides (elements), chosen so the MFMA operand reads of 16 lanes
  // on 16 different rows fall in distinct banks
  static constexpr int KS = (DT == kF32) ? D + 4 : D + 8;   // K rows: [key][d]
  static constexpr int VS = (DT == kF32) ? D + 4 : BN + 8;  // fp32 V [key][d]; 16-bit V^T [d][key]
  static constexpr int KELEMS = BN * KS;
  static constexpr int VELEMS = (DT == kF32) ? BN * VS : D * VS;
  static constexpr int CHUNKS = BN * D * e / 16;           // 16-byte chunks per block per tensor
  static constexpr int CPT = (CHUNKS + kThreads - 1) / kThreads;  // per thread
  static constexpr int DSTEPS = (DT == kF32) ? D / 4 : D / 16;  // S^T MFMA steps
  static constexpr int DT16 = D / 16;                      // O^T tiles
  static constexpr bool ok = D >= 16 && D % 16 == 0 && D * e <= 512;
};

template <int DT> struct LdsT { using T = float; };
template <> struct LdsT<kF16> { using T = uint16_t; };
template <> struct LdsT<kBF16> { using T = uint16_t; };

// Key swizzle of row d of the transposed V tile (16-bit types): XOR of key
// bits 3..4 with (d / 8) mod 4, so groups of 8 consecutive keys stay
// contiguous and in order.
__device__ __forceinline__ int vt_swizzle(int d) { return ((d >> 3) & 3) << 3; }

// 16-bit types: row i of the block's score tile kt holds key 8 (i / 4) +
// 4 kt + i % 4, so lane group g, which receives rows 4g .. 4g + 3 of both
// tiles, holds keys 8g .. 8g + 7 -- one contiguous run of the block, for its
// attention_bias entries and its part of the 32-key value products.  K is
// staged in that order (key k at LDS row k_slot(k) = 16 kt + i), so the score
// products read consecutive rows.  fp32 keeps key 16 kt + i (its value
// products run per tile, and a second tile past the band's end is skipped).
template <int DT>
__device__ __forceinline__ int k_slot(int k) {
  if constexpr (DT == kF32) return k;
  else return 16 * ((k >> 2) & 1) + 4 * (k >> 3) + (k & 3);
}
// The key of score r (0..3) of tile kt in lane group g.
template <int DT>
__device__ __forceinline__ int score_key(int kt, int g, int r) {
  if constexpr (DT == kF32) return 16 * kt + 4 * g + r;
  else return 8 * g + 4 * kt + r;
}

// Key and 16-byte part of chunk c of a staged block whose rows are CPR
// chunks long.  In every 64 chunks (one wave's), lane group g = (c / 16) % 4
// holds key 4 q + g at the same parts as the other three groups (keys 4 q ..
// 4 q + 3: what the transposed V store exchanges across lane groups), and
// the 16 lanes of a group run along rows, so each row's chunks stay
// contiguous in memory.
template <int CPR>
__device__ __forceinline__ int chunk_key(int c) {
  const int g = (c >> 4) & 3, p = c & 15, unit = c >> 6;
  if constexpr (CPR >= 16) return 4 * (unit / (CPR / 16)) + g;
  else return 4 * (unit * (16 / CPR) + p / CPR) + g;
}
template <int CPR>
__device__ __forceinline__ int chunk_part(int c) {
  const int p = c & 15, unit = c >> 6;
  if constexpr (CPR >= 16) return 16 * (unit % (CPR / 16)) + p;
  else return p % CPR;
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  union { _Float16 h; uint16_t u; } c;
  c.h = (_Float16)x;
  return c.u;
}

// BIAS: attention_bias present (a separate instantiation, so that the loads
// of a block are the same on every path and the compiler can wait for
// exactly the block it stages).
// 16 / e codes (4 bytes for fp32, 8 for fp16 / bf16) at a global address, in
// the low words of a chunk register.
template <int DT>
__device__ __forceinline__ u32x4 load_codes(uint64_t addr) {
  u32x4 r = {0u, 0u, 0u, 0u};
  if constexpr (DT == kF32) {
    r[0] = *(const uint32_t __attribute__((address_space(1)))*)addr;
  } else {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = *(const u32x2 __attribute__((address_space(1)))*)addr;
    r[0] = v[0];
    r[1] = v[1];
  }
  return r;
}

// Codes (low words of c) as the element type, one 16-byte chunk: exact
// (int8 integers and fp8 E4M3 values are fp32, fp16 and bf16 numbers).
template <int DT, int CT>
__device__ __forceinline__ u32x4 codes_to_elems(const u32x4& c) {
  u32x4 r;
  if constexpr (DT == kF32) {
    float x[4];
    codes4_t<CT>(c[0], x);
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(x[i]);
  } else {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      float x[4];
      codes4_t<CT>(c[w], x);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float lo = x[2 * h], hi = x[2 * h + 1];
        if constexpr (DT == kBF16)
          r[2 * w + h] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
        else
          r[2 * w + h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
      }
    }
  }
  return r;
}

// CT: 0 for a cache in the element type, else the code type of the cache.
#ifndef SWGQA_CHUNK_DB_ALL
#define SWGQA_CHUNK_DB_ALL 0
#endif

// Blocks of loads in flight, 16-bit rows of under 512 bytes.
#ifndef SWGQA_CHUNK_RING16
#define SWGQA_CHUNK_RING16 3
#endif

// Two LDS buffers per block (fp32), else one staged between two barriers.
template <int DT>
constexpr bool chunk_double_buffer() { return SWGQA_CHUNK_DB_ALL || DT == kF32; }
// Whether the kernel's key splits can move a compacting slice's surviving
// rows (one LDS buffer, a cache in the element type).
template <int DT, int CT>
constexpr bool chunk_split_moves() { return !chunk_double_buffer<DT>() && CT == 0; }

// Waves per SIMD the compiler must leave room for: fp32 with rows of at
// most 256 bytes, 4 in 8-wave workgroups without bias (its operands fit 128
// registers with two blocks of loads in flight; measured faster than 2 or 3
// waves) and 3 otherwise (the bias path and 4-wave workgroups need a little
// more); 16-bit rows of at most 128 bytes in 8-wave workgroups without bias,
// 4 (two workgroups per CU); no floor for the other shapes.
// Blocks of loads in flight in the register ring: three (16-bit rows under
// 512 bytes, tunable; fp32 rows of at most 256 bytes, except 4-wave
// workgroups with bias, which would spill), else two, which keeps the rest
// within the registers of their occupancy.
template <int DT, int D, int NW, bool BIAS>
constexpr int chunk_ring() {
  if constexpr (DT == kF32) return D <= 64 && !(BIAS && NW == 4) ? 3 : 2;
  else return D * 2 >= 512 ? 2 : SWGQA_CHUNK_RING16;
}

template <int DT, int D, int NW, bool BIAS, int GRP = 1>
constexpr int chunk_min_waves() {
  if constexpr (GRP > 1) return 1;  // (its register ring is GRP blocks deep per round)
  else if constexpr (DT == kF32) return D <= 64 ? (NW == 8 && !BIAS ? 4 : 3) : 1;
  else return D <= 64 && NW == 8 && !BIAS ? 4 : 1;
}

// GRP > 1: the waves form GRP groups of NW / GRP waves; every group holds
// the tile's query rows (16 per wave) and computes every GRP-th block of the
// split, so a split of n blocks takes ceil(n / GRP) staging rounds; the
// groups' softmax states are merged in LDS at the end.  For tiles of few
// query rows (short multi-token steps), whose waves would otherwise walk the
// band one block after another with nothing to overlap.
template <int DT, int D, bool BIAS, int NW, int CT, int GRP = 1>
__global__ __launch_bounds__(NW * kWave)
__attribute__((amdgpu_waves_per_eu(chunk_min_waves<DT, D, NW, BIAS, GRP>(), 8)))
void attn_chunk_kernel(AttnArgs a) {
  constexpr bool Q8 = CT != 0;
  using Sh = ChunkShape<DT, D, NW>;
  constexpr int kThreads = Sh::kThreads;
  constexpr int NWQ = NW / GRP;  // waves per group
  constexpr int BQ = 16 * NWQ;   // query rows per workgroup
  static_assert(NW % GRP == 0, "whole groups of waves");
  using LT = typename LdsT<DT>::T;
  constexpr int e = Sh::e, KS = Sh::KS, VS = Sh::VS, CPT = Sh::CPT, DSTEPS = Sh::DSTEPS;
  constexpr int DT16 = Sh::DT16;
  constexpr int CPR = D * e / 16;  // 16-byte element chunks per row
  constexpr int CE = Q8 ? 1 : e;   // bytes of a cache (or new-row copy) element
  constexpr int CPRC = D * CE / 16;  // 16-byte chunks per cache row
  static_assert(Sh::ok, "unsupported chunk shape");
  static_assert(!Q8 || D >= 16, "int8 rows of whole 16-byte chunks");

  // DB (fp32): two K/V buffers, block blk staged in buffer blk & 1 while the
  // other holds the block being computed; 16-bit types stage every block in
  // one buffer between two barriers (measured faster for them)
  constexpr bool DB = chunk_double_buffer<DT>();
  static_assert(GRP == 1 || !DB, "wave groups stage one buffer per group");
  constexpr int NBUF = DB ? 2 : GRP;
  __shared__ __attribute__((aligned(16))) LT sK[NBUF * Sh::KELEMS];
  __shared__ __attribute__((aligned(16))) LT sV[NBUF * Sh::VELEMS];

  // work item P of the launch: slice P / T, item (tile, split) P % T
  const uint32_t T = gridDim.x;  // ntiles * nsplit
  const uint32_t P = xcd_contiguous(blockIdx.x + T * (blockIdx.y + gridDim.y * blockIdx.z),
                                    T * gridDim.y * gridDim.z);
  const uint32_t slice = div_gap(P, a.tdiv);
  const uint32_t t = P - slice * T;
  const int b = (int)div_gap(slice, a.hdiv);
  const int kvh = (int)slice - b * a.Hkv;
  const int tile = (int)div_gap(t, a.sdiv);
  const int split = (int)t - tile * a.nsplit;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int wq = wave % NWQ;   // the wave's query rows: 16 wq .. 16 wq + 15 of the tile
  const int grp = wave / NWQ;  // its group: blocks grp, grp + GRP, ...
  const int lane = tid % kWave;
  const int lq = lane % 16;   // query column of this lane
  const int lg = lane / 16;   // lane group (0..3)

  // seqlens_k first: the plan and every K/V address wait on it
  const int32_t seqlen = load_seqlen(a.seqlens, b);
  // The launch arguments the plan and the addresses use, wanted here (an
  // empty statement that takes them in scalar registers): their scalar
  // loads then go out in one batch with seqlens_k's, not one round trip
  // each where first used behind the plan's branches.
  asm volatile("" ::"s"(a.k), "s"(a.v), "s"(a.past_k), "s"(a.past_v), "s"(a.C), "s"(a.W),
               "s"(a.total), "s"(a.S), "s"(a.Hkv), "s"(a.gdiv.magic), "s"(a.gdiv.G),
               "s"(a.gdiv.sh1), "s"(a.gdiv.sh2));
  const int nq_item = a.S * a.group;
  const int q0 = tile * BQ;

  // This lane's query (column lq of wave's 16 rows), loaded before the
  // plan: its address does not depend on seqlens_k.
  const int my_qi = q0 + wq * 16 + lq;
  const bool my_ok = my_qi < nq_item;
  const int my_qc = my_ok ? my_qi : nq_item - 1;
  // (divisions by invariants)
  const int my_i = (int)div_gap((uint32_t)my_qc, a.qdiv);
  const int my_h = kvh * a.group + my_qc - my_i * a.group;
  const int i_first = (int)div_gap((uint32_t)q0, a.qdiv);
  const int i_last = (int)div_gap((uint32_t)(min(q0 + BQ, nq_item) - 1), a.qdiv);

  // Q^T operand: fp32 step s holds Q[q][(D / 4) lg + s] (the steps split
  // the head dimension as d = (D / 4) k + s over the 4 reduction lanes k, so
  // a lane's K and Q operands are D / 4 consecutive elements); 16-bit step s
  // holds Q[q][32s + 8lg .. +7] (16x16x32 products; D = 16: Q[q][4lg .. +3],
  // one 16x16x16 product).
  constexpr bool QX32 = DT != kF32 && D % 32 == 0;
  constexpr int QST = QX32 ? D / 32 : DSTEPS;  // 16-bit S^T MFMA steps
  const char* qrow = (const char*)a.q + ((((int64_t)b * a.S + my_i) * a.Hq + my_h) * D) * e;
  float qf[DT == kF32 ? DSTEPS : 1];
  uint32_t qh[DT == kF32 ? 1 : QST][QX32 ? 4 : 2];
  if constexpr (DT == kF32) {
#pragma unroll
    for (int s = 0; s < DSTEPS; s += 4) {
      const f4 v = *(const f4*)((const float*)qrow + DSTEPS * lg + s);
      qf[s] = v[0]; qf[s + 1] = v[1]; qf[s + 2] = v[2]; qf[s + 3] = v[3];
    }
  } else if constexpr (QX32) {
#pragma unroll
    for (int s = 0; s < QST; ++s) {
      const uint4 v = *(const uint4*)(qrow + (32 * s + 8 * lg) * 2);
      qh[s][0] = v.x;
      qh[s][1] = v.y;
      qh[s][2] = v.z;
      qh[s][3] = v.w;
    }
  } else {
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s) {
      const uint2 v = *(const uint2*)(qrow + (16 * s + 4 * lg) * 2);
      qh[s][0] = v.x;
      qh[s][1] = v.y;
    }
  }

  const ItemPlan pl = plan_item(seqlen, a.S, a.C, a.gdiv, a.total);
  const int64_t my_pos = pl.P + my_i;

  if (!pl.ok) {
    if (tid == 0 && tile == 0 && split == 0 && kvh == 0) flag_status(a.status, kStatusBadItem);
    for (int idx = tid; idx < BQ * D; idx += kThreads) {
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

  // Key band of the tile and this split's part of it.
  const int64_t p_first = pl.P + i_first;
  const int64_t p_last = pl.P + i_last;
  const int64_t lo = p_first - a.W + 1 > 0 ? p_first - a.W + 1 : 0;
  const int64_t nkeys = p_last - lo + 1;
  // (nkeys + nsplit - 1 < 2^32: the division by invariant)
  const int64_t per =
      ((int64_t)div_gap((uint32_t)(nkeys + a.nsplit - 1), a.sdiv) + BN - 1) / BN * BN;
  const int64_t kb = lo + split * per;
  const int64_t ke = kb + per < p_last + 1 ? kb + per : p_last + 1;

  const int64_t base = pl.P - pl.Lb;
  // (with Q8, a.k / a.v hold the new rows' codes)
  const uint64_t ck = (uint64_t)((const char*)a.past_k + ((int64_t)(b * a.Hkv + kvh) * a.C) * D * CE);
  const uint64_t cv = (uint64_t)((const char*)a.past_v + ((int64_t)(b * a.Hkv + kvh) * a.C) * D * CE);
  const uint64_t nk = (uint64_t)((const char*)a.k + (((int64_t)b * a.S) * a.Hkv + kvh) * D * CE);
  const uint64_t nv = (uint64_t)((const char*)a.v + (((int64_t)b * a.S) * a.Hkv + kvh) * D * CE);
  const int64_t new_stride = (int64_t)a.Hkv * D * CE;

  const bool has_cap = a.softcap > 0.0f;
  const float cap = a.softcap;
  const float inv_cap = a.inv_softcap;  // (made on the host)
  constexpr bool has_bias = BIAS;
  const int64_t bias_row = has_bias
      ? ((((a.bias_b ? (int64_t)b : 0) * (a.bias_h ? a.Hq : 1) + (a.bias_h ? my_h : 0)) * a.S + my_i) *
         (int64_t)a.total)
      : 0;

  // Block loads into registers, issued unconditionally (so the compiler can
  // wait for exactly the loads it needs): chunk c of the block = key
  // chunk_key(c), 16-byte part chunk_part(c); keys past the band's end are
  // clamped to its last key (finite data the mask removes); chunks past the
  // block repeat the last one and are not stored.  The attention_bias entries this lane scores in
  // the block (keys j0 + 16 kt + 4 lg + r) come with them.
  // The bias entries stay raw words until the block is computed: converting
  // them where they are loaded would make every block wait for all loads in
  // flight.
  constexpr int BW = 8 * e / 4;  // words of the 8 bias entries
  // (with wave groups each thread scores another block than most it
  // stages: its bias words are loaded apart, see load_bias)
  struct BlockRegs {
    u32x4 k[CPT], v[CPT];
    uint32_t bias[GRP == 1 ? BW : 1];
  };
  // Per-lane parts of the addresses: chunk u of a block is key kc + j0,
  // 16-byte part pc; blocks made only of cache rows (nearly all) add j0 rows
  // to these, the rest take the two-segment select with clamping.
  constexpr int kRowB = D * CE;
  constexpr int kPartB = Q8 ? 16 / e : 16;  // bytes of a chunk's part of a row
  uint64_t kc_lane[CPT], vc_lane[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int c = min(tid + u * kThreads, Sh::CHUNKS - 1);
    const uint64_t off = (uint64_t)(((int64_t)chunk_key<CPR>(c) - base) * kRowB +
                                    chunk_part<CPR>(c) * kPartB);
    kc_lane[u] = ck + off;
    vc_lane[u] = cv + off;
  }
  // and of new rows: the chunk's key at new row (j0 - P) + key
  uint32_t nw_lane[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int c = min(tid + u * kThreads, Sh::CHUNKS - 1);
    nw_lane[u] = (uint32_t)(chunk_key<CPR>(c) * new_stride + chunk_part<CPR>(c) * kPartB);
  }
  const uint64_t bias_lane =
      BIAS ? (uint64_t)a.bias + (uint64_t)((bias_row + (DT == kF32 ? 4 : 8) * lg) * e) : 0;
  const int64_t cache_end = pl.P < ke ? pl.P : ke;  // keys below this are cache rows

  // Compaction by the key splits (16-bit cache; the host gives a stash only
  // to one-tile launches over a shared buffer, and both sides take the same
  // per-item decision): the surviving rows this split reads, positions
  // [mv_lo, mv_hi), are stored at their new place pos - shift from the block
  // registers once their block is staged -- every load of that block and of
  // the blocks before it has completed by then, and the blocks still to come
  // lie above every row it overwrites; no other split reads this split's
  // rows -- except those below mv_stash, whose new place lies in the previous
  // split's part, possibly still being read: they go to this split's stash
  // slots (pos - kb) for the step tail to store.
  constexpr bool kCanMove = chunk_split_moves<DT, CT>();
  bool fmove = false;
  int64_t mv_lo = 0, mv_hi = 0, mv_stash = 0;
  uint64_t mv_k = 0, mv_v = 0, st_k = 0, st_v = 0;
  if constexpr (kCanMove) {
    fmove = a.stash != nullptr && chunk_moves_rows(pl, a.W, a.stash_rows);
    if (fmove) {
      mv_lo = base + pl.shift > kb ? base + pl.shift : kb;
      mv_hi = cache_end;
      mv_stash = split > 0 ? kb + pl.shift : kb;
      const int64_t slice_off = (int64_t)(b * a.Hkv + kvh) * a.C * kRowB;
      mv_k = (uint64_t)((char*)a.present_k + slice_off - (base + pl.shift) * kRowB);
      mv_v = (uint64_t)((char*)a.present_v + slice_off - (base + pl.shift) * kRowB);
      const int64_t slot = ((int64_t)(b * a.Hkv + kvh) * a.nsplit + split) * 2 * a.stash_rows;
      st_k = (uint64_t)((char*)a.stash + (slot - kb) * kRowB);
      st_v = (uint64_t)((char*)a.stash + (slot + a.stash_rows - kb) * kRowB);
    }
  }

  // The attention_bias entries this lane scores in the block at j0, as raw
  // words.
  auto load_bias = [&](int64_t j0, uint32_t* w) __attribute__((always_inline)) {
    if constexpr (BIAS) {
      // the keys of this lane's scores (16-bit: j0 + 8 lg + [0, 8), one
      // 8-element load; fp32: j0 + 16 kt + 4 lg + [0, 4), one 4-element
      // load per tile) at element (not vector) alignment -- global memory
      // takes unaligned vector loads on this target.  The start is clamped
      // to total - (elements loaded) so the load stays inside the row (a
      // valid item has total >= T >= S, and the host sends steps here only
      // when total >= 8); entries of keys past the band's end are masked,
      // and a group moved back by the clamp is shifted into place when the
      // block is computed.  One path for every block, so no load waits on
      // another.
      if constexpr (DT == kF32) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int64_t g0 = min(j0 + kt * 16, (int64_t)a.total - 4 - 4 * lg);
          load4_raw_unaligned<DT>(bias_lane + (uint64_t)(g0 * e), w + kt * BW / 2);
        }
      } else {
        const int64_t g0 = min(j0, (int64_t)a.total - 8 - 8 * lg);
        load8_raw_unaligned<DT>(bias_lane + (uint64_t)(g0 * e), w);
      }
    }
  };
  auto load_block = [&](int64_t j0, BlockRegs& rg) __attribute__((always_inline)) {
    if (j0 + BN <= cache_end) {  // uniform
      const uint64_t boff = (uint64_t)(j0 * kRowB);
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        if constexpr (Q8) {
          rg.k[u] = load_codes<DT>(kc_lane[u] + boff);
          rg.v[u] = load_codes<DT>(vc_lane[u] + boff);
        } else {
          rg.k[u] = load16_global<false>(kc_lane[u] + boff);
          rg.v[u] = load16_global<false>(vc_lane[u] + boff);
        }
      }
    } else if (j0 >= pl.P && j0 + BN <= ke) {  // uniform: only new rows (prefill)
      const uint64_t boff = (uint64_t)((j0 - pl.P) * new_stride);
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        if constexpr (Q8) {
          rg.k[u] = load_codes<DT>(nk + boff + nw_lane[u]);
          rg.v[u] = load_codes<DT>(nv + boff + nw_lane[u]);
        } else {
          rg.k[u] = load16_global<false>(nk + boff + nw_lane[u]);
          rg.v[u] = load16_global<false>(nv + boff + nw_lane[u]);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int c = min(tid + u * kThreads, Sh::CHUNKS - 1);
        const int key = chunk_key<CPR>(c), part = chunk_part<CPR>(c);
        const int64_t j = min(j0 + key, ke - 1);
        const bool in_cache = j < pl.P;
        const uint64_t msk = 0ull - (uint64_t)in_cache;
        const uint64_t off_c = (uint64_t)((j - base) * kRowB + part * kPartB);
        const uint64_t off_n = (uint64_t)((j - pl.P) * new_stride + part * kPartB);
        const uint64_t ka = ((ck + off_c) & msk) | ((nk + off_n) & ~msk);
        const uint64_t va = ((cv + off_c) & msk) | ((nv + off_n) & ~msk);
        if constexpr (Q8) {
          rg.k[u] = load_codes<DT>(ka);
          rg.v[u] = load_codes<DT>(va);
        } else {
          rg.k[u] = load16_global<false>(ka);
          rg.v[u] = load16_global<false>(va);
        }
      }
    }
    if constexpr (BIAS && GRP == 1) load_bias(j0, rg.bias);
  };
  auto store_block = [&](const BlockRegs& rg, int buf) __attribute__((always_inline)) {
    LT* const bK = sK + buf * Sh::KELEMS;
    LT* const bV = sV + buf * Sh::VELEMS;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + u * kThreads;
      if constexpr (Sh::CHUNKS % kThreads != 0)
        if (c >= Sh::CHUNKS) continue;
      const int key = chunk_key<CPR>(c), part = chunk_part<CPR>(c);
      const int d0 = part * (16 / e);
      const u32x4 kw = Q8 ? codes_to_elems<DT, CT>(rg.k[u]) : rg.k[u];
      const u32x4 vw = Q8 ? codes_to_elems<DT, CT>(rg.v[u]) : rg.v[u];
      if constexpr (DT == kF32) {
        // rows of 16-byte multiples: one store per chunk
        *(u32x4*)((float*)bK + k_slot<DT>(key) * KS + d0) = kw;
        *(u32x4*)((float*)bV + key * VS + d0) = vw;
      } else {
        // K rows are 16-byte aligned: one store per chunk
        *(u32x4*)((uint16_t*)bK + k_slot<DT>(key) * KS + d0) = kw;
        // V transposed, sV[d][key ^ swz(d)].  The wave's 4 lane groups hold
        // keys 4q .. 4q + 3 at the same columns d0 .. d0 + 7, word w = columns
        // d0 + 2w, + 1: a 4x4 exchange of the words across lane groups (two
        // swaps of lane halves, two of lane rows; every lane of the wave
        // takes part) leaves group g with word g of all 4 keys, i.e. columns
        // d0 + 2g and d0 + 2g + 1 of keys 4q .. 4q + 3: two 8-byte rows.
        const int g = (tid >> 4) & 3;
        uint32_t w0 = vw[0], w1 = vw[1], w2 = vw[2], w3 = vw[3];
        {
          const auto r = __builtin_amdgcn_permlane32_swap(w0, w2, false, false);
          w0 = r[0];
          w2 = r[1];
        }
        {
          const auto r = __builtin_amdgcn_permlane32_swap(w1, w3, false, false);
          w1 = r[0];
          w3 = r[1];
        }
        {
          const auto r = __builtin_amdgcn_permlane16_swap(w0, w1, false, false);
          w0 = r[0];
          w1 = r[1];
        }
        {
          const auto r = __builtin_amdgcn_permlane16_swap(w2, w3, false, false);
          w2 = r[0];
          w3 = r[1];
        }
        // word i now holds key 4q + i; columns d0 + 2g (low halves) and
        // d0 + 2g + 1 (high halves)
        const int col = (key - g) ^ vt_swizzle(d0);
        uint16_t* const vr = (uint16_t*)bV + (d0 + 2 * g) * VS + col;
        *(uint2*)vr = make_uint2(__builtin_amdgcn_perm(w1, w0, 0x05040100u),
                                 __builtin_amdgcn_perm(w3, w2, 0x05040100u));
        *(uint2*)(vr + VS) = make_uint2(__builtin_amdgcn_perm(w1, w0, 0x07060302u),
                                        __builtin_amdgcn_perm(w3, w2, 0x07060302u));
      }
    }
  };

  // The block's surviving rows to their new place (or the stash).
  auto move_block = [&](int blk, const BlockRegs& rg) __attribute__((always_inline)) {
    const int64_t j0 = kb + (int64_t)blk * BN;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + u * kThreads;
      if constexpr (Sh::CHUNKS % kThreads != 0)
        if (c >= Sh::CHUNKS) continue;
      const int64_t pos = j0 + chunk_key<CPR>(c);
      if (pos < mv_lo || pos >= mv_hi) continue;
      const bool st = pos < mv_stash;
      const uint64_t off = (uint64_t)(pos * kRowB + chunk_part<CPR>(c) * kPartB);
      store16_global<SWGQA_FM_NT>((st ? st_k : mv_k) + off, rg.k[u]);
      store16_global<SWGQA_FM_NT>((st ? st_v : mv_v) + off, rg.v[u]);
    }
  };

  // visibility of key kb + jr for this lane's query, as 32-bit bounds on jr
  const int64_t vlo = my_pos - a.W + 1 - kb;
  const int64_t vhi = (my_pos < ke - 1 ? my_pos : ke - 1) - kb;
  const int32_t vis_lo = my_ok ? (int32_t)(vlo < -(int64_t)0x7fffffff ? -0x7fffffff : vlo) : 1;
  const int32_t vis_hi = my_ok ? (int32_t)vhi : 0;
  // the keys every query of this wave sees: [w_vis_lo, w_vis_hi] -- both
  // bounds grow with the position, so they are those of the wave's last and
  // first query rows (scalars; lanes without a query do not narrow it)
  int32_t w_vis_lo = INT32_MIN;
  int32_t w_vis_hi = INT32_MAX;
  {
    const int qw0 = q0 + 16 * __builtin_amdgcn_readfirstlane(wq);
    if (qw0 < nq_item) {
      const int qw1 = min(qw0 + 15, nq_item - 1);
      // largest position: the highest lower bound; smallest: the lowest upper bound
      const int64_t p_lo = pl.P + div_gap((uint32_t)qw1, a.qdiv);
      const int64_t p_hi = pl.P + div_gap((uint32_t)qw0, a.qdiv);
      const int64_t wlo = p_lo - a.W + 1 - kb;
      w_vis_lo = (int32_t)(wlo < -(int64_t)0x7fffffff ? -0x7fffffff : wlo);
      w_vis_hi = (int32_t)((p_hi < ke - 1 ? p_hi : ke - 1) - kb);
    }
  }

  float m_run = -INFINITY;  // log2 units, per query (same in all 4 lane groups)
  float l_run = 0.0f;       // this lane's share of the sum
  f4 o[DT16];               // O^T tiles: d = 16 dt + 4 lg + r, query lq
#pragma unroll
  for (int t = 0; t < DT16; ++t) o[t] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  const int nblocks = ke > kb ? (int)((ke - kb + BN - 1) / BN) : 0;
  const int32_t nk_band = ke > kb ? (int32_t)(ke - kb) : 0;  // keys of this split
  const float qk_scale = Q8 ? a.scale * a.k_scale : a.scale;
  // One block: scores, online softmax, PV, from the block staged in LDS.
  auto compute_block = [&](int blk, int buf, const float* bias_blk) __attribute__((always_inline)) {
    const LT* const bK = sK + buf * Sh::KELEMS;
    const LT* const bV = sV + buf * Sh::VELEMS;
    // the block's second score tile (fp32: keys 16 .. 31; 16-bit: keys
    // 8g + 4 .. 8g + 7) holds keys of the band (else its scores are masked
    // and its products are skipped: P = 0 there)
    const bool tile1 = blk * BN + (DT == kF32 ? 16 : 4) < nk_band;
    // S^T for the two 16-key tiles of the block
    f4 sc[2];
    if constexpr (DT == kF32) {
      // lane: key row 16 kt + lq, elements [DSTEPS lg, DSTEPS lg + DSTEPS),
      // four at a time
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if (kt == 0 || tile1) {
          const float* kr = (const float*)bK + (16 * kt + lq) * KS + DSTEPS * lg;
#pragma unroll
          for (int s = 0; s < DSTEPS; s += 4) {
            const f4 k4 = *(const f4*)(kr + s);
#pragma unroll
            for (int t = 0; t < 4; ++t)
              acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k4[t], qf[s + t], acc, 0, 0, 0);
          }
        }
        sc[kt] = acc;
      }
    } else if constexpr (QX32) {
      // lane: key row 16 kt + lq, elements 32 s + 8 lg .. +7; two
      // accumulators per tile (even and odd steps) shorten the dependent
      // chains of products
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if (kt == 0 || tile1) {
          const uint16_t* kr = (const uint16_t*)bK + (16 * kt + lq) * KS + 8 * lg;
          f4 acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s = 0; s < QST; ++s) {
            const uint4 kv = *(const uint4*)(kr + 32 * s);
            const uint4 qv = make_uint4(qh[s][0], qh[s][1], qh[s][2], qh[s][3]);
            if (s % 2 == 0) acc = mfma_x32<DT>(kv, qv, acc);
            else acc1 = mfma_x32<DT>(kv, qv, acc1);
          }
          if constexpr (QST > 1) acc += acc1;
        }
        sc[kt] = acc;
      }
    } else {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      if (kt == 0 || tile1) {
        const uint16_t* kr = (const uint16_t*)bK + (16 * kt + lq) * KS + 4 * lg;
#pragma unroll
        for (int s = 0; s < DSTEPS; ++s) {
          const uint2 kv = *(const uint2*)(kr + 16 * s);
          if constexpr (DT == kF16) {
            acc = __builtin_amdgcn_mfma_f32_16x16x16f16(
                __builtin_bit_cast(h4, make_uint2(kv.x, kv.y)),
                __builtin_bit_cast(h4, make_uint2(qh[s][0], qh[s][1])), acc, 0, 0, 0);
          } else {
            acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                __builtin_bit_cast(s4, make_uint2(kv.x, kv.y)),
                __builtin_bit_cast(s4, make_uint2(qh[s][0], qh[s][1])), acc, 0, 0, 0);
          }
        }
      }
      sc[kt] = acc;
    }
    }

    // Scores: key j = j0 + 16 kt + 4 lg + r, query lq.  Blocks every query
    // of the wave sees whole, without softcap or bias, take the plain
    // transform (the same roundings); the others one of two loops chosen
    // once per block, with and without softcap.
    float smax = -INFINITY;
    auto transform = [&](auto capc) __attribute__((always_inline)) {
      constexpr bool CAP = decltype(capc)::value;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int32_t jr = blk * BN + score_key<DT>(kt, lg, r);
          const bool vis = jr >= vis_lo && jr <= vis_hi;
          float x = sc[kt][r] * qk_scale;
          if constexpr (CAP) {
            const float y = x * inv_cap;
            if constexpr (DT == kF32) {
              x = cap * tanhf(y);
            } else {
              const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(
                                         __builtin_amdgcn_exp2f(2.0f * kLog2e * fabsf(y)) + 1.0f);
              x = cap * copysignf(t, y);
            }
          }
          if (has_bias) x += bias_blk[kt * 4 + r];
          x = vis ? x * kLog2e : -INFINITY;
          sc[kt][r] = x;
          smax = fmaxf(smax, x);
        }
    };
    if (!has_cap && !has_bias && blk * BN >= w_vis_lo && blk * BN + BN - 1 <= w_vis_hi) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = (sc[kt][r] * qk_scale) * kLog2e;
          sc[kt][r] = x;
          smax = fmaxf(smax, x);
        }
    } else if (has_cap) {
      transform(std::true_type{});
    } else {
      transform(std::false_type{});
    }
    auto fmax_op = [](float x, float y) { return fmaxf(x, y); };
    smax = reduce_xor16(smax, fmax_op);
    smax = reduce_xor32(smax, fmax_op);
    const float m_new = fmaxf(m_run, smax);
    const float corr = (m_run == m_new) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.0f;
    uint32_t p16[2][2] = {{0u, 0u}, {0u, 0u}};  // fp16: P as the PV operand, packed
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p = (sc[kt][r] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sc[kt][r] - m_new);
        if constexpr (DT == kF16) {
          // the normaliser sums P as rounded for the product
          const uint32_t h = f32_to_f16_bits(p);
          p16[kt][r / 2] |= h << (16 * (r % 2));
          p = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
        }
        sc[kt][r] = p;
        psum += p;
      }
    l_run = l_run * corr + psum;
    // rescale only when some query's maximum moved: after the first blocks
    // the maxima settle and this is skipped
    if (__any(corr != 1.0f)) {
#pragma unroll
      for (int t = 0; t < DT16; ++t) o[t] *= corr;
    }

    // O^T += V^T . P^T
    if constexpr (DT == kF32) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if (kt == 1 && !tile1) break;
        // fp32: O^T tile dt holds rows d = DT16 i + dt, so a lane's V
        // operands for all tiles are DT16 consecutive elements of one key
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          const float* vr = (const float*)bV + (kt * 16 + 4 * lg + t4) * VS + DT16 * lq;
          float va[DT16];
          if constexpr (DT16 % 4 == 0) {
#pragma unroll
            for (int c = 0; c < DT16; c += 4) {
              const f4 w = *(const f4*)(vr + c);
              va[c] = w[0]; va[c + 1] = w[1]; va[c + 2] = w[2]; va[c + 3] = w[3];
            }
          } else if constexpr (DT16 == 2) {
            const float2 w = *(const float2*)vr;
            va[0] = w.x; va[1] = w.y;
          } else {
            va[0] = vr[0];
          }
#pragma unroll
          for (int dt = 0; dt < DT16; ++dt)
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va[dt], sc[kt][t4], o[dt], 0, 0, 0);
        }
      }
    } else {
      // One 16x16x32 product per O^T tile over the block's 32 keys: lane
      // group lg's reduction elements are keys 8lg .. 8lg + 7, the keys its
      // scores hold.  P is 0 on masked keys, and on the whole second score
      // tile when it lies past the band (whose V rows are clamped copies of
      // the band's last row: finite).
      uint32_t pw[4], pl2[4];
      if constexpr (DT == kF16) {
        pw[0] = p16[0][0];
        pw[1] = p16[0][1];
        pw[2] = p16[1][0];
        pw[3] = p16[1][1];
      } else {
        // bf16 keeps 8 significant bits, too few for P: P = hi + lo, both
        // bf16, and two products (relative error ~2^-17)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          uint16_t hi[4], lo[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            hi[r] = f32_to_bf16(sc[kt][r]);
            lo[r] = f32_to_bf16(sc[kt][r] - __uint_as_float((uint32_t)hi[r] << 16));
          }
          pw[2 * kt] = (uint32_t)hi[0] | ((uint32_t)hi[1] << 16);
          pw[2 * kt + 1] = (uint32_t)hi[2] | ((uint32_t)hi[3] << 16);
          pl2[2 * kt] = (uint32_t)lo[0] | ((uint32_t)lo[1] << 16);
          pl2[2 * kt + 1] = (uint32_t)lo[2] | ((uint32_t)lo[3] << 16);
        }
      }
      const uint4 pv = make_uint4(pw[0], pw[1], pw[2], pw[3]);
#pragma unroll
      for (int dt = 0; dt < DT16; ++dt) {
        const uint16_t* vrow = (const uint16_t*)bV + (16 * dt + lq) * VS;
        const int sw = vt_swizzle(16 * dt + lq);
        const uint4 vv = *(const uint4*)(vrow + ((8 * lg) ^ sw));
        o[dt] = mfma_x32<DT>(vv, pv, o[dt]);
        if constexpr (DT == kBF16)
          o[dt] = mfma_x32<DT>(vv, make_uint4(pl2[0], pl2[1], pl2[2], pl2[3]), o[dt]);
      }
    }
  };
  // The attention_bias entries of block blk as floats, from its raw words.
  auto block_bias = [&](int blk, const uint32_t* braw, float* bias_blk) __attribute__((always_inline)) {
    if constexpr (BIAS) {
      const int64_t j0 = kb + (int64_t)blk * BN;
      float x[8];  // entry 4 kt + r: the bias of score r of tile kt
      if constexpr (DT == kF32) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          // elements the clamp moved the group back by (0 unless the group
          // passes the end of the row)
          const int64_t g = j0 + kt * 16 + 4 * lg;
          const int sh = (int)min(g - min(g, (int64_t)a.total - 4), (int64_t)3);
          const uint32_t* w = braw + kt * BW / 2;
          // (selects, not an index: a register array indexed at run time
          // would live in scratch memory)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = min(r + sh, 3);
            x[4 * kt + r] =
                __uint_as_float(i == 0 ? w[0] : i == 1 ? w[1] : i == 2 ? w[2] : w[3]);
          }
        }
      } else {
        // elements the clamp moved the group back by (0 unless the group
        // passes the end of the row; entries r >= 8 - sh are then past it,
        // and masked)
        const int64_t g = j0 + 8 * lg;
        const int sh = (int)min(g - min(g, (int64_t)a.total - 8), (int64_t)7);
        const uint32_t* w = braw;
        // the 8 entries as one 128-bit value, shifted right by sh entries
        const uint64_t lo = ((uint64_t)w[1] << 32) | w[0];
        const uint64_t hi = ((uint64_t)w[3] << 32) | w[2];
        const int bits = 16 * sh;
        const uint64_t nlo =
            bits == 0 ? lo : bits < 64 ? (lo >> bits) | (hi << (64 - bits)) : hi >> (bits - 64);
        const uint64_t nhi = bits < 64 ? hi >> bits : 0;
        unpack_word<DT>((uint32_t)nlo, x);
        unpack_word<DT>((uint32_t)(nlo >> 32), x + 2);
        unpack_word<DT>((uint32_t)nhi, x + 4);
        unpack_word<DT>((uint32_t)(nhi >> 32), x + 6);
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) bias_blk[r] = x[r];
    }
  };
  // A block's K/V/bias loads are issued three steps before it is staged
  // (register ring of three), so two blocks of loads stay in flight while
  // one is computed; no loads are issued for blocks past the split's end
  // (they only took load-unit cycles from the blocks still wanted).  Step
  // blk computes block blk from LDS buffer blk & 1, then stages block blk + 1
  // (in the ring since step blk - 3) into the other buffer -- whose block,
  // blk - 1, every wave finished before the barrier that ended step blk - 1
  // -- reloads those registers with block blk + 4, and ends with a barrier,
  // after which block blk + 1 is visible and buffer blk & 1 free: one
  // barrier per block.
  auto block_start = [&](int blk) { return kb + (int64_t)min(blk, nblocks - 1) * BN; };
  float bias_cur[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  constexpr int RING = chunk_ring<DT, D, NW, BIAS>();
  auto step = [&](int blk, BlockRegs& rg) __attribute__((always_inline)) {
    compute_block(blk, blk & 1, bias_cur);
    store_block(rg, (blk + 1) & 1);
    block_bias(blk + 1, rg.bias, bias_cur);  // compute_block(blk) is done with it
    if (blk + 1 + RING < nblocks) load_block(block_start(blk + 1 + RING), rg);
    __syncthreads();
  };
  // single buffer: barrier, stage block blk, barrier, reload its registers
  // with block blk + RING, compute block blk
  auto step1 = [&](int blk, BlockRegs& rg) __attribute__((always_inline)) {
    __syncthreads();  // the previous block's LDS reads are done
    store_block(rg, 0);
    block_bias(blk, rg.bias, bias_cur);
    __syncthreads();
    if constexpr (kCanMove)
      if (fmove) move_block(blk, rg);
    if (blk + RING < nblocks) load_block(block_start(blk + RING), rg);
    compute_block(blk, 0, bias_cur);
  };
  if constexpr (GRP > 1) {
    // Staging round r: blocks r GRP + g into buffers g (those inside the
    // split), bias of block r GRP + grp, a barrier, the surviving rows of
    // the staged blocks moved, their registers reloaded with the blocks of
    // round r + RG, then each group computes its block.  A barrier opens the
    // next round once every group is done with the buffers.
    constexpr int RG = 2;  // rounds of loads in flight
    const int nrounds = (nblocks + GRP - 1) / GRP;
    if (nblocks > 0) {
      BlockRegs rg[RG][GRP];
      uint32_t brg[RG][BW];
#pragma unroll
      for (int i = 0; i < RG; ++i) {
#pragma unroll
        for (int g = 0; g < GRP; ++g)
          if (i * GRP + g < nblocks) load_block(block_start(i * GRP + g), rg[i][g]);
        if (i * GRP + grp < nblocks) load_bias(block_start(i * GRP + grp), brg[i]);
      }
      for (int r = 0; r < nrounds;) {
#pragma unroll
        for (int i = 0; i < RG; ++i) {
          if (r >= nrounds) break;
          const int b0 = r * GRP;
          __syncthreads();  // the previous round's LDS reads are done
#pragma unroll
          for (int g = 0; g < GRP; ++g)
            if (b0 + g < nblocks) store_block(rg[i][g], g);
          if (b0 + grp < nblocks) block_bias(b0 + grp, brg[i], bias_cur);
          __syncthreads();
          if constexpr (kCanMove) {
            if (fmove) {
#pragma unroll
              for (int g = 0; g < GRP; ++g)
                if (b0 + g < nblocks) move_block(b0 + g, rg[i][g]);
            }
          }
#pragma unroll
          for (int g = 0; g < GRP; ++g)
            if (b0 + RG * GRP + g < nblocks) load_block(block_start(b0 + RG * GRP + g), rg[i][g]);
          if (b0 + RG * GRP + grp < nblocks) load_bias(block_start(b0 + RG * GRP + grp), brg[i]);
          if (b0 + grp < nblocks) compute_block(b0 + grp, grp, bias_cur);
          ++r;
        }
      }
    }
  } else if constexpr (!DB) {
    if (nblocks > 0) {
      BlockRegs rg[RING];
#pragma unroll
      for (int i = 0; i < RING; ++i)
        if (i < nblocks) load_block(block_start(i), rg[i]);
      for (int blk = 0; blk < nblocks;) {
#pragma unroll
        for (int i = 0; i < RING; ++i) {
          if (blk >= nblocks) break;
          step1(blk, rg[i]);
          ++blk;
        }
      }
    }
  } else if (nblocks > 0) {
    BlockRegs rg[RING];
#pragma unroll
    for (int i = 0; i < RING; ++i)
      if (i < nblocks) load_block(block_start(i), rg[i]);
    store_block(rg[0], 0);
    block_bias(0, rg[0].bias, bias_cur);
    if (RING < nblocks) load_block(block_start(RING), rg[0]);
    __syncthreads();
    for (int blk = 0; blk < nblocks;) {
#pragma unroll
      for (int i = 0; i < RING; ++i) {
        if (blk >= nblocks) break;
        step(blk, rg[(i + 1) % RING]);
        ++blk;
      }
    }
  }

  if constexpr (GRP > 1) {
    // Groups 1 .. GRP - 1 hand their softmax states (per lane: O^T column
    // parts, running maximum, partial sum) to group 0 through LDS; group 0
    // merges them with its own, as the split merge does.
    // (16-byte slots per lane: the DT16 O^T words, then max and sum; slot k
    // of every lane of a wave is one contiguous 1 KiB row)
    constexpr int NS = DT16 + 1;
    __shared__ f4 sG[GRP > 1 ? (GRP - 1) * NWQ * NS * kWave : 1];
    auto at = [&](int g1, int k) { return ((g1 * NWQ + wq) * NS + k) * kWave + lane; };
    if (grp > 0) {
#pragma unroll
      for (int dt = 0; dt < DT16; ++dt) sG[at(grp - 1, dt)] = o[dt];
      sG[at(grp - 1, DT16)] = f4{m_run, l_run, 0.0f, 0.0f};
    }
    __syncthreads();
    if (grp == 0) {
      f4 ml[GRP - 1 > 0 ? GRP - 1 : 1];
      float M = m_run;
#pragma unroll
      for (int g1 = 0; g1 < GRP - 1; ++g1) {
        ml[g1] = sG[at(g1, DT16)];
        M = fmaxf(M, ml[g1][0]);
      }
      const float c0 = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - M);
      l_run *= c0;
#pragma unroll
      for (int dt = 0; dt < DT16; ++dt) o[dt] *= c0;
#pragma unroll
      for (int g1 = 0; g1 < GRP - 1; ++g1) {
        const float c = ml[g1][0] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml[g1][0] - M);
        l_run += ml[g1][1] * c;
#pragma unroll
        for (int dt = 0; dt < DT16; ++dt) o[dt] += sG[at(g1, dt)] * c;
      }
      m_run = M;
    }
  }

  // Sum of P over the four lane groups; write O (or the split partial).
  l_run = reduce_xor16(l_run, add_f);
  l_run = reduce_xor32(l_run, add_f);
  if (my_ok && (GRP == 1 || grp == 0)) {
    const int64_t row = ((int64_t)b * a.S + my_i) * a.Hq + my_h;
    if (a.nsplit == 1) {
      float m_fin = m_run;
      const float inv = fold_sink<DT>(a.sink, a.smooth, my_h, m_fin, l_run) / l_run *
                        (Q8 ? a.v_scale : 1.0f);
      if constexpr (DT == kF32) {
        // element DT16 (4 lg + r) + dt of the row is o[dt][r]
        float* orow = (float*)a.out + row * D + DT16 * 4 * lg;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (DT16 % 4 == 0) {
#pragma unroll
            for (int c = 0; c < DT16; c += 4)
              *(f4*)(orow + DT16 * r + c) =
                  f4{o[c][r] * inv, o[c + 1][r] * inv, o[c + 2][r] * inv, o[c + 3][r] * inv};
          } else {
#pragma unroll
            for (int dt = 0; dt < DT16; ++dt) orow[DT16 * r + dt] = o[dt][r] * inv;
          }
        }
      } else {
#pragma unroll
      for (int dt = 0; dt < DT16; ++dt) {
        const int d0 = 16 * dt + 4 * lg;
        {
          uint32_t w0, w1;
          if constexpr (DT == kF16) {
            w0 = (uint32_t)f32_to_f16_bits(o[dt][0] * inv) | ((uint32_t)f32_to_f16_bits(o[dt][1] * inv) << 16);
            w1 = (uint32_t)f32_to_f16_bits(o[dt][2] * inv) | ((uint32_t)f32_to_f16_bits(o[dt][3] * inv) << 16);
          } else {
            w0 = (uint32_t)f32_to_bf16(o[dt][0] * inv) | ((uint32_t)f32_to_bf16(o[dt][1] * inv) << 16);
            w1 = (uint32_t)f32_to_bf16(o[dt][2] * inv) | ((uint32_t)f32_to_bf16(o[dt][3] * inv) << 16);
          }
          *(uint2*)((uint16_t*)a.out + row * D + d0) = make_uint2(w0, w1);
        }
      }
      }
    } else {
      float* op = a.opart + (row * a.nsplit + split) * D;
      const float vs = Q8 ? a.v_scale : 1.0f;
      if constexpr (DT == kF32) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int dt = 0; dt < DT16; ++dt) op[DT16 * (4 * lg + r) + dt] = o[dt][r] * vs;
      } else {
#pragma unroll
        for (int dt = 0; dt < DT16; ++dt) *(f4*)(op + 16 * dt + 4 * lg) = o[dt] * vs;
      }
      if (lg == 0) {
        a.ml[(row * a.nsplit + split) * 2 + 0] = m_run;
        a.ml[(row * a.nsplit + split) * 2 + 1] = l_run;
      }
    }
  }
  // Appends on drifting steps with a shared buffer: rows [Lb, Lb + S) lie
  // beyond every cache row attention reads, so they are written last.
  if (a.present_k && pl.shift == 0 && tile == 0 && split == 0) {
    char* pk = (char*)a.present_k + ((int64_t)(b * a.Hkv + kvh) * a.C) * D * CE;
    char* pv = (char*)a.present_v + ((int64_t)(b * a.Hkv + kvh) * a.C) * D * CE;
    for (int idx = tid; idx < a.S * CPRC; idx += kThreads) {
      const int i = idx / CPRC, w = idx % CPRC;
      const int64_t src = ((int64_t)(b * a.S + i) * a.Hkv + kvh) * D * CE + w * 16;
      const int64_t dst = (pl.Lb + i) * (int64_t)D * CE + w * 16;
      *(u32x4*)(pk + dst) = *(const u32x4*)((const char*)a.k + src);
      *(u32x4*)(pv + dst) = *(const u32x4*)((const char*)a.v + src);
    }
  }

  slice_tail_rows<8>(a, pl, b, kvh, D, CE, nullptr, nullptr);
}

// Wave groups: 16-bit element-type caches with rows of at most 256 bytes.
template <int DT, int D, int CT>
constexpr bool chunk_groups_ok() { return DT != kF32 && CT == 0 && D * 2 <= 256 && !chunk_double_buffer<DT>(); }

template <int DT, int D, int NW, int CT>
hipError_t launch_w(const AttnArgs& a, hipStream_t st) {
  const dim3 grid(a.ntiles * a.nsplit, a.Hkv, a.B);
  if constexpr (NW == 8 && chunk_groups_ok<DT, D, CT>()) {
    if (a.chunk_groups == 4) {
      if (a.bias)
        attn_chunk_kernel<DT, D, true, 8, CT, 4><<<grid, 8 * kWave, 0, st>>>(a);
      else
        attn_chunk_kernel<DT, D, false, 8, CT, 4><<<grid, 8 * kWave, 0, st>>>(a);
      return hipGetLastError();
    }
  }
  if (a.chunk_groups > 1) return hipErrorInvalidValue;
  if (a.bias)
    attn_chunk_kernel<DT, D, true, NW, CT><<<grid, NW * kWave, 0, st>>>(a);
  else
    attn_chunk_kernel<DT, D, false, NW, CT><<<grid, NW * kWave, 0, st>>>(a);
  return hipGetLastError();
}

template <int DT, int D, int CT>
hipError_t launch_d(const AttnArgs& a, hipStream_t st) {
  if constexpr (ChunkShape<DT, D, 4>::ok) {
    return a.waves == 8 ? launch_w<DT, D, 8, CT>(a, st) : launch_w<DT, D, 4, CT>(a, st);
  } else {
    return hipErrorInvalidValue;
  }
}

template <int DT, int CT>
hipError_t launch_t(int D, const AttnArgs& a, hipStream_t st) {
  switch (D) {
    case 16: return launch_d<DT, 16, CT>(a, st);
    case 32: return launch_d<DT, 32, CT>(a, st);
    case 64: return launch_d<DT, 64, CT>(a, st);
    case 128: return launch_d<DT, 128, CT>(a, st);
    case 256: return launch_d<DT, 256, CT>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

}  // namespace swgqa
