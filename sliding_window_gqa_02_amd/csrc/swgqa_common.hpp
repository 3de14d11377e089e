// swgqa_common.hpp -- device-side pieces shared by the libswgqa kernels:
// the resident-range planner, element loads/stores and small wave helpers.
//
// Target: AMD CDNA4 (gfx950), wave64.  Nothing here is shared with the CPU
// oracle under oracle/.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swgqa {

// Element type tags (match swgqa_dtype).
enum : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Status word bits, stored at workspace offset 0.
enum : uint32_t { kStatusBadItem = 1u };

constexpr int kWave = 64;

// Native 16-byte vector (HIP's uint4 is a struct, and arrays of it are not
// promoted to registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Resident-range planner.  "Specify GroupQueryAttention windowed KV cache
// layout contract" (onnxruntime PR #32419), Description: G = C - W + 1,
// L(T) = T for T <= C, else T - G * ceil((T - C) / G).  "[CPU] Add windowed
// kv cache for GQA" (PR #31142), review thread: per-item plan computed in
// int64 from seqlens_k.
struct ItemPlan {
  int64_t T;      // total length after the step
  int64_t P;      // past length (absolute position of the first new token)
  int64_t Lb;     // resident rows before the step
  int64_t La;     // resident rows after the step
  int64_t kept;   // La - S: old rows that survive (may be negative)
  int64_t shift;  // Lb + S - La: rows evicted by this step
  bool ok;        // seqlens_k[b] consistent with S and total length
};

__host__ __device__ __forceinline__ int64_t resident_len(int64_t T, int64_t C,
                                                         int64_t W) {
  if (T <= C) return T;
  const int64_t G = C - W + 1;
  return T - G * ((T - C + G - 1) / G);
}

// Division by the gap G = C - W + 1, an invariant of the call, as a multiply
// and two shifts (Granlund and Montgomery, "Division by Invariant Integers
// using Multiplication", PLDI 1994, the round-up method for unsigned N-bit
// division, N = 32): with l = ceil(log2 G), m = floor(2^32 (2^l - G) / G) + 1,
// t = mulhi(m, n), the quotient floor(n / G) = (t + ((n - t) >> min(l, 1)))
// >> max(l - 1, 0) for every 0 <= n < 2^32.  The magic is made on the host.
struct GapDiv {
  uint32_t G;
  uint32_t magic;
  uint32_t sh1, sh2;
};

inline GapDiv make_gap_div(uint32_t G) {  // 1 <= G < 2^31
  uint32_t l = 0;
  while ((1ull << l) < G) ++l;
  GapDiv d;
  d.G = G;
  d.magic = (uint32_t)((((1ull << l) - G) << 32) / G + 1);
  d.sh1 = l < 1 ? l : 1;
  d.sh2 = l > 1 ? l - 1 : 0;
  return d;
}

__host__ __device__ __forceinline__ uint32_t div_gap(uint32_t n, const GapDiv& d) {
#ifdef __HIP_DEVICE_COMPILE__
  const uint32_t t = __umulhi(d.magic, n);
#else
  const uint32_t t = (uint32_t)(((uint64_t)d.magic * n) >> 32);
#endif
  return (t + ((n - t) >> d.sh1)) >> d.sh2;
}

// XCD-aware placement.  The workgroups of a launch are dealt to the chip's 8
// XCDs, each with its own L2, round-robin by linear id.  This maps linear id
// L (of N) to a work index P such that every XCD receives one contiguous
// range of P: consecutive work items -- the query tiles and key splits of one
// (item, KV head) slice, which read the same K/V rows -- then share an L2.
// XCD x holds ids x, x + 8, ...: q + (x < r) of them for N = 8q + r, and
// receives P in [x q + min(x, r), (x + 1) q + min(x + 1, r)).
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t L, uint32_t N) {
  constexpr uint32_t kXcds = 8;
  const uint32_t x = L % kXcds, k = L / kXcds;
  const uint32_t q = N / kXcds, r = N % kXcds;
  return x * q + (x < r ? x : r) + k;
}

// L(T) for the lengths a step can see: 0 <= T <= 2^31 and 1 <= W <= C < 2^31,
// so ceil((T - C) / G) = (T - C - 1) / G + 1 with a 32-bit numerator.
__host__ __device__ __forceinline__ int64_t resident_len_step(int64_t T, int32_t C,
                                                              const GapDiv& gd) {
  if (T <= C) return T;
  const uint32_t q = div_gap((uint32_t)(T - C - 1), gd) + 1u;
  return T - (int64_t)gd.G * q;
}

__host__ __device__ __forceinline__ ItemPlan plan_item(int32_t seqlen_k, int64_t S,
                                                       int32_t C, const GapDiv& gd,
                                                       int64_t total) {
  ItemPlan pl;
  pl.T = (int64_t)seqlen_k + 1;
  pl.P = pl.T - S;
  pl.ok = pl.P >= 0 && pl.T <= total;
  if (!pl.ok) {
    pl.T = pl.P = pl.Lb = pl.La = pl.kept = pl.shift = -1;
    return pl;
  }
  pl.Lb = resident_len_step(pl.P, C, gd);
  pl.La = resident_len_step(pl.T, C, gd);
  pl.kept = pl.La - S;
  pl.shift = pl.Lb + S - pl.La;
  return pl;
}

// ---------------------------------------------------------------------------
// Element access.  fp32 = float, fp16 = _Float16, bf16 = upper half of a
// binary32 (kept as uint16_t).  Conversions to the narrow types round to
// nearest-even.
template <int DT> struct Elem;
template <> struct Elem<kF32> { using T = float; static constexpr int bytes = 4; };
template <> struct Elem<kF16> { using T = _Float16; static constexpr int bytes = 2; };
template <> struct Elem<kBF16> { using T = uint16_t; static constexpr int bytes = 2; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // NaN
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Unpacks one 32-bit word holding 1 (fp32) or 2 (fp16/bf16) elements.
template <int DT> __device__ __forceinline__ void unpack_word(uint32_t w, float* out);
template <> __device__ __forceinline__ void unpack_word<kF32>(uint32_t w, float* out) {
  out[0] = __uint_as_float(w);
}
template <> __device__ __forceinline__ void unpack_word<kF16>(uint32_t w, float* out) {
  union { uint32_t u; _Float16 h[2]; } c;
  c.u = w;
  out[0] = (float)c.h[0];
  out[1] = (float)c.h[1];
}
template <> __device__ __forceinline__ void unpack_word<kBF16>(uint32_t w, float* out) {
  out[0] = bf16_lo(w);
  out[1] = bf16_hi(w);
}

template <int DT> __device__ __forceinline__ uint32_t pack_word(const float* in);
template <> __device__ __forceinline__ uint32_t pack_word<kF32>(const float* in) {
  return __float_as_uint(in[0]);
}
template <> __device__ __forceinline__ uint32_t pack_word<kF16>(const float* in) {
  union { uint32_t u; _Float16 h[2]; } c;
  c.h[0] = (_Float16)in[0];
  c.h[1] = (_Float16)in[1];
  return c.u;
}
template <> __device__ __forceinline__ uint32_t pack_word<kBF16>(const float* in) {
  return (uint32_t)f32_to_bf16(in[0]) | ((uint32_t)f32_to_bf16(in[1]) << 16);
}

template <int DT> __device__ __forceinline__ float load_one(const void* base, int64_t idx) {
  if constexpr (DT == kF32) {
    return ((const float*)base)[idx];
  } else if constexpr (DT == kF16) {
    return (float)((const _Float16*)base)[idx];
  } else {
    return __uint_as_float((uint32_t)((const uint16_t*)base)[idx] << 16);
  }
}

// Loads NW consecutive 32-bit words (NW*4 bytes, 4-byte aligned at least;
// 16-byte aligned when NW % 4 == 0) with the widest vector accesses.
template <int NW>
__device__ __forceinline__ void load_words(const void* p, uint32_t* w) {
  if constexpr (NW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const uint4 v = ((const uint4*)p)[i];
      w[4 * i + 0] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  } else if constexpr (NW == 2) {
    const uint2 v = *(const uint2*)p;
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = ((const uint32_t*)p)[i];
  }
}

template <int NW>
__device__ __forceinline__ void store_words(void* p, const uint32_t* w) {
  if constexpr (NW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i)
      ((uint4*)p)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  } else if constexpr (NW == 2) {
    *(uint2*)p = make_uint2(w[0], w[1]);
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) ((uint32_t*)p)[i] = w[i];
  }
}

// 16-byte load from a global-memory address held as an integer.  Casting to
// an address-space-1 pointer makes it a GLOBAL instruction; through a generic
// pointer it would be a FLAT one, which also counts against the LDS wait
// counter, so every wait for an LDS result would wait for it as well.
template <bool NT>
__device__ __forceinline__ u32x4 load16_global(uint64_t addr) {
  typedef const u32x4 __attribute__((address_space(1)))* gptr;
  if constexpr (NT) return __builtin_nontemporal_load((gptr)addr);
  else return *(gptr)addr;
}

// 16-byte store to a global-memory address held as an integer (a GLOBAL
// instruction, for the same reason).
template <bool NT = false>
__device__ __forceinline__ void store16_global(uint64_t addr, const u32x4& v) {
  typedef u32x4 __attribute__((address_space(1)))* gptr;
  if constexpr (NT) __builtin_nontemporal_store(v, (gptr)addr);
  else *(gptr)addr = v;
}

// Decode kernels: the variant that moves a compacting slice's surviving rows
// while reading them (1), and whether those stores are non-temporal (1).
#ifndef SWGQA_FUSED_MOVE
#define SWGQA_FUSED_MOVE 1
#endif
#ifndef SWGQA_FM_NT
#define SWGQA_FM_NT 1
#endif

// Workgroup barrier that a wave reaches only once `tok` -- a value computed
// from its last stage's loaded words -- exists, i.e. once those loads (and,
// returning in order, all earlier ones) have returned; no wait for memory
// beyond that, so the loads of later stages stay in flight.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_after(uint32_t tok) {
  asm volatile("" ::"v"(tok) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One element at a global-memory address held as an integer, as float.
template <int DT>
__device__ __forceinline__ float load_elem_global(uint64_t addr) {
  if constexpr (DT == kF32) {
    return *(const float __attribute__((address_space(1)))*)addr;
  } else if constexpr (DT == kF16) {
    return (float)*(const _Float16 __attribute__((address_space(1)))*)addr;
  } else {
    return __uint_as_float((uint32_t)*(const uint16_t __attribute__((address_space(1)))*)addr << 16);
  }
}

// Four consecutive elements at a global address aligned only to the element
// size, as raw words (4 for fp32, 2 for fp16 / bf16) for callers that convert
// them later (one vector load; AMD global memory accepts unaligned vector
// accesses).
template <int DT>
__device__ __forceinline__ void load4_raw_unaligned(uint64_t addr, uint32_t* out) {
  if constexpr (DT == kF32) {
    typedef u32x4 v_t __attribute__((aligned(4)));
    const v_t w = *(const v_t __attribute__((address_space(1)))*)addr;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = w[i];
  } else {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    typedef u32x2 v_t __attribute__((aligned(2)));
    const v_t w = *(const v_t __attribute__((address_space(1)))*)addr;
    out[0] = w[0];
    out[1] = w[1];
  }
}

// The same for 8 consecutive elements (fp32: two 16-byte loads).
template <int DT>
__device__ __forceinline__ void load8_raw_unaligned(uint64_t addr, uint32_t* out) {
  if constexpr (DT == kF32) {
    load4_raw_unaligned<DT>(addr, out);
    load4_raw_unaligned<DT>(addr + 16, out + 4);
  } else {
    typedef u32x4 v_t __attribute__((aligned(2)));
    const v_t w = *(const v_t __attribute__((address_space(1)))*)addr;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = w[i];
  }
}

// int8 cache codes ("GQA In-Place KV Cache: Investigation Report", section
// 1.1, names k_scale / v_scale; reading: the code of x is the binary32
// quotient x / scale rounded to an integer with ties to even, saturated to
// [-128, 127], NaN going to -128).
__device__ __forceinline__ uint32_t quant_code(float x, float scale) {
  float t = rintf(x / scale);
  t = fminf(fmaxf(t, -128.0f), 127.0f);
  return (uint32_t)((int32_t)t & 0xFF);
}

// Code types of a quantized cache.
constexpr int kCodeInt8 = 1;
constexpr int kCodeFp8 = 2;  // OCP E4M3 ("FN"): bias 7, no infinities, 0x7F NaN, max 448

// The fp8 E4M3 code of t: nearest value with ties to the even code (the
// mantissa rounded to 3 bits on the float's bits), magnitudes of 448 or more
// saturated to 448, NaN to 0x7F, results of zero coded +0.
__device__ __forceinline__ uint32_t e4m3_code(float t) {
  if (t != t) return 0x7Fu;
  const uint32_t sign = (__float_as_uint(t) >> 24) & 0x80u;
  const float a = fabsf(t);
  uint32_t c;
  if (a >= 448.0f) {
    c = 0x7Eu;
  } else if (a < 0.015625f) {  // below 2^-6: subnormal steps of 2^-9 (8 -> 2^-6)
    c = (uint32_t)rintf(a * 512.0f);
  } else {
    const uint32_t u = __float_as_uint(a);
    const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);  // 3 mantissa bits, ties to even
    c = (r >> 20) - (120u << 3);                          // float exponent E -> E - 120
  }
  return c == 0u ? 0u : (c | sign);
}

// The code of x for a quantization scale (binary32 quotient first).
template <int CT>
__device__ __forceinline__ uint32_t quant_code_t(float x, float scale) {
  if constexpr (CT == kCodeFp8) return e4m3_code(x / scale);
  else return quant_code(x, scale);
}

// The four codes of a word as floats (exact): int8 by sign-extending
// conversion, fp8 E4M3 by the hardware's packed conversion (OCP E4M3 on this
// target).
template <int CT>
__device__ __forceinline__ void codes4_t(uint32_t w, float* out) {
  if constexpr (CT == kCodeFp8) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    out[0] = lo[0];
    out[1] = lo[1];
    out[2] = hi[0];
    out[3] = hi[1];
  } else {
    out[0] = (float)(int32_t)(int8_t)(w & 0xFFu);
    out[1] = (float)(int32_t)(int8_t)((w >> 8) & 0xFFu);
    out[2] = (float)(int32_t)(int8_t)((w >> 16) & 0xFFu);
    out[3] = (float)(int32_t)(int8_t)(w >> 24);
  }
}

// The 16 codes of elements [c0, c0 + 16) of a row of the element type (row
// and c0 * e 16-byte aligned).
template <int DT, int CT = kCodeInt8>
__device__ __forceinline__ u32x4 quant_chunk16(const void* row, int64_t c0, float scale) {
  constexpr int e = Elem<DT>::bytes;
  float x[16];
#pragma unroll
  for (int i = 0; i < e; ++i) {  // 16 * e bytes in 16-byte loads
    const u32x4 v = *(const u32x4*)((const char*)row + c0 * e + i * 16);
#pragma unroll
    for (int w = 0; w < 4; ++w) unpack_word<DT>(v[w], x + i * (16 / e) + w * (4 / e));
  }
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    r[w] = quant_code_t<CT>(x[4 * w], scale) | (quant_code_t<CT>(x[4 * w + 1], scale) << 8) |
           (quant_code_t<CT>(x[4 * w + 2], scale) << 16) |
           (quant_code_t<CT>(x[4 * w + 3], scale) << 24);
  return r;
}

// op(x of lane l, x of lane l ^ 16) in every lane: v_permlane16_swap on two
// copies of x exchanges rows 1 and 3 of the first with rows 0 and 2 of the
// second, so each lane then holds its own value in one copy and its
// partner's in the other (a VALU exchange; no LDS round trip).  Needs a
// commutative op and every lane active.
template <typename Op>
__device__ __forceinline__ float reduce_xor16(float x, Op op) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// The same for lane l ^ 32 (v_permlane32_swap exchanges the upper half of
// the first copy with the lower half of the second).
template <typename Op>
__device__ __forceinline__ float reduce_xor32(float x, Op op) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float add_f(float a, float b) { return a + b; }

// seqlens_k[b] (uniform across the workgroup) read through the scalar data
// cache: the array is read-only for the whole launch, and one scalar fetch per
// CU replaces a vector load from every wave.
__device__ __forceinline__ int32_t load_seqlen(const int32_t* seqlens, int b) {
  return ((const int32_t __attribute__((address_space(4)))*)seqlens)[b];
}

// Softmax sink of query head h: folds one more logit (head_sink[h], or 0 for
// smooth_softmax) into a finished online-softmax state (running maximum m
// and sum l, log2 units; the accumulators scale by the returned factor).  The
// sink's value row is zero, so only the denominator grows.
template <int DT>
__device__ __forceinline__ float fold_sink(const void* sink, int smooth, int h, float& m,
                                           float& l) {
  if (sink == nullptr && smooth == 0) return 1.0f;
  const float s2 = (sink ? load_one<DT>(sink, h) : 0.0f) * 1.4426950408889634f;
  const float m2 = fmaxf(m, s2);
  const float c = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - m2);
  l = l * c + __builtin_amdgcn_exp2f(s2 - m2);
  m = m2;
  return c;
}

// Marks the workspace status word (sticky).
__device__ __forceinline__ void flag_status(uint32_t* status, uint32_t bits) {
  atomicOr(status, bits);
}

}  // namespace swgqa
