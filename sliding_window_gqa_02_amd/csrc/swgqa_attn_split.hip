// swgqa_attn_split.hip -- split-K grouped-query attention over a windowed KV
// cache for short steps (decode and small multi-token steps), on CDNA4.
//
// What is computed ("Specify GroupQueryAttention windowed KV cache layout
// contract", Description; "Fix CPU Attention causal mask ..." Description;
// "GQA In-Place KV Cache: Investigation Report" 1.1-1.3): query i of item b
// sits at absolute position p = P + i and attends to keys p - W < j <= p of
// the logical concatenation [resident rows | S new rows].  Keys below P are
// read from the cache at row j - (P - Lb); keys from P on are read straight
// from the new key/value rows.  This two-segment read is the staging buffer
// of "[CPU] Add windowed kv cache for GQA" (staging for hazardous steps)
// without a copy: the cache is only rewritten after attention (write-back
// kernel), so no history a query reads is ever lost.
//
// Work decomposition: one workgroup (4 wave64s) per (item, KV head, query
// tile, key split).  A query tile is NQ consecutive (position, head) pairs of
// the KV head's group, so every K/V row loaded is used by all NQ queries.
// Lanes are laid out as (row, sub): LPR lanes share one key row, each holding
// E = D / LPR elements; scores are reduced across those LPR lanes.  Each row
// slot keeps its own online-softmax state (max, sum, accumulator); row slots
// and waves are merged once at the end.  With one split the workgroup writes
// the output; otherwise it writes (max, sum, accumulator) partials that
// the step-tail kernel (swgqa_step_tail.hip) merges.
#include "swgqa_common.hpp"
#include "swgqa_internal.hpp"
#include "swgqa_tail.hpp"

#include <math.h>

namespace swgqa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr float kLog2e = 1.4426950408889634f;
// NQ * D bound: keeps the per-wave merge buffer at <= 8 KiB.
constexpr int kMaxTileElems = kSplitMaxTileElems;

template <int DT, int D, int NQ>
struct SplitShape {
  static constexpr int e = Elem<DT>::bytes;
  static constexpr int EPW = 4 / e;                   // elements per 32-bit word
  static constexpr int E0 = 64 / NQ;                  // keep NQ*E <= 64 floats
  static constexpr int E1 = E0 < EPW ? EPW : E0;
  static constexpr int E = E1 > D ? D : E1;           // elements per lane
  static constexpr int LPR = D / E;                   // lanes per key row
  static constexpr int RPW = kWave / LPR;             // key rows per wave step
  static constexpr int NW = E / EPW;                  // 32-bit words per lane
  static_assert(LPR >= 1 && LPR <= kWave && (LPR & (LPR - 1)) == 0, "lanes per row");
};

__device__ __forceinline__ float xor_shfl(float x, int mask) {
  return __shfl_xor(x, mask, kWave);
}

template <int DT, int D, int NQ>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(AttnArgs a) {
  using Sh = SplitShape<DT, D, NQ>;
  constexpr int E = Sh::E, LPR = Sh::LPR, RPW = Sh::RPW, NW = Sh::NW, e = Sh::e;

  const int b = blockIdx.z;
  const int kvh = blockIdx.y;
  const int tile = blockIdx.x / a.nsplit;
  const int split = blockIdx.x % a.nsplit;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int rslot = lane / LPR;   // row slot within a wave step
  const int sub = lane % LPR;     // element chunk within the row

  const ItemPlan pl = plan_item(a.seqlens[b], a.S, a.C, a.gdiv, a.total);
  const int nq_item = a.S * a.group;
  const int q0 = tile * NQ;

  __shared__ float s_m[kWaves][NQ];
  __shared__ float s_l[kWaves][NQ];
  __shared__ float s_acc[kWaves][NQ][D];

  if (!pl.ok) {
    if (tid == 0 && tile == 0 && split == 0 && kvh == 0) flag_status(a.status, kStatusBadItem);
    // zero-filled output (or empty partials) for every query of the tile
    for (int idx = tid; idx < NQ * D; idx += kThreads) {
      const int t = idx / D, d = idx % D;
      const int qi = q0 + t;
      if (qi >= nq_item) continue;
      const int i = qi / a.group, h = kvh * a.group + qi % a.group;
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

  // Fused append on drifting steps with a shared buffer: rows [Lb, Lb + S)
  // are beyond every row attention reads, so they can be written now.
  if (a.present_k && pl.shift == 0 && tile == 0 && split == 0) {
    constexpr int W16 = D * e / 16;
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

  // Query tile: NQ (position, head) pairs, position-major.
  float qv[NQ][E];
  int64_t qpos[NQ];
  bool qok[NQ];
  int i_first = q0 / a.group;
  int i_last = (min(q0 + NQ, nq_item) - 1) / a.group;
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    const int qi = q0 + t;
    qok[t] = qi < nq_item;
    const int i = qok[t] ? qi / a.group : i_last;
    const int h = kvh * a.group + (qok[t] ? qi % a.group : 0);
    qpos[t] = pl.P + i;
    const char* qp = (const char*)a.q + ((((int64_t)b * a.S + i) * a.Hq + h) * D + sub * E) * e;
    uint32_t w[NW];
    load_words<NW>(qp, w);
#pragma unroll
    for (int k = 0; k < NW; ++k) unpack_word<DT>(w[k], &qv[t][k * Sh::EPW]);
#pragma unroll
    for (int k = 0; k < E; ++k) qv[t][k] = qok[t] ? qv[t][k] * a.scale : 0.0f;
  }

  // Union key range of the tile, split evenly across the splits.
  const int64_t p_first = pl.P + i_first;
  const int64_t p_last = pl.P + i_last;
  const int64_t lo = p_first - a.W + 1 > 0 ? p_first - a.W + 1 : 0;
  const int64_t n = p_last - lo + 1;
  const int64_t chunk = (n + a.nsplit - 1) / a.nsplit;
  const int64_t kb = lo + split * chunk;
  const int64_t ke = kb + chunk < p_last + 1 ? kb + chunk : p_last + 1;

  float m[NQ], l[NQ], acc[NQ][E];
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    m[t] = -INFINITY;
    l[t] = 0.0f;
#pragma unroll
    for (int k = 0; k < E; ++k) acc[t][k] = 0.0f;
  }

  const int64_t base = pl.P - pl.Lb;  // absolute position of cache row 0
  const char* cache_k = (const char*)a.past_k + ((int64_t)(b * a.Hkv + kvh) * a.C) * D * e;
  const char* cache_v = (const char*)a.past_v + ((int64_t)(b * a.Hkv + kvh) * a.C) * D * e;
  const bool has_bias = a.bias != nullptr;
  const bool has_cap = a.softcap > 0.0f;
  const float cap = a.softcap;
  const float inv_cap = a.inv_softcap;  // (made on the host)

  for (int64_t j0 = kb + (int64_t)wave * RPW; j0 < ke; j0 += (int64_t)kWaves * RPW) {
    const int64_t j = j0 + rslot;
    const bool jok = j < ke;
    const char* kp;
    const char* vp;
    if (j < pl.P) {
      const int64_t r = j - base;
      kp = cache_k + (r * D + sub * E) * e;
      vp = cache_v + (r * D + sub * E) * e;
    } else {
      const int64_t off = ((((int64_t)b * a.S + (j - pl.P)) * a.Hkv + kvh) * D + sub * E) * e;
      kp = (const char*)a.k + off;
      vp = (const char*)a.v + off;
    }
    uint32_t kw[NW], vw[NW];
    if (jok) {
      load_words<NW>(kp, kw);
      load_words<NW>(vp, vw);
    } else {
#pragma unroll
      for (int k = 0; k < NW; ++k) kw[k] = vw[k] = 0u;
    }
    float kf[E];
#pragma unroll
    for (int k = 0; k < NW; ++k) unpack_word<DT>(kw[k], &kf[k * Sh::EPW]);

    float s[NQ];
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      float acc_s = 0.0f;
#pragma unroll
      for (int k = 0; k < E; ++k) acc_s = fmaf(qv[t][k], kf[k], acc_s);
      s[t] = acc_s;
    }
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) {
#pragma unroll
      for (int t = 0; t < NQ; ++t) s[t] += xor_shfl(s[t], off);
    }
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      const bool vis = jok && qok[t] && j <= qpos[t] && j > qpos[t] - a.W;
      float x = s[t];
      if (has_cap) x = cap * tanhf(x * inv_cap);
      if (has_bias && vis) {
        const int qi = q0 + t;
        const int i = qi / a.group;
        const int h = kvh * a.group + qi % a.group;
        const int64_t bb = a.bias_b ? b : 0;
        const int64_t bh = a.bias_h ? h : 0;
        const int64_t hb = a.bias_h ? a.Hq : 1;
        x += load_one<DT>(a.bias, ((bb * hb + bh) * a.S + i) * (int64_t)a.total + j);
      }
      s[t] = vis ? x * kLog2e : -INFINITY;
    }

    float vf[E];
#pragma unroll
    for (int k = 0; k < NW; ++k) unpack_word<DT>(vw[k], &vf[k * Sh::EPW]);
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      const float mn = fmaxf(m[t], s[t]);
      const float corr = (m[t] == mn) ? 1.0f : exp2f(m[t] - mn);
      const float p = (s[t] == -INFINITY) ? 0.0f : exp2f(s[t] - mn);
      l[t] = l[t] * corr + p;
#pragma unroll
      for (int k = 0; k < E; ++k) acc[t][k] = fmaf(acc[t][k], corr, p * vf[k]);
      m[t] = mn;
    }
  }

  // Merge the row slots of this wave (lanes with equal `sub`).
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      const float mo = xor_shfl(m[t], off);
      const float lo2 = xor_shfl(l[t], off);
      const float mn = fmaxf(m[t], mo);
      const float ca = (m[t] == mn) ? 1.0f : exp2f(m[t] - mn);
      const float cb = (mo == mn) ? 1.0f : exp2f(mo - mn);
      l[t] = l[t] * ca + lo2 * cb;
#pragma unroll
      for (int k = 0; k < E; ++k) {
        const float ao = xor_shfl(acc[t][k], off);
        acc[t][k] = acc[t][k] * ca + ao * cb;
      }
      m[t] = mn;
    }
  }
  if (rslot == 0) {
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      if (sub == 0) {
        s_m[wave][t] = m[t];
        s_l[wave][t] = l[t];
      }
#pragma unroll
      for (int k = 0; k < E; ++k) s_acc[wave][t][sub * E + k] = acc[t][k];
    }
  }
  __syncthreads();

  // Merge the waves and write the output or the split partial.
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
      const float c = (s_m[w][t] == -INFINITY) ? 0.0f : exp2f(s_m[w][t] - M);
      L += s_l[w][t] * c;
      A += s_acc[w][t][d] * c;
    }
    const int i = qi / a.group, h = kvh * a.group + qi % a.group;
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
  slice_tail<DT>(a, pl, b, kvh, D);
}

template <int DT, int D, int NQ>
hipError_t launch_split_nq(const AttnArgs& a, hipStream_t st) {
  if constexpr (NQ * D <= kMaxTileElems) {
    const dim3 grid(a.ntiles * a.nsplit, a.Hkv, a.B);
    attn_split_kernel<DT, D, NQ><<<grid, kThreads, 0, st>>>(a);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <int DT, int D>
hipError_t launch_split_d(int nq, const AttnArgs& a, hipStream_t st) {
  switch (nq) {
    case 2: return launch_split_nq<DT, D, 2>(a, st);
    case 4: return launch_split_nq<DT, D, 4>(a, st);
    case 8: return launch_split_nq<DT, D, 8>(a, st);
    case 16: return launch_split_nq<DT, D, 16>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_split_t(int D, int nq, const AttnArgs& a, hipStream_t st) {
  switch (D) {
    case 8: return launch_split_d<DT, 8>(nq, a, st);
    case 16: return launch_split_d<DT, 16>(nq, a, st);
    case 32: return launch_split_d<DT, 32>(nq, a, st);
    case 64: return launch_split_d<DT, 64>(nq, a, st);
    case 128: return launch_split_d<DT, 128>(nq, a, st);
    case 256: return launch_split_d<DT, 256>(nq, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool head_size_supported(int D) {
  return D == 8 || D == 16 || D == 32 || D == 64 || D == 128 || D == 256;
}

hipError_t launch_attn_split(int dtype, int D, int nq, const AttnArgs& a,
                             hipStream_t st) {
  switch (dtype) {
    case kF32: return launch_split_t<kF32>(D, nq, a, st);
    case kF16: return launch_split_t<kF16>(D, nq, a, st);
    case kBF16: return launch_split_t<kBF16>(D, nq, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace swgqa
