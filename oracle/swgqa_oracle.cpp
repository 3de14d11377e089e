// swgqa_oracle.cpp -- CPU oracle for one GroupQueryAttention step over a
// windowed KV cache.
//
// TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
// CPU-baseline leg of the benchmark may load or call this library.  It is the
// plain definition of what a step computes, written out in fp64 with one
// fixed loop order, and shares no code with the HIP library.
//
// Sources (page title, section):
//  * "Specify GroupQueryAttention windowed KV cache layout contract"
//    (onnxruntime PR #32419), Description: the resident length L(T), the
//    row layout after a step, step-split invariance, the rollback rule, and
//    attention_bias columns in absolute key coordinates.
//  * "[CPU] Add windowed kv cache for GQA" (onnxruntime PR #31142), key design
//    decisions: gap = C - W + 1, the drifting layout, the per-item plan
//    (end before / end after / rows kept), staging of hazardous multi-token
//    steps, and results equal to those of a full-length cache.
//  * "GQA In-Place KV Cache: Investigation Report" (onnxruntime/mobius issue
//    #111), sections 1.1-1.3: operator inputs/outputs, BNSH caches,
//    seqlens_k = total length - 1, buffer-sharing modes, attributes (scale
//    default 1/sqrt(head_size), local_window_size, softcap).
//  * "Fix CPU Attention causal mask for q_len=1 with past_key and kv_len > 1"
//    (onnxruntime PR #34226), Description: query i sees key j iff
//    j <= i + past_sequence_length.
//
// Readings where the pages leave a step open (each is a single place below):
//  * window: a query at absolute position p sees keys p-W < j <= p (W keys
//    including itself) -- the PR #31142 design note says rows older than
//    end-W are already hidden by the window mask, which holds only for this
//    width;
//  * score order: scale, then softcap c*tanh(s/c), then + bias, then softmax;
//  * bias shape (B or 1, Hq or 1, S, total_sequence_length), row = query
//    index in the step, column = absolute key position;
//  * query head h reads KV head h / (Hq/Hkv);
//  * seqlens_k[b]+1 < S or > total_sequence_length is an error for item b;
//  * outputs are rounded to nearest-even from fp64; cache rows are byte
//    copies;
//  * rotary embedding (Investigation Report sections 1.1 and 1.3 name the
//    inputs cos_cache / sin_cache (max_S, D/2), position_ids (B, S) and the
//    attributes do_rotary / rotary_interleaved, without formulas): query and
//    new key rows are rotated before attention and before they are stored;
//    the pair (a, b) -- elements (k, k + D/2), or (2k, 2k + 1) when
//    interleaved -- at position pos becomes (a c - b s, b c + a s) with
//    c = cos_cache[pos][k], s = sin_cache[pos][k], each product, sum and
//    difference rounded to binary32, then the result to the element type;
//    pos = position_ids[b][i], or P + i without them; a position outside the
//    caches makes the item invalid (status 4, zero output, present untouched);
//  * softmax sink (Investigation Report sections 1.1 and 1.3 name the input
//    head_sink, one value per query head, and the attribute smooth_softmax
//    without defining them): one more logit -- head_sink[h] as given, or 0
//    when only smooth_softmax is set -- joins the softmax denominator with a
//    zero value row: out = sum_j e^{s_j} v_j / (e^{sink} + sum_j e^{s_j});
//  * quantized cache (the Investigation Report, section 1.1, names inputs
//    k_scale / v_scale, "KV cache quantization scale", and a cache type
//    T_CACHE apart from T, without formulas): with kv_cache_type = 1 the
//    caches hold int8 codes, one scale per tensor (k_scale for keys, v_scale
//    for values); a cache element stands for code * scale; a new row element
//    x (after rotary) is stored as the code nearest to x / scale -- the
//    quotient rounded to binary32, then to an integer with ties to even,
//    then saturated to [-128, 127] -- and every key and value row the step
//    attends to, the new ones included, is read in that dequantized form;
//    with kv_cache_type = 2 the codes are fp8 E4M3 (OCP "FN": bias 7, no
//    infinities, 0x7F / 0xFF NaN, largest finite 448): the quotient rounded to
//    the nearest E4M3 value, ties to the even code, magnitudes of 448 or more
//    saturated to 448, NaN to 0x7F.

#include "swgqa_oracle.h"

#include <cmath>
#include <cstring>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

int g_threads = 0;

// ---------------------------------------------------------------------------
// Resident length, PR #32419 Description (the L(T) formula) and PR #31142
// key design decisions (end(T) of the drifting layout): with G = C - W + 1,
// L(T) = T while T <= C, else T - G * ceil((T - C) / G).  int64 throughout,
// as the PR #31142 review thread asks.
int64_t resident_length(int64_t T, int64_t C, int64_t W) {
  const int64_t G = C - W + 1;
  if (T <= C) return T;
  const int64_t blocks = (T - C + G - 1) / G;  // ceil((T - C) / G), T > C
  return T - G * blocks;
}

struct Plan {
  int64_t T, P, Lb, La, kept, shift, first, hazard;
};

// Per-item plan, PR #31142 review thread (the planner) and key design
// decisions (staging): T = seqlens_k[b] + 1, P = T - S, resident rows before
// and after the step, rows of the old cache that survive, and whether
// compacting before attention would drop history the first query reads.
bool make_plan(int32_t seqlen_k, int64_t S, int64_t C, int64_t W, int64_t total,
               Plan* pl) {
  const int64_t T = (int64_t)seqlen_k + 1;
  const int64_t P = T - S;
  if (P < 0 || T > total) return false;
  pl->T = T;
  pl->P = P;
  pl->Lb = resident_length(P, C, W);
  pl->La = resident_length(T, C, W);
  pl->kept = pl->La - S;
  pl->shift = pl->Lb + S - pl->La;
  pl->first = T - pl->La;
  const int64_t need = P < W - 1 ? P : W - 1;  // history rows query 0 reads
  pl->hazard = pl->kept < need ? 1 : 0;
  return true;
}

// ---------------------------------------------------------------------------
// Element conversions.  fp16 = IEEE binary16, bf16 = top half of binary32.
size_t elem_bytes(int32_t dt) { return dt == 0 ? 4 : 2; }


double decode_f16(uint32_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 31;
  const int m = h & 1023;
  double v;
  if (e == 0) v = std::ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp((double)(1024 + m), e - 25);
  return sign ? -v : v;
}

double decode_bf16(uint32_t h) {
  const uint32_t u = h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// Round |x| to nearest-even in a binary format with p significant bits whose
// smallest normal binade is 2^emin and largest is 2^emax; overflow -> inf.
double round_format(double x, int p, int emin, int emax) {
  if (x == 0.0 || std::isnan(x) || std::isinf(x)) return x;
  const double a = std::fabs(x);
  int e;
  std::frexp(a, &e);                 // a = m * 2^e, m in [0.5, 1)
  int lead = e - 1;                  // exponent of the leading bit
  if (lead < emin) lead = emin;      // subnormal range: fixed quantum
  const int q = lead - (p - 1);      // exponent of one unit in the last place
  const double r = std::ldexp(std::nearbyint(std::ldexp(a, -q)), q);
  const double r_ok = (r >= std::ldexp(1.0, emax + 1)) ? INFINITY : r;
  return x < 0 ? -r_ok : r_ok;
}

uint32_t encode_f16(double x) {
  if (std::isnan(x)) return 0x7E00u;
  const double r = round_format(x, 11, -14, 15);
  const uint32_t sign = std::signbit(r) ? 0x8000u : 0u;
  const double a = std::fabs(r);
  if (std::isinf(a)) return sign | 0x7C00u;
  if (a == 0.0) return sign;
  int e;
  std::frexp(a, &e);
  const int lead = e - 1;
  if (lead < -14) return sign | (uint32_t)std::ldexp(a, 24);  // subnormal
  const uint32_t mant = (uint32_t)std::ldexp(a, 10 - lead) - 1024u;
  return sign | ((uint32_t)(lead + 15) << 10) | mant;
}

uint32_t encode_bf16(double x) {
  if (std::isnan(x)) return 0x7FC0u;
  const double r = round_format(x, 8, -126, 127);
  const float f = (float)r;  // exact: r is representable in binary32
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u >> 16;
}

double load(int32_t dt, const void* base, size_t idx) {
  if (dt == 0) {
    float f;
    std::memcpy(&f, (const char*)base + 4 * idx, 4);
    return (double)f;
  }
  uint16_t h;
  std::memcpy(&h, (const char*)base + 2 * idx, 2);
  return dt == 1 ? decode_f16(h) : decode_bf16(h);
}

void store(int32_t dt, void* base, size_t idx, double x) {
  if (dt == 0) {
    const float f = (float)x;  // C++ conversion rounds to nearest-even
    std::memcpy((char*)base + 4 * idx, &f, 4);
    return;
  }
  const uint16_t h = (uint16_t)(dt == 1 ? encode_f16(x) : encode_bf16(x));
  std::memcpy((char*)base + 2 * idx, &h, 2);
}

// Bytes of one cache element: the element type, or one int8 code.
size_t cache_elem_bytes(const swgqa_oracle_params* p) {
  return p->kv_cache_type != 0 ? 1 : elem_bytes(p->dtype);
}

// The int8 code of x for a quantization scale (binary32 quotient, ties to
// even, saturation).
int8_t quantize_int8(double x, float scale) {
  const float t = std::nearbyint((float)x / scale);  // default mode: ties to even
  if (!(t > -128.0f)) return (int8_t)-128;
  if (t > 127.0f) return (int8_t)127;
  return (int8_t)t;
}

// Value of an fp8 E4M3 ("FN") code: sign, 4 exponent bits (bias 7), 3
// mantissa bits; exponent 0 is subnormal (m * 2^-9); 0x7F / 0xFF are NaN.
double decode_e4m3(uint8_t c) {
  if ((c & 0x7F) == 0x7F) return NAN;
  const int e = (c >> 3) & 15, m = c & 7;
  const double mag = e == 0 ? std::ldexp((double)m, -9) : std::ldexp(8.0 + m, e - 10);
  return (c & 0x80) ? -mag : mag;
}

// The fp8 E4M3 code of x for a quantization scale: the binary32 quotient
// rounded to the nearest finite code value by search over all codes (ties to
// the even code), saturated at 448, NaN to 0x7F.
uint8_t quantize_e4m3(double x, float scale) {
  const float t = (float)x / scale;
  if (t != t) return 0x7F;
  const double a = std::fabs((double)t);
  uint8_t best = 0;
  if (a >= 448.0) {
    best = 0x7E;
  } else {
    double bd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
      const double d = std::fabs(decode_e4m3((uint8_t)c) - a);
      if (d < bd || (d == bd && (c & 1) == 0)) {
        bd = d;
        best = (uint8_t)c;
      }
    }
  }
  return (uint8_t)(best | (t < 0.0f && best != 0 ? 0x80 : 0));
}

// Element idx of a cache row buffer (element type, or a dequantized code).
double load_cache(const swgqa_oracle_params* p, const void* base, size_t idx, float scale) {
  if (p->kv_cache_type == 0) return load(p->dtype, base, idx);
  uint8_t c;
  std::memcpy(&c, (const char*)base + idx, 1);
  if (p->kv_cache_type == 2) return decode_e4m3(c) * (double)scale;  // exact in fp64
  return (double)(int8_t)c * (double)scale;
}

// ---------------------------------------------------------------------------
int validate(const swgqa_oracle_params* p) {
  if (!p) return 1;
  if (p->batch_size < 0 || p->sequence_length < 1 || p->num_heads < 1 ||
      p->kv_num_heads < 1 || p->head_size < 1)
    return 1;
  if (p->num_heads % p->kv_num_heads != 0) return 1;
  // local_window_size = -1 ("disabled") leaves the gap undefined: rejected.
  if (p->local_window_size < 1 || p->local_window_size > p->capacity) return 1;
  if (p->total_sequence_length < 1) return 1;
  if (p->dtype < 0 || p->dtype > 2) return 2;
  if (!(p->scale >= 0.0f) || !(p->softcap >= 0.0f)) return 1;
  if (p->smooth_softmax != 0 && p->smooth_softmax != 1) return 1;
  if (p->do_rotary != 0 && p->do_rotary != 1) return 1;
  if (p->do_rotary && (p->head_size % 2 != 0 || p->rotary_cache_rows < 1)) return 1;
  if (p->kv_cache_type < 0 || p->kv_cache_type > 2) return 2;
  if (p->kv_cache_type != 0 &&
      !(p->k_scale > 0.0f && p->v_scale > 0.0f && std::isfinite(p->k_scale) &&
        std::isfinite(p->v_scale)))
    return 1;
  return 0;
}

// Rotary embedding of rows [0, nrows) of a (B, S, heads, D) tensor in place
// (a private copy of query or key).  ok[b] is cleared for an item with a
// position outside the cos/sin caches.
void rotate_rows(const swgqa_oracle_params* p, void* x, int64_t heads, const Plan* plans,
                 std::vector<char>& ok, const void* cos_cache, const void* sin_cache,
                 const int64_t* position_ids) {
  const int64_t B = p->batch_size, S = p->sequence_length, D = p->head_size;
  const int64_t half = D / 2;
  for (int64_t b = 0; b < B; ++b) {
    if (!ok[b]) continue;
    for (int64_t i = 0; i < S; ++i) {
      const int64_t pos = position_ids ? position_ids[b * S + i] : plans[b].P + i;
      if (pos < 0 || pos >= p->rotary_cache_rows) {
        ok[b] = 0;
        break;
      }
    }
  }
  for (int64_t b = 0; b < B; ++b) {
    if (!ok[b]) continue;
    for (int64_t i = 0; i < S; ++i) {
      const int64_t pos = position_ids ? position_ids[b * S + i] : plans[b].P + i;
      for (int64_t h = 0; h < heads; ++h) {
        const size_t row = (size_t)((b * S + i) * heads + h) * D;
        for (int64_t k = 0; k < half; ++k) {
          const size_t ia = row + (p->rotary_interleaved ? 2 * k : k);
          const size_t ib = row + (p->rotary_interleaved ? 2 * k + 1 : k + half);
          const float a = (float)load(p->dtype, x, ia);
          const float bv = (float)load(p->dtype, x, ib);
          const float c = (float)load(p->dtype, cos_cache, (size_t)(pos * half + k));
          const float sn = (float)load(p->dtype, sin_cache, (size_t)(pos * half + k));
          const float ac = a * c, bs = bv * sn, bc = bv * c, as = a * sn;
          const float ra = ac - bs;
          const float rb = bc + as;
          store(p->dtype, x, ia, (double)ra);
          store(p->dtype, x, ib, (double)rb);
        }
      }
    }
  }
}

// Buffer-sharing modes, Investigation Report section 1.2: past and present
// are the same buffer (in place) or separate; a partial overlap is neither.
bool partial_overlap(const void* a, const void* b, size_t n) {
  const char* x = (const char*)a;
  const char* y = (const char*)b;
  if (x == y) return false;
  return x < y + n && y < x + n;
}

double default_scale(const swgqa_oracle_params* p) {
  return p->scale > 0.0f ? (double)p->scale : 1.0 / std::sqrt((double)p->head_size);
}

// Score transform for one (query, key) pair: scale, softcap, bias.
double finish_score(const swgqa_oracle_params* p, double dot, double scale,
                    const void* bias, int64_t b, int64_t h, int64_t i,
                    int64_t j) {
  double s = scale * dot;
  if (p->softcap > 0.0f) {
    const double c = (double)p->softcap;
    s = c * std::tanh(s / c);
  }
  if (bias) {
    const int64_t bb = p->bias_dim0_is_batch ? b : 0;
    const int64_t bh = p->bias_dim1_is_heads ? h : 0;
    const int64_t Hb = p->bias_dim1_is_heads ? p->num_heads : 1;
    const size_t idx = (size_t)(((bb * Hb + bh) * p->sequence_length + i) *
                                    (int64_t)p->total_sequence_length + j);
    s += load(p->dtype, bias, idx);
  }
  return s;
}

// Softmax-weighted sum over the visible keys of one query.  keys[t] / vals[t]
// are element pointers into rows whose absolute positions ascend with t;
// js[t] is that absolute position.
void attend_one(const swgqa_oracle_params* p, const void* qrow, size_t qoff,
                const std::vector<const void*>& krow,
                const std::vector<size_t>& koff,
                const std::vector<const void*>& vrow,
                const std::vector<size_t>& voff, const std::vector<int64_t>& js,
                double scale, const void* bias, const void* sink, int64_t b, int64_t h,
                int64_t i, void* out, size_t ooff) {
  const int64_t D = p->head_size;
  const size_t n = js.size();
  std::vector<double> s(n);
  double m = -INFINITY;
  for (size_t t = 0; t < n; ++t) {
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d)
      dot += load(p->dtype, qrow, qoff + d) * load_cache(p, krow[t], koff[t] + d, p->k_scale);
    s[t] = finish_score(p, dot, scale, bias, b, h, i, js[t]);
    if (s[t] > m) m = s[t];
  }
  // the sink logit joins the denominator only (its value row is zero)
  const bool has_sink = sink != nullptr || p->smooth_softmax != 0;
  const double sink_logit = sink ? load(p->dtype, sink, (size_t)h) : 0.0;
  if (has_sink && sink_logit > m) m = sink_logit;
  double l = has_sink ? std::exp(sink_logit - m) : 0.0;
  for (size_t t = 0; t < n; ++t) {
    s[t] = std::exp(s[t] - m);
    l += s[t];
  }
  for (int64_t d = 0; d < D; ++d) {
    double acc = 0.0;
    for (size_t t = 0; t < n; ++t) acc += s[t] * load_cache(p, vrow[t], voff[t] + d, p->v_scale);
    store(p->dtype, out, ooff + d, acc / l);
  }
}

}  // namespace

extern "C" {

int64_t swgqa_oracle_resident_length(int64_t T, int64_t C, int64_t W) {
  return resident_length(T, C, W);
}

void swgqa_oracle_resident_lengths(const int64_t* T, int64_t n, int64_t C,
                                   int64_t W, int64_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = resident_length(T[i], C, W);
}

// Rollback rule ("Specify GroupQueryAttention windowed KV cache layout
// contract", Description): dropping the last k of T positions leaves the
// cache valid as it stands iff L(T - k) == L(T) - k.
int swgqa_oracle_rollback_exact(int64_t T, int64_t k, int64_t C, int64_t W) {
  if (k < 0 || k > T) return 0;
  return resident_length(T - k, C, W) == resident_length(T, C, W) - k ? 1 : 0;
}

int swgqa_oracle_plan(const swgqa_oracle_params* p, const int32_t* seqlens_k,
                      int64_t* plan_out) {
  const int v = validate(p);
  if (v) return v;
  int status = 0;
  for (int64_t b = 0; b < p->batch_size; ++b) {
    Plan pl;
    int64_t* o = plan_out + SWGQA_ORACLE_PLAN_FIELDS * b;
    if (!make_plan(seqlens_k[b], p->sequence_length, p->capacity,
                   p->local_window_size, p->total_sequence_length, &pl)) {
      for (int f = 0; f < SWGQA_ORACLE_PLAN_FIELDS; ++f) o[f] = -1;
      status = 4;
      continue;
    }
    const int64_t f[8] = {pl.T, pl.P, pl.Lb, pl.La, pl.kept, pl.shift, pl.first, pl.hazard};
    std::memcpy(o, f, sizeof f);
  }
  return status;
}

int swgqa_oracle_forward(const swgqa_oracle_params* p, const void* query,
                         const void* key, const void* value,
                         const void* past_key, const void* past_value,
                         const int32_t* seqlens_k, const void* attention_bias,
                         const void* head_sink, const void* cos_cache,
                         const void* sin_cache, const int64_t* position_ids,
                         void* output, void* present_key, void* present_value,
                         int64_t* plan_out) {
  const int v = validate(p);
  if (v) return v;
  const int64_t B = p->batch_size, S = p->sequence_length, Hq = p->num_heads,
                Hkv = p->kv_num_heads, D = p->head_size, C = p->capacity,
                W = p->local_window_size;
  if (B == 0) return 0;
  if (!query || !key || !value || !past_key || !past_value || !seqlens_k ||
      !output || !present_key || !present_value)
    return 1;
  const size_t e = elem_bytes(p->dtype);
  const size_t ce = cache_elem_bytes(p);
  const size_t cache_bytes = (size_t)(B * Hkv * C * D) * ce;
  if (partial_overlap(past_key, present_key, cache_bytes) ||
      partial_overlap(past_value, present_value, cache_bytes))
    return 3;
  const int64_t group = Hq / Hkv;
  const double scale = default_scale(p);

  // 1. Plans.
  std::vector<Plan> plans((size_t)B);
  std::vector<char> ok((size_t)B, 0);
  int status = 0;
  for (int64_t b = 0; b < B; ++b) {
    ok[b] = make_plan(seqlens_k[b], S, C, W, p->total_sequence_length, &plans[b]);
    if (!ok[b]) status = 4;
  }
  if (plan_out) swgqa_oracle_plan(p, seqlens_k, plan_out);

  // 1b. Rotary embedding of private copies of the query and the new keys.
  std::vector<char> qrot, krot;
  if (p->do_rotary) {
    if (!cos_cache || !sin_cache) return 1;
    const size_t e0 = elem_bytes(p->dtype);
    qrot.assign((const char*)query, (const char*)query + (size_t)(B * S * Hq * D) * e0);
    krot.assign((const char*)key, (const char*)key + (size_t)(B * S * Hkv * D) * e0);
    rotate_rows(p, qrot.data(), Hq, plans.data(), ok, cos_cache, sin_cache, position_ids);
    rotate_rows(p, krot.data(), Hkv, plans.data(), ok, cos_cache, sin_cache, position_ids);
    for (int64_t b = 0; b < B; ++b)
      if (!ok[b]) {
        status = 4;
        if (plan_out)
          for (int f = 0; f < SWGQA_ORACLE_PLAN_FIELDS; ++f) plan_out[SWGQA_ORACLE_PLAN_FIELDS * b + f] = -1;
      }
    query = qrot.data();
    key = krot.data();
  }

  // 2. Logical concatenation per (b, kvh): the Lb resident rows followed by
  //    the S new rows; row r holds absolute position P - Lb + r.  A separate
  //    allocation, so writing present afterwards is safe when present==past.
  //    New rows enter in the cache's form (int8 codes when quantized).
  std::vector<std::vector<char>> XK((size_t)(B * Hkv)), XV((size_t)(B * Hkv));
  const size_t row = (size_t)D * ce;
  for (int64_t b = 0; b < B; ++b) {
    if (!ok[b]) continue;
    const Plan& pl = plans[b];
    for (int64_t g = 0; g < Hkv; ++g) {
      std::vector<char>& xk = XK[b * Hkv + g];
      std::vector<char>& xv = XV[b * Hkv + g];
      xk.resize((size_t)(pl.Lb + S) * row);
      xv.resize((size_t)(pl.Lb + S) * row);
      const size_t slice = (size_t)((b * Hkv + g) * C) * row;
      if (pl.Lb > 0) {
        std::memcpy(xk.data(), (const char*)past_key + slice, (size_t)pl.Lb * row);
        std::memcpy(xv.data(), (const char*)past_value + slice, (size_t)pl.Lb * row);
      }
      for (int64_t i = 0; i < S; ++i) {
        const size_t src = (size_t)((b * S + i) * Hkv + g) * D;  // element index
        char* dk = xk.data() + (size_t)(pl.Lb + i) * row;
        char* dv = xv.data() + (size_t)(pl.Lb + i) * row;
        if (p->kv_cache_type == 1) {
          for (int64_t d = 0; d < D; ++d) {
            const int8_t qk = quantize_int8(load(p->dtype, key, src + d), p->k_scale);
            const int8_t qv = quantize_int8(load(p->dtype, value, src + d), p->v_scale);
            std::memcpy(dk + d, &qk, 1);
            std::memcpy(dv + d, &qv, 1);
          }
        } else if (p->kv_cache_type == 2) {
          for (int64_t d = 0; d < D; ++d) {
            const uint8_t qk = quantize_e4m3(load(p->dtype, key, src + d), p->k_scale);
            const uint8_t qv = quantize_e4m3(load(p->dtype, value, src + d), p->v_scale);
            std::memcpy(dk + d, &qk, 1);
            std::memcpy(dv + d, &qv, 1);
          }
        } else {
          std::memcpy(dk, (const char*)key + src * e, row);
          std::memcpy(dv, (const char*)value + src * e, row);
        }
      }
    }
  }

  int broken = 0;
  // 3. Attention per (b, h, i) in absolute coordinates: query i sits at
  //    p = P + i and sees keys max(0, p - W + 1) .. p (causal rule of
  //    PR #34226 with past = P, intersected with the local window).
#ifdef _OPENMP
  const int nth = g_threads > 0 ? g_threads : omp_get_max_threads();
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(nth) reduction(| : broken)
#endif
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t h = 0; h < Hq; ++h) {
      if (!ok[b]) {
        for (int64_t i = 0; i < S; ++i)
          for (int64_t d = 0; d < D; ++d)
            store(p->dtype, output, (size_t)((b * S + i) * Hq + h) * D + d, 0.0);
        continue;
      }
      const Plan& pl = plans[b];
      const int64_t g = h / group;
      const std::vector<char>& xk = XK[b * Hkv + g];
      const std::vector<char>& xv = XV[b * Hkv + g];
      const int64_t base = pl.P - pl.Lb;  // absolute position of concat row 0
      for (int64_t i = 0; i < S; ++i) {
        const int64_t pos = pl.P + i;
        const int64_t lo = pos - W + 1 > 0 ? pos - W + 1 : 0;
        std::vector<const void*> kr, vr;
        std::vector<size_t> ko, vo;
        std::vector<int64_t> js;
        for (int64_t j = lo; j <= pos; ++j) {
          const int64_t r = j - base;  // >= 0 because Lb >= min(P, W)
          if (r < 0 || r >= pl.Lb + S) {  // cannot happen; reported if it does
            broken = 1;
            continue;
          }
          kr.push_back(xk.data());
          ko.push_back((size_t)r * D);
          vr.push_back(xv.data());
          vo.push_back((size_t)r * D);
          js.push_back(j);
        }
        attend_one(p, query, (size_t)((b * S + i) * Hq + h) * D, kr, ko, vr, vo,
                   js, scale, attention_bias, head_sink, b, h, i, output,
                   (size_t)((b * S + i) * Hq + h) * D);
      }
    }
  }

  if (broken) return 1;
  // 4. Present rows [0, La) = the newest La rows of the concatenation; rows
  //    [La, C) are left as they were (unspecified by the contract).
  for (int64_t b = 0; b < B; ++b) {
    if (!ok[b]) continue;
    const Plan& pl = plans[b];
    for (int64_t g = 0; g < Hkv; ++g) {
      const size_t slice = (size_t)((b * Hkv + g) * C) * row;
      const size_t from = (size_t)(pl.Lb + S - pl.La) * row;
      std::memcpy((char*)present_key + slice, XK[b * Hkv + g].data() + from,
                  (size_t)pl.La * row);
      std::memcpy((char*)present_value + slice, XV[b * Hkv + g].data() + from,
                  (size_t)pl.La * row);
    }
  }
  return status;
}

int swgqa_oracle_forward_compact_first(const swgqa_oracle_params* p,
                                       const void* query, const void* key,
                                       const void* value, void* cache_key,
                                       void* cache_value,
                                       const int32_t* seqlens_k,
                                       const void* attention_bias,
                                       const void* head_sink, void* output) {
  const int v = validate(p);
  if (v) return v;
  if (p->kv_cache_type != 0) return 2;  // only the plain cache pins the staging rule
  const int64_t B = p->batch_size, S = p->sequence_length, Hq = p->num_heads,
                Hkv = p->kv_num_heads, D = p->head_size, C = p->capacity,
                W = p->local_window_size;
  const size_t e = elem_bytes(p->dtype);
  const size_t row = (size_t)D * e;
  const int64_t group = Hq / Hkv;
  const double scale = default_scale(p);
  int status = 0;
  for (int64_t b = 0; b < B; ++b) {
    Plan pl;
    if (!make_plan(seqlens_k[b], S, C, W, p->total_sequence_length, &pl)) return 4;
    // Compaction first (PR #31142, the per-slice row move), then append.
    for (int64_t g = 0; g < Hkv; ++g) {
      char* ck = (char*)cache_key + (size_t)((b * Hkv + g) * C) * row;
      char* cv = (char*)cache_value + (size_t)((b * Hkv + g) * C) * row;
      if (pl.kept > 0) {
        std::memmove(ck, ck + (size_t)pl.shift * row, (size_t)pl.kept * row);
        std::memmove(cv, cv + (size_t)pl.shift * row, (size_t)pl.kept * row);
      }
      for (int64_t i = 0; i < S; ++i) {
        const int64_t r = pl.kept + i;  // row of new token i
        if (r < 0) continue;            // dropped by an S > C step
        const size_t src = (size_t)((b * S + i) * Hkv + g) * row;
        std::memcpy(ck + (size_t)r * row, (const char*)key + src, row);
        std::memcpy(cv + (size_t)r * row, (const char*)value + src, row);
      }
    }
    // Attention over cache rows only: row r holds position T - La + r.
    const int64_t base = pl.T - pl.La;
    for (int64_t h = 0; h < Hq; ++h) {
      const int64_t g = h / group;
      const char* ck = (const char*)cache_key + (size_t)((b * Hkv + g) * C) * row;
      const char* cv = (const char*)cache_value + (size_t)((b * Hkv + g) * C) * row;
      for (int64_t i = 0; i < S; ++i) {
        const int64_t pos = pl.P + i;
        const int64_t lo = pos - W + 1 > 0 ? pos - W + 1 : 0;
        std::vector<const void*> kr, vr;
        std::vector<size_t> ko, vo;
        std::vector<int64_t> js;
        for (int64_t j = lo; j <= pos; ++j) {
          const int64_t r = j - base;
          if (r < 0) {  // evicted before this query could read it
            status = 5;
            continue;
          }
          kr.push_back(ck);
          ko.push_back((size_t)r * D);
          vr.push_back(cv);
          vo.push_back((size_t)r * D);
          js.push_back(j);
        }
        attend_one(p, query, (size_t)((b * S + i) * Hq + h) * D, kr, ko, vr, vo,
                   js, scale, attention_bias, head_sink, b, h, i, output,
                   (size_t)((b * S + i) * Hq + h) * D);
      }
    }
  }
  return status;
}

uint32_t swgqa_oracle_quantize_e4m3(double x, float scale) { return quantize_e4m3(x, scale); }

double swgqa_oracle_decode_e4m3(uint32_t code) { return decode_e4m3((uint8_t)code); }

double swgqa_oracle_decode(int32_t dtype, uint32_t bits) {
  if (dtype == 0) {
    float f;
    std::memcpy(&f, &bits, 4);
    return (double)f;
  }
  return dtype == 1 ? decode_f16(bits & 0xFFFFu) : decode_bf16(bits & 0xFFFFu);
}

uint32_t swgqa_oracle_encode(int32_t dtype, double x) {
  if (dtype == 0) {
    const float f = (float)x;
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return u;
  }
  return dtype == 1 ? encode_f16(x) : encode_bf16(x);
}

int swgqa_oracle_set_threads(int n) {
  g_threads = n > 0 ? n : 0;
#ifdef _OPENMP
  return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
  return 1;
#endif
}

}  // extern "C"
