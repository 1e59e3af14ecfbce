// device_common.hpp -- gfx950 device helpers shared by the verification and
// expansion kernels: the Philox4x32-10 stream, 8-element logit groups, and
// 64-lane wavefront / 256-thread workgroup reductions.
#pragma once

#include <float.h>
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

namespace specv {

constexpr int kWG = 256;           // threads per workgroup (4 wave64)
constexpr int kWaves = kWG / 64;

// ---------------------------------------------------------------- Philox --
// Philox4x32-10 (Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3",
// SC'11): per round the two multipliers give 64-bit products of counter
// words 0 and 2, whose halves are recombined with words 1, 3 and the round
// key; the key advances by the Weyl increments after every round.
struct Philox4 {
  uint32_t w[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                  uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint32_t a0 = 0xD2511F53u * c0, b0 = __umulhi(0xD2511F53u, c0);
    const uint32_t a2 = 0xCD9E8D57u * c2, b2 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = b2 ^ c1 ^ k0;
    const uint32_t n2 = b0 ^ c3 ^ k1;
    c0 = n0;
    c1 = a2;
    c2 = n2;
    c3 = a0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// 24 high bits of a word as a uniform in [0, 1); exact in float and double.
__device__ __forceinline__ double unit_uniform(uint32_t w) { return (double)(w >> 8) * 0x1p-24; }

// ---------------------------------------------------------- logit groups --
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// A group is 8 consecutive logits widened to fp32: one 16-byte load for bf16,
// two for fp32 (VEC), or 8 scalar loads when the row is not 16-byte aligned.
template <int ES, bool VEC>
__device__ __forceinline__ void load_group(const char* __restrict__ row, int64_t e0, float x[8]) {
  if constexpr (ES == 2) {
    if constexpr (VEC) {
      // streamed once: a non-temporal load keeps it from displacing reusable lines
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + e0 * 2));
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
      const uint16_t* r = reinterpret_cast<const uint16_t*>(row) + e0;
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __uint_as_float((uint32_t)r[i] << 16);
    }
  } else {
    if constexpr (VEC) {
      const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + e0 * 4));
      const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + e0 * 4 + 16));
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
      const float* r = reinterpret_cast<const float*>(row) + e0;
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = r[i];
    }
  }
}

// The same 8 logits kept as loaded (two bf16 per dword, or fp32), so that many
// groups can be in flight in few registers; widened by unpack_group.
template <int ES, bool VEC>
struct RawGroup;
template <>
struct RawGroup<2, true> {
  u32x4 v;
};
template <>
struct RawGroup<4, true> {
  f32x4 a, b;
};
template <int ES>
struct RawGroup<ES, false> {
  float x[8];
};

template <int ES, bool VEC>
__device__ __forceinline__ RawGroup<ES, VEC> load_raw(const char* __restrict__ row, int64_t e0) {
  RawGroup<ES, VEC> r;
  if constexpr (!VEC) {
    load_group<ES, false>(row, e0, r.x);
  } else if constexpr (ES == 2) {
    r.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + e0 * 2));
  } else {
    r.a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + e0 * 4));
    r.b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + e0 * 4 + 16));
  }
  return r;
}

template <int ES, bool VEC>
__device__ __forceinline__ void unpack_group(const RawGroup<ES, VEC>& r, float x[8]) {
  if constexpr (!VEC) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = r.x[i];
  } else if constexpr (ES == 2) {
    const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
    x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
  }
}

// An empty register-to-register step the compiler cannot see through: a
// group widened twice from its loaded registers stays loaded-size in between
// (the compiler would otherwise keep the first widening alive).
template <int ES, bool VEC>
__device__ __forceinline__ void opaque_group(RawGroup<ES, VEC>& r) {
  if constexpr (VEC && ES == 2) {
    asm volatile("" : "+v"(r.v));
  } else if constexpr (VEC) {
    asm volatile("" : "+v"(r.a), "+v"(r.b));
  }
}

// A group whose 8 logits are all -inf (padding past a row end).
template <int ES, bool VEC>
__device__ __forceinline__ RawGroup<ES, VEC> neg_inf_group() {
  RawGroup<ES, VEC> r;
  if constexpr (!VEC) {
#pragma unroll
    for (int i = 0; i < 8; ++i) r.x[i] = -INFINITY;
  } else if constexpr (ES == 2) {
    const uint32_t ni = 0xff80ff80u;  // two bf16 -inf
    r.v = u32x4{ni, ni, ni, ni};
  } else {
    r.a = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    r.b = r.a;
  }
  return r;
}

// One logit as stored (bf16 bits zero-extended, or fp32 bits), and its value.
template <int ES>
__device__ __forceinline__ uint32_t load_bits(const char* __restrict__ row, int64_t e) {
  if constexpr (ES == 2)
    return (uint32_t)reinterpret_cast<const uint16_t*>(row)[e];
  else
    return reinterpret_cast<const uint32_t*>(row)[e];
}

template <int ES>
__device__ __forceinline__ float bits_to_logit(uint32_t w) {
  return __uint_as_float(ES == 2 ? w << 16 : w);
}

template <int ES>
__device__ __forceinline__ float load_one(const char* __restrict__ row, int64_t e) {
  if constexpr (ES == 2)
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[e] << 16);
  else
    return reinterpret_cast<const float*>(row)[e];
}

// ------------------------------------------------------ scaled exponentials --
// Logits enter as t = x * s - M with s = log2(e) / T split into s_hi (fp32,
// rounded toward zero) + s_lo (>= FLT_MIN, so -inf logits stay -inf and give 0)
// and M = ceil(max * s_hi) an integer-valued reference, so t <= 0 for the row
// maximum up to the product's rounding and the s_lo term (t < 2 while
// |M| <= 2^24, the range a sampled row must stay in).
// The large terms cancel first: x * s_hi - M is exact before its one rounding,
// which is relative to the small result t, and the correction x * s_lo is
// added to that.  (Adding x * s_lo to -M first would round at the ulp of M,
// an error in t that grows with |logit| / T.)
__device__ __forceinline__ float scaled_exp2(float x, float s_hi, float s_lo, float negM) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(x, s_lo, __builtin_fmaf(x, s_hi, negM)));
}

// log2(e) / T split as s_hi + s_lo with s_hi rounded toward zero and
// s_lo >= FLT_MIN (keeps -inf * s = -inf in both fma terms).
__device__ __forceinline__ void temperature_scale(float T, float& s_hi, float& s_lo) {
  const double s = 1.4426950408889634074 / (double)T;
  s_hi = __double2float_rz(s);
  s_lo = fmaxf(__double2float_rn(s - (double)s_hi), FLT_MIN);
}

// A usable temperature: 0 (greedy) or a positive finite normal fp32 value
// (for subnormal T, log2(e) / T nears the top of the fp32 range and, below
// about 4.2e-39, leaves it).
__device__ __forceinline__ bool temperature_valid(float T) { return T == 0.0f || (T >= FLT_MIN && T <= FLT_MAX); }

// Largest |reference| a sampled row may have: ceil(max * s_hi) must be an
// exact fp32 integer for the scaled exponents near the maximum to be exact.
constexpr float kMaxRef = 0x1p24f;

// Sum of 2^(x * s - M) over a group of 8, pairwise in fp32.
__device__ __forceinline__ float sum8_exp(const float x[8], float s_hi, float s_lo, float negM) {
  float e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = scaled_exp2(x[i], s_hi, s_lo, negM);
  return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
}

// ---------------------------------------------------------- reductions --
// (M, S) pairs stand for S * 2^M with M integer-valued; merging is exact in
// the exponent (ldexp) and rounds only in the double add.
struct MS {
  float m;
  double s;
};

__device__ __forceinline__ MS ms_merge(MS a, MS b) {
  const float m = fmaxf(a.m, b.m);
  MS r;
  r.m = m;
  const int da = a.m < m ? (int)fmaxf(a.m - m, -2000.f) : 0;
  const int db = b.m < m ? (int)fmaxf(b.m - m, -2000.f) : 0;
  r.s = ldexp(a.s, da) + ldexp(b.s, db);
  return r;
}


// ----------------------------------------------- DPP lane movement (wave64) --
// Cross-lane moves through the VALU's data-parallel-primitive path instead of
// the LDS permute unit: a few cycles each rather than an LDS round trip.
// Controls (gfx9 encoding): row_shr:n = 0x110 + n within each 16-lane row,
// row_bcast:15 = 0x142 (lane 15 of a row to the whole next row) and
// row_bcast:31 = 0x143 (lane 31 to rows 2 and 3).  A lane whose source is
// outside its row, or whose row is not in ROW_MASK, receives `fill`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int x, int fill) {
  return __builtin_amdgcn_update_dpp(fill, x, CTRL, ROW_MASK, 0xf, false);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_d0(double x) {  // fill 0.0
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)dpp_i<CTRL, ROW_MASK>((int)(uint32_t)b, 0);
  const uint32_t hi = (uint32_t)dpp_i<CTRL, ROW_MASK>((int)(uint32_t)(b >> 32), 0);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive prefix sum over the 64 lanes in a fixed order: within 16-lane
// rows by doubling shifts, then the row totals carried across rows.
__device__ __forceinline__ double wave_scan_d(double x) {
  x += dpp_d0<0x111, 0xf>(x);
  x += dpp_d0<0x112, 0xf>(x);
  x += dpp_d0<0x114, 0xf>(x);
  x += dpp_d0<0x118, 0xf>(x);
  x += dpp_d0<0x142, 0xa>(x);
  x += dpp_d0<0x143, 0xc>(x);
  return x;
}

// The value of lane l (l the same in every lane).
__device__ __forceinline__ int lane_i(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

__device__ __forceinline__ float lane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

__device__ __forceinline__ double lane_d(double x, int l) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Maximum over the 64 lanes, the same in every lane.
__device__ __forceinline__ float wave_max_f(float x) {
  const int ninf = __float_as_int(-INFINITY);
  x = fmaxf(x, __int_as_float(dpp_i<0x111, 0xf>(__float_as_int(x), ninf)));
  x = fmaxf(x, __int_as_float(dpp_i<0x112, 0xf>(__float_as_int(x), ninf)));
  x = fmaxf(x, __int_as_float(dpp_i<0x114, 0xf>(__float_as_int(x), ninf)));
  x = fmaxf(x, __int_as_float(dpp_i<0x118, 0xf>(__float_as_int(x), ninf)));
  x = fmaxf(x, __int_as_float(dpp_i<0x142, 0xa>(__float_as_int(x), ninf)));
  x = fmaxf(x, __int_as_float(dpp_i<0x143, 0xc>(__float_as_int(x), ninf)));
  return lane_f(x, 63);
}

// The value of lane l - 1 in lane l (the whole wave shifted by one lane,
// wave_shr:1 = 0x138), 0 in lane 0: with an inclusive scan, the exclusive one.
__device__ __forceinline__ double wave_shr1_d(double x) { return dpp_d0<0x138, 0xf>(x); }

// Maximum over the 64 lanes, the same in every lane.
__device__ __forceinline__ int wave_max_i(int x) {
  x = max(x, dpp_i<0x111, 0xf>(x, INT_MIN));
  x = max(x, dpp_i<0x112, 0xf>(x, INT_MIN));
  x = max(x, dpp_i<0x114, 0xf>(x, INT_MIN));
  x = max(x, dpp_i<0x118, 0xf>(x, INT_MIN));
  x = max(x, dpp_i<0x142, 0xa>(x, INT_MIN));
  x = max(x, dpp_i<0x143, 0xc>(x, INT_MIN));
  return lane_i(x, 63);
}

// Sum over the 64 lanes in a fixed order (the last lane of the inclusive
// scan), the same in every lane.
__device__ __forceinline__ double wave_total_d(double x) { return lane_d(wave_scan_d(x), 63); }

// The (M, S) merge of the 64 lanes through DPP: prefix merges across the rows
// (empty lanes enter as (-inf, 0)), lane 63's read out; every lane ends with
// the same value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ MS dpp_ms(MS v) {
  MS o;
  o.m = __int_as_float(dpp_i<CTRL, ROW_MASK>(__float_as_int(v.m), __float_as_int(-INFINITY)));
  o.s = dpp_d0<CTRL, ROW_MASK>(v.s);
  return o;
}

__device__ __forceinline__ MS wave_merge_ms(MS v) {
  v = ms_merge(v, dpp_ms<0x111, 0xf>(v));
  v = ms_merge(v, dpp_ms<0x112, 0xf>(v));
  v = ms_merge(v, dpp_ms<0x114, 0xf>(v));
  v = ms_merge(v, dpp_ms<0x118, 0xf>(v));
  v = ms_merge(v, dpp_ms<0x142, 0xa>(v));
  v = ms_merge(v, dpp_ms<0x143, 0xc>(v));
  return MS{lane_f(v.m, 63), lane_d(v.s, 63)};
}


// (value, index) with larger value first, lower index on ties.
struct VI {
  float v;
  int i;
};

__device__ __forceinline__ VI vi_pick(VI a, VI b) {
  const bool take_b = (b.v > a.v) || (b.v == a.v && b.i < a.i);
  return take_b ? b : a;
}

// The greedy argmax counts a NaN logit as -inf.  vi_pick never takes a NaN,
// so a lane's scan over elements e0, e0 + 1, ... ends above -inf exactly when
// the NaN-as--inf maximum is above -inf, and it then holds the right element;
// otherwise every element it saw ties at -inf and the lowest, e0, wins.
// Applied once per lane after its scan, so padding lanes and indices past
// the row never come out of a merge.
__device__ __forceinline__ VI vi_floor(VI v, int e0) { return v.v > -INFINITY ? v : VI{-INFINITY, e0}; }

// The lowest-index argmax of the 64 lanes through DPP: prefix picks across the
// rows, lane 63's read out; every lane ends with the same value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ VI dpp_vi(VI v) {
  VI o;
  o.v = __int_as_float(dpp_i<CTRL, ROW_MASK>(__float_as_int(v.v), __float_as_int(-INFINITY)));
  o.i = dpp_i<CTRL, ROW_MASK>(v.i, INT_MAX);
  return o;
}

__device__ __forceinline__ VI wave_argmax(VI v) {
  v = vi_pick(v, dpp_vi<0x111, 0xf>(v));
  v = vi_pick(v, dpp_vi<0x112, 0xf>(v));
  v = vi_pick(v, dpp_vi<0x114, 0xf>(v));
  v = vi_pick(v, dpp_vi<0x118, 0xf>(v));
  v = vi_pick(v, dpp_vi<0x142, 0xa>(v));
  v = vi_pick(v, dpp_vi<0x143, 0xc>(v));
  return VI{lane_f(v.v, 63), lane_i(v.i, 63)};
}


}  // namespace specv
