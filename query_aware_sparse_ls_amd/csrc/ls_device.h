// Device helpers shared by the libls kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ls {

constexpr int kWave = 64;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16 ----

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// a and b rounded to bf16 (nearest even) and packed (a in the low half): one
// gfx950 v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// One step of splitting two floats into bf16 parts: *part = their bf16
// roundings (packed), and a, b become what is left (a - bf16(a), ...).
__device__ __forceinline__ void bf16x2_split(float& a, float& b, uint32_t* part) {
  const uint32_t h = pack_bf16x2(a, b);
  *part = h;
  a -= bf16_lo(h);
  b -= bf16_hi(h);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (NaN -> quiet NaN).
// 2^x by the hardware exponential (v_exp_f32, about 1 ulp; 2^-inf = 0):
// softmax weights of arguments <= 0, where the library exp2f's extra range
// handling is not needed.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp64 -> bf16 with ONE round-to-nearest-even step. First round to fp32 by
// round-to-odd (truncate, then force the last bit to 1 if anything was cut
// off), then RNE to bf16: rounding to odd at >= p+2 bits and then to nearest
// at p bits equals a single rounding to nearest at p bits (Boldo & Melquiond,
// "Emulation of FMA and correctly rounded sums: proved algorithms using
// rounding to odd", IEEE TC 2008). fp32 keeps 24 >= 8+2 bits, also in the
// subnormal range, where fp32's quantum is 2^16 times finer than bf16's.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  float f = (float)x;                             // nearest-even
  if (!(fabs(x) <= 3.4028234663852886e38)) {      // inf / NaN / beyond FLT_MAX
    if (x != x) return 0x7fc0u;
    // |x| > FLT_MAX: truncation gives FLT_MAX, round-to-odd keeps it odd.
    uint32_t u = 0x7f7fffffu | (x < 0 ? 0x80000000u : 0u);
    if (__builtin_isinf(x)) u = x < 0 ? 0xff800000u : 0x7f800000u;
    return f32_to_bf16_rne(__uint_as_float(u));
  }
  double back = (double)f;
  uint32_t u = __float_as_uint(f);
  if (back != x) {
    // truncate toward zero: if rounding went away from zero, step back one ulp
    if (fabs(back) > fabs(x)) u -= 1u;             // magnitude bits decrement
    u |= 1u;                                        // sticky -> odd
  }
  return f32_to_bf16_rne(__uint_as_float(u));
}

// OCP fp8 e4m3fn -> fp32, exact (1 sign, 4 exponent bits bias 7, 3 mantissa
// bits, exponent field 0 subnormal, S.1111.111 NaN, no infinity).
__device__ __forceinline__ float fp8e4m3fn_to_f32(uint32_t b) {
  uint32_t e = (b >> 3) & 0xfu, m = b & 7u;
  float mag;
  if (e == 0) {
    mag = (float)m * 0.001953125f;                         // m * 2^-9
  } else {
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20)); // (1 + m/8) 2^(e-7)
  }
  if (e == 15 && m == 7) mag = __uint_as_float(0x7fc00000u);
  return (b & 0x80u) ? -mag : mag;
}

// bf16 pair of fp8 e4m3fn bytes 0,1 (hi = false) or 2,3 (hi = true) of x,
// exact (every e4m3fn value is a bf16 value): the gfx950 packed convert.
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t x, bool hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true)
                        : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------- reductions ----

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v |= __shfl_xor(v, o, kWave);
  return v;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int n = __shfl_up(v, o, kWave);
    if (lane >= o) v += n;
  }
  return v;
}

// ------------------------------------------------------------------ DPP ----
// Sum over aligned groups of LPR lanes (LPR = 4, 8 or 16: DPP works inside
// 16-lane rows), every lane of the group receiving the total: two quad
// swaps, then the half-row mirror (pairs quads inside 8 lanes), then the row
// mirror (pairs the 8-lane halves of a row).
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(LPR == 4 || LPR == 8 || LPR == 16, "group size");
  v += dpp_mov<kDppXor1>(v);
  v += dpp_mov<kDppXor2>(v);
  if constexpr (LPR >= 8) v += dpp_mov<kDppRowHalfMirror>(v);
  if constexpr (LPR >= 16) v += dpp_mov<kDppRowMirror>(v);
  return v;
}

// ------------------------------------------------- lane-pair exchanges ----
// The values of this lane and of lane ^ O (O = 8, 16 or 32), returned in lane
// order: lo = value of the lane whose bit O is clear, hi = the other. Both
// lanes of a pair get the same (lo, hi), so a pair combined as f(lo, hi) is
// identical in both lanes. VALU only: DPP row_ror:8 inside 16-lane rows, and
// gfx950's v_permlane16_swap / v_permlane32_swap across rows (no LDS path).
template <int O>
__device__ __forceinline__ void xor_pair(float v, float& lo, float& hi) {
  static_assert(O == 8 || O == 16 || O == 32, "lane distance");
  const unsigned u = __float_as_uint(v);
  if constexpr (O == 8) {
    const float w = __uint_as_float(__builtin_amdgcn_update_dpp(0u, u, 0x128, 0xf, 0xf, false));
    const bool upper = (__lane_id() & 8) != 0;
    lo = upper ? w : v;
    hi = upper ? v : w;
  } else if constexpr (O == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
  }
}

// Sum of the value over lanes l and l ^ O, identical in both lanes.
template <int O>
__device__ __forceinline__ float xor_pair_sum(float v) {
  float lo, hi;
  xor_pair<O>(v, lo, hi);
  return lo + hi;
}

// ---------------------------------------------- low-latency wave reductions
// Float min / max over the 64 lanes: DPP inside each 16-lane row, then the
// four row results read into scalars (no LDS-crossbar permutes).
__device__ __forceinline__ float rl_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ float wave_max_fast(float v) {
  v = fmaxf(v, dpp_mov<kDppXor1>(v));
  v = fmaxf(v, dpp_mov<kDppXor2>(v));
  v = fmaxf(v, dpp_mov<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_mov<kDppRowMirror>(v));
  return fmaxf(fmaxf(rl_f(v, 0), rl_f(v, 16)), fmaxf(rl_f(v, 32), rl_f(v, 48)));
}
__device__ __forceinline__ float wave_min_fast(float v) {
  v = fminf(v, dpp_mov<kDppXor1>(v));
  v = fminf(v, dpp_mov<kDppXor2>(v));
  v = fminf(v, dpp_mov<kDppRowHalfMirror>(v));
  v = fminf(v, dpp_mov<kDppRowMirror>(v));
  return fminf(fminf(rl_f(v, 0), rl_f(v, 16)), fminf(rl_f(v, 32), rl_f(v, 48)));
}

// Index of this thread's wave in the workgroup, known uniform to the compiler.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Number of set bits of the wave mask m in lanes below this one.
__device__ __forceinline__ int mbcnt(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0));
}
// Exclusive prefix sum and total of small non-negative ints (< 2^BITS) over
// the wave, by bit planes: one ballot and one masked count per bit.
template <int BITS>
__device__ __forceinline__ int wave_excl_scan_small(int v, int* total) {
  int pre = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b) {
    const unsigned long long m = __ballot((v >> b) & 1);
    pre += mbcnt(m) << b;
    tot += __popcll(m) << b;
  }
  *total = tot;
  return pre;
}

// Order LDS traffic of one wavefront: every LDS access issued before this
// point has completed before any issued after it (wave-synchronous code).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ int wave_excl_scan(int v, int lane) {
  return wave_incl_scan(v, lane) - v;
}

// Order-preserving map of a (finite) float to uint32; -0.0 is mapped like +0.0
// so that equal scores compare equal.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------ device-coherent access ----
// Data handed from one workgroup to another inside a kernel (scores,
// selections, split partials) is written and read with agent-scope
// (device-coherent) accesses, which bypass the per-XCD L2 instead of
// requiring whole-cache write-back / invalidate fences.
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Plain or device-coherent, chosen at compile time: kernels that hand data to
// other workgroups of the SAME launch use the coherent form; kernels whose
// consumer is a later launch use plain (cached) accesses.
template <bool kDev, typename T>
__device__ __forceinline__ void st_x(T* p, T v) {
  if constexpr (kDev) st_dev(p, v); else *p = v;
}
template <bool kDev, typename T>
__device__ __forceinline__ T ld_x(const T* p) {
  if constexpr (kDev) return ld_dev(p); else return *p;
}

// Wait until every store this wave issued has completed (vmcnt(0)), and keep
// the compiler from moving memory operations across the wait.
__device__ __forceinline__ void wait_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0), expcnt/lgkmcnt untouched
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// 16-byte global load through the vector memory path.
__device__ __forceinline__ uint4 ldg16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// 16-byte streaming load: data read once (key/value tiles, summary rows),
// marked non-temporal so it does not displace reused lines in the caches.
__device__ __forceinline__ uint4 ldg16_stream(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

}  // namespace ls
