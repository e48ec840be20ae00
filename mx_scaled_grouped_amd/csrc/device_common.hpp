// Device helpers shared by the quantization and GEMM kernels (gfx950 only).
//
// FP8 here is OCP e4m3 / e5m2, the formats the float8 MoE pages name
// (e4m3 in the Megatron-LM single-grouped-weight PR's coverage table, hybrid
// e4m3 / e5m2 in the Megatron-LM FP8-vs-BF16 bug report). On gfx950 the
// v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 instructions convert to the OCP
// formats with round-to-nearest-even; saturation is made explicit by
// clamping to +-fmax first (for finite inputs, RNE of the clamped value
// equals the saturating RNE of the value).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxsg {

enum Recipe : int { kTensorwise = 0, kDelayed = 1, kBlockwise = 2, kMx = 3, kNvfp4 = 4, kTile128 = 5 };
enum Format : int { kE4M3 = 0, kE5M2 = 1, kE2M1 = 2 };
enum Mode : int { kFwd = 0, kDgrad = 1, kWgrad = 2 };

// fmax = F * 2^emax; sig_man = the fp32 mantissa field of F (the MX
// exponent rounds up when amax's significand exceeds F)
template <int FMT> struct Fp8;
template <> struct Fp8<kE4M3> {
  static constexpr float fmax = 448.0f;
  static constexpr int emax = 8;  // 448 = 1.75 * 2^8
  static constexpr uint32_t sig_man = 0x600000u;
};
template <> struct Fp8<kE5M2> {
  static constexpr float fmax = 57344.0f;
  static constexpr int emax = 15;  // 57344 = 1.75 * 2^15
  static constexpr uint32_t sig_man = 0x600000u;
};
// OCP MX e2m1 (MXFP4 element): magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6
template <> struct Fp8<kE2M1> {
  static constexpr float fmax = 6.0f;
  static constexpr int emax = 2;  // 6 = 1.5 * 2^2
  static constexpr uint32_t sig_man = 0x400000u;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// |bf16| bit magnitudes of the two halves; for non-negative floats the order
// of the bit patterns is the order of the values, so max is exact.
__device__ __forceinline__ uint32_t absmax_bits2(uint32_t w, uint32_t m) {
  uint32_t lo = w & 0x7fffu, hi = (w >> 16) & 0x7fffu;
  m = lo > m ? lo : m;
  return hi > m ? hi : m;
}

__device__ __forceinline__ uint32_t absmax_bits8(uint4 v, uint32_t m) {
  m = absmax_bits2(v.x, m);
  m = absmax_bits2(v.y, m);
  m = absmax_bits2(v.z, m);
  return absmax_bits2(v.w, m);
}

// amax as float from a bf16 magnitude (exact)
__device__ __forceinline__ float bits_to_amax(uint32_t m) { return __uint_as_float(m << 16); }

// Four floats -> four FP8 codes in one dword (byte i = code of the i-th value).
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  constexpr float m = Fp8<FMT>::fmax;
  a = __builtin_fminf(__builtin_fmaxf(a, -m), m);
  b = __builtin_fminf(__builtin_fmaxf(b, -m), m);
  c = __builtin_fminf(__builtin_fmaxf(c, -m), m);
  d = __builtin_fminf(__builtin_fmaxf(d, -m), m);
  int r;
  if constexpr (FMT == kE4M3) {
    r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  } else {
    r = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, r, true);
  }
  return (uint32_t)r;
}

// 8 bf16 (one 16-byte vector) times inv -> 8 codes
template <int FMT>
__device__ __forceinline__ uint2 cvt8(uint4 v, float inv) {
  uint2 r;
  r.x = cvt4<FMT>(bf16_lo(v.x) * inv, bf16_hi(v.x) * inv, bf16_lo(v.y) * inv, bf16_hi(v.y) * inv);
  r.y = cvt4<FMT>(bf16_lo(v.z) * inv, bf16_hi(v.z) * inv, bf16_lo(v.w) * inv, bf16_hi(v.w) * inv);
  return r;
}

// Two floats -> two e2m1 codes (4 bits each, sign in bit 3; `a` in the low
// nibble) written into byte SEL of `old`: saturating round to nearest even,
// by v_cvt_scalef32_pk_fp4_f32 with scale 1.0 (the multiplier is applied
// before, in fp32). Measured on the device against a comparison-based
// encoder over all 2^32 non-NaN fp32 inputs: identical, including the ties
// to the even code, the saturation to 6 and the sign of zero results.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pk(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// 8 bf16 (one 16-byte vector) times inv -> 8 e2m1 codes, element i in
// nibble i (element 2j in the low nibble of byte j)
__device__ __forceinline__ uint32_t cvt8_e2m1(uint4 v, float inv) {
  uint32_t r = 0;
  r = e2m1_pk<0>(r, bf16_lo(v.x) * inv, bf16_hi(v.x) * inv);
  r = e2m1_pk<1>(r, bf16_lo(v.y) * inv, bf16_hi(v.y) * inv);
  r = e2m1_pk<2>(r, bf16_lo(v.z) * inv, bf16_hi(v.z) * inv);
  r = e2m1_pk<3>(r, bf16_lo(v.w) * inv, bf16_hi(v.w) * inv);
  return r;
}

// fp32 scale pair of a unit: s = amax / fmax, inv = fmax / amax (IEEE
// correctly rounded divisions); amax == 0 gives (1, 1).
template <int FMT>
__device__ __forceinline__ void scale_pair(float amax, float &s, float &inv) {
  if (amax > 0.0f) {
    s = __fdiv_rn(amax, Fp8<FMT>::fmax);
    inv = __fdiv_rn(Fp8<FMT>::fmax, amax);
  } else {
    s = 1.0f;
    inv = 1.0f;
  }
}

// MX shared exponent: the smallest k with amax <= fmax * 2^k, clamped to
// [-127, 127], from the bits of amax = f * 2^E (1 <= f < 2):
// k = E - emax + (f > F), because fmax = F * 2^emax (F = 1.75 for e4m3 and
// e5m2, 1.5 for e2m1).
template <int FMT>
__device__ __forceinline__ int mx_exponent(float amax) {
  uint32_t u = __float_as_uint(amax) & 0x7fffffffu;
  if (u == 0) return 0;
  int eb = (int)(u >> 23);
  uint32_t man = u & 0x7fffffu;
  int E;
  if (eb == 0) {  // subnormal amax: normalize the mantissa
    int top = 31 - __clz(man);
    E = top - 149;
    man = (man << (23 - top)) & 0x7fffffu;
  } else {
    E = eb - 127;
  }
  int k = E - Fp8<FMT>::emax + (man > Fp8<FMT>::sig_man ? 1 : 0);
  return k < -127 ? -127 : (k > 127 ? 127 : k);
}

// 2^-k as float (exact for k in [-127, 127]; 2^-127 is subnormal)
__device__ __forceinline__ float exp2_neg(int k) {
  int e = 127 - k;
  if (e >= 1) return __uint_as_float((uint32_t)e << 23);
  return __uint_as_float(1u << (22 + e));  // e == 0: 2^-127
}

// NVFP4 (e2m1 elements; an e4m3 scale per 16 elements along the contraction
// dim; an fp32 scale per tensor unit). Tensor decode scale s_t = fp32(amax /
// 2688) (6 * 448, the e2m1 maximum times the e4m3 maximum), 1 for amax == 0.
constexpr float kNvTensorDen = 2688.0f;
__device__ __forceinline__ float nv_tensor_scale(float amax) {
  return amax > 0.0f ? __fdiv_rn(amax, kNvTensorDen) : 1.0f;
}

// A 16-element block's e4m3 scale code and the element multiplier:
// t = fp32(fp32(amax / 6) / s_t), code = saturating RNE e4m3 of t,
// M = fp32(value(code) * s_t), inv = fp32(1 / M) (0 when M == 0 or 1 / M
// overflows), each an IEEE fp32 operation.
__device__ __forceinline__ uint32_t nv_block_scale(float amax, float s_t, float &inv) {
  const float t = __fdiv_rn(__fdiv_rn(amax, 6.0f), s_t);
  const float tc = __builtin_fminf(t, 448.0f);                  // t >= 0; saturate
  const uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(tc, tc, 0, false) & 0xFFu;
  const float d = __builtin_amdgcn_cvt_f32_fp8((int)code, 0);   // exact decode
  const float m = d * s_t;
  const float r = __fdiv_rn(1.0f, m);
  inv = (m > 0.0f && r < __builtin_inff()) ? r : 0.0f;
  return code;
}

// NVFP4 code order inside each 128-element (64-byte) piece of a row: the 8
// elements 16 s + 8 h .. 16 s + 8 h + 7 (k16 step s, half h) form the dword
// at byte 32 (s / 4) + 16 h + 4 (s % 4), so that the 16-byte chunks h and
// 2 + h of a piece hold, for MFMA lane half h, its 8 k-values of each of the
// piece's 8 steps (measured operand layout of the 32x32x16 f16 MFMA: lane
// half h holds k in [8h, 8h + 8) of a step).
__device__ __forceinline__ int nv_dword_off(int s, int h) { return ((s & 4) << 3) + 16 * h + 4 * (s & 3); }

// wave-wide max of a uint (64 lanes)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t t = (uint32_t)__shfl_xor((int)v, o, 64);
    v = t > v ? t : v;
  }
  return v;
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// bf16 bits of a float, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Clamped group bounds: rows [lo, hi) of group g from int32 cumulative ends.
__device__ __forceinline__ void group_bounds(const int32_t *__restrict__ ends, int g, int64_t M,
                                             int64_t &lo, int64_t &hi) {
  int64_t a = g > 0 ? (int64_t)ends[g - 1] : 0;
  int64_t b = (int64_t)ends[g];
  a = a < 0 ? 0 : (a > M ? M : a);
  b = b < 0 ? 0 : (b > M ? M : b);
  lo = a;
  hi = b < a ? a : b;
}

// Max-reduce a non-negative fp32 bit pattern into *p (bit order = value
// order for non-negative floats). The atomic is skipped when the stored value
// is already at least as large, so a tensor's tiles mostly stop contending for
// one word once its maximum is in; a stale read only costs an extra atomic.
__device__ __forceinline__ void atomic_max_bits(uint32_t *p, uint32_t v) {
  if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < v) atomicMax(p, v);
}

// Byte offset of code (r, l) in a pair-interleaved code matrix with rows of
// L bytes (L a multiple of 64): rows 2p and 2p+1 share 2L bytes, as lines of
// 128 bytes that each hold 64 bytes of row 2p followed by the same 64 bytes
// of row 2p+1. A GEMM stage of 64 contraction bytes over an even run of rows
// is then whole 128-byte lines.
// Streaming (nontemporal) 16- and 8-byte global accesses: data read or
// written exactly once by a pass that moves far more bytes than the caches
// hold bypasses them instead of evicting what other passes reuse.
typedef unsigned int nt_v4u __attribute__((ext_vector_type(4)));
typedef unsigned int nt_v2u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load16_stream(const void *p) {
  const nt_v4u v = __builtin_nontemporal_load(reinterpret_cast<const nt_v4u *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store16_stream(void *p, uint4 v) {
  const nt_v4u w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<nt_v4u *>(p));
}
__device__ __forceinline__ void store8_stream(void *p, uint2 v) {
  const nt_v2u w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<nt_v2u *>(p));
}

__device__ __forceinline__ int64_t pi_off(int64_t r, int64_t l, int64_t L) {
  return (r >> 1) * (2 * L) + ((l >> 6) << 7) + ((r & 1) << 6) + (l & 63);
}

}  // namespace mxsg
