// lq_device.h — device-side pieces of liblq for gfx950 (CDNA4, wave64).
//
// Number formats, scale rules and the per-tile element pipeline shared by the
// fake-quant, quantize and dequantize kernels. One lane owns a tile of 16
// consecutive elements of a row (two or four 16-byte loads); a block of B
// elements is B/16 neighbouring lanes, whose statistic is combined with DPP
// lane permutations (no LDS round trip).
//
// Sources (web pages, by address and section): affine map and INT ranges,
// guijiagi.com/posts/quantization-int4-int8-fp8 "INT8量化"/"INT4量化"; AbsMax
// scale and symmetric INT8, MXINT8 blocks of 32 with UE8M0 scales,
// cyqw.cn/news/1000169 §2.1; FP value formula §2.2; element formats and ranges,
// walkerchi.com quantization playbook §4.1 table; NV blocks of 16 with E4M3
// scales §4.3.1; Hadamard rotation cyqw.cn §4.2/§7.2 and playbook §5.3; QSNR
// cyqw.cn §4.1.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lq.h"

namespace lqd {

constexpr int kTile = 16;          // elements per lane per tile
constexpr int kThreads = 256;      // threads per workgroup (4 waves)
#ifndef LQ_MAX_WG
#define LQ_MAX_WG 8192
#endif
constexpr int kMaxWG = LQ_MAX_WG;  // most workgroups of a launch whose partials k_finish sums
// Most workgroups of a launch that finishes its QSNR sum itself (the
// lane-contiguous one-pass grids: C4's 134M elements are 32768 workgroups of
// 4 waves, one 1024-element chunk per wave).
#ifndef LQ_MAX_WG_INLINE
#define LQ_MAX_WG_INLINE 32768
#endif
constexpr int kMaxWGInline = LQ_MAX_WG_INLINE;
static_assert(kMaxWG <= kMaxWGInline, "grids capped at kMaxWG also finish their QSNR in-kernel");
// Records one collecting workgroup sums (two per thread of 256, so one round
// of loads: the collection is a chain of memory round trips at the end of
// every call), and the group records of the most collectors a grid can have.
constexpr int kGroupRecords = 512;
constexpr int kMaxGroups = (kMaxWGInline + kGroupRecords - 1) / kGroupRecords;
// Most partials the per-tensor statistic leaves (its grid is capped at this
// many workgroups); every workgroup of the per-tensor k_flat combines them.
constexpr int kStatParts = 512;

// ---------------------------------------------------------------- workspace
// Per-workgroup partial results of a reducing launch, combined by a
// one-workgroup finishing kernel that runs after it on the same stream. The
// kernel boundary orders the two, so the streaming kernels need no fences or
// atomics: a release fence writes back every dirty line of the XCD's L2
// (buffer_wbl2) and serialises a streaming kernel, and a last-workgroup
// handshake keeps every workgroup waiting on a memory round trip before it
// can exit.
//
// The specialised kernels (and k_flat) finish the sum themselves instead:
// every workgroup publishes its partials as five 64-bit words, each carrying
// the call's epoch in its high half (err low/high, sig low/high, non-finite
// count), written with agent-scope atomic stores that need no fence and no
// read-modify-write. The grid's last K = ceil(N / kGroupRecords) workgroups
// collect: collector j polls records j*kGroupRecords .. (j+1)*kGroupRecords-1
// until every tag shows the current epoch, sums them and publishes a group
// record the same way; the last workgroup also sums the K group records and
// writes the result (the wide one-pass lane-contiguous grids instead launch
// one workgroup more that only collects). A 64-bit atomic store is seen
// whole, so a word with the right tag holds this call's payload half.
constexpr int kTagWords = 5;
struct Workspace {
  double part_err[kMaxWG];
  double part_sig[kMaxWG];
  uint32_t part_bad[kMaxWG];
  float part_amax[kStatParts];         // statistic pass: max|x|, min x, max x
  float part_min[kStatParts];
  float part_max[kStatParts];
  uint64_t tagged[kMaxWGInline][kTagWords];   // one record per workgroup
  uint64_t group[kMaxGroups][kTagWords];      // one record per collector
};

// ---------------------------------------------------------------- formats
template <int F> struct Fmt;
constexpr int kFormats = 7;   // LQ_INT8 .. LQ_E3M2
// Qmax: INT8 127, INT4 7, E4M3 448, E5M2 57344, E2M1 6, E2M3 7.5, E3M2 28.
// qmant/qexp are the frexp() parts of Qmax (Qmax = qmant * 2^qexp, qmant in
// [0.5, 1)). four: two codes per byte; six: 6-bit codes (FP6, 12 bytes per
// 16 elements).
template <> struct Fmt<LQ_INT8> { static constexpr bool is_int = true;  static constexpr bool four = false; static constexpr bool six = false; static constexpr float qmax = 127.f;   static constexpr float qmant = 0.9921875f; static constexpr int qexp = 7; };
template <> struct Fmt<LQ_INT4> { static constexpr bool is_int = true;  static constexpr bool four = true;  static constexpr bool six = false; static constexpr float qmax = 7.f;     static constexpr float qmant = 0.875f;     static constexpr int qexp = 3; };
template <> struct Fmt<LQ_E4M3> { static constexpr bool is_int = false; static constexpr bool four = false; static constexpr bool six = false; static constexpr float qmax = 448.f;   static constexpr float qmant = 0.875f;     static constexpr int qexp = 9;
                                  static constexpr int E = 4, M = 3, BIAS = 7; };
template <> struct Fmt<LQ_E5M2> { static constexpr bool is_int = false; static constexpr bool four = false; static constexpr bool six = false; static constexpr float qmax = 57344.f; static constexpr float qmant = 0.875f;     static constexpr int qexp = 16;
                                  static constexpr int E = 5, M = 2, BIAS = 15; };
template <> struct Fmt<LQ_E2M1> { static constexpr bool is_int = false; static constexpr bool four = true;  static constexpr bool six = false; static constexpr float qmax = 6.f;     static constexpr float qmant = 0.75f;      static constexpr int qexp = 3;
                                  static constexpr int E = 2, M = 1, BIAS = 1; };
// FP6 (walkerchi.com playbook §4.1 table: E2M3 ±7.5 = 1.875 * 2^2, E3M2 ±28 =
// 1.75 * 2^4, every code a number)
template <> struct Fmt<LQ_E2M3> { static constexpr bool is_int = false; static constexpr bool four = false; static constexpr bool six = true;  static constexpr float qmax = 7.5f;    static constexpr float qmant = 0.9375f;    static constexpr int qexp = 3;
                                  static constexpr int E = 2, M = 3, BIAS = 1; };
template <> struct Fmt<LQ_E3M2> { static constexpr bool is_int = false; static constexpr bool four = false; static constexpr bool six = true;  static constexpr float qmax = 28.f;    static constexpr float qmant = 0.875f;     static constexpr int qexp = 5;
                                  static constexpr int E = 3, M = 2, BIAS = 3; };

// Native converters (v_cvt_pk_fp8_f32, v_cvt_pk_bf8_f32,
// v_cvt_scalef32_pk_fp4_f32 and their inverses) round to nearest even in the
// default mode; inputs are clamped to +-Qmax first so they never overflow. A
// build can switch any format to the bit-manipulation encoders below.
#ifndef LQ_NATIVE_E4M3
#define LQ_NATIVE_E4M3 1
#endif
#ifndef LQ_NATIVE_E5M2
#define LQ_NATIVE_E5M2 1
#endif
#ifndef LQ_NATIVE_E2M1
#define LQ_NATIVE_E2M1 1
#endif

__device__ __forceinline__ float clampf(float v, float lo, float hi) {
  return __builtin_amdgcn_fmed3f(v, lo, hi);
}

// Bit-manipulation encoder of a float format with E exponent bits, M
// mantissa bits and bias BIAS, for |v| <= its largest finite value: round to
// nearest even, gradual underflow, sign kept.
template <int E, int M, int BIAS>
__device__ __forceinline__ uint32_t alu_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 31) << (E + M);
  const float a = fabsf(v);
  // below the smallest normal the grid is uniform with step 2^(1-BIAS-M):
  // the code is the rounded multiple (scaling by a power of two is exact)
  const float sub_scale = __builtin_bit_cast(float, (uint32_t)(127 + BIAS - 1 + M) << 23);
  const uint32_t sub = (uint32_t)__builtin_rintf(a * sub_scale);
  // normal: round the binary32 significand to M bits (ties to even), rebias
  uint32_t ab = __float_as_uint(a);
  ab += (1u << (22 - M)) - 1u + ((ab >> (23 - M)) & 1u);
  const uint32_t nor = (ab >> (23 - M)) - ((uint32_t)(127 - BIAS) << M);
  const float min_normal = __builtin_bit_cast(float, (uint32_t)(127 + 1 - BIAS) << 23);
  return sign | (a < min_normal ? sub : nor);
}

// alu_encode together with the value its code stands for: the rounded
// significand (normal) or the rounded multiple of the subnormal step, with
// v's sign (so -0 for a negative value that rounds to zero), which is what
// alu_decode of the code gives, without decoding it.
template <int E, int M, int BIAS>
__device__ __forceinline__ uint32_t alu_encode_v(float v, float& val) {
  const uint32_t sgn = __float_as_uint(v) & 0x80000000u;
  const float a = fabsf(v);
  const float sub_scale = __builtin_bit_cast(float, (uint32_t)(127 + BIAS - 1 + M) << 23);
  const float sub_step = __builtin_bit_cast(float, (uint32_t)(127 + 1 - BIAS - M) << 23);
  const float subf = __builtin_rintf(a * sub_scale);
  uint32_t ab = __float_as_uint(a);
  ab += (1u << (22 - M)) - 1u + ((ab >> (23 - M)) & 1u);
  const uint32_t nor = (ab >> (23 - M)) - ((uint32_t)(127 - BIAS) << M);
  const float min_normal = __builtin_bit_cast(float, (uint32_t)(127 + 1 - BIAS) << 23);
  const bool is_sub = a < min_normal;
  const float mag = is_sub ? subf * sub_step : __uint_as_float(ab & ~((1u << (23 - M)) - 1u));
  val = __uint_as_float(__float_as_uint(mag) | sgn);
  return (sgn >> (31 - E - M)) | (is_sub ? (uint32_t)subf : nor);
}

// Value of a code of the same kind of format (finite codes only).
template <int E, int M, int BIAS>
__device__ __forceinline__ float alu_decode(uint32_t c) {
  const uint32_t s = (c >> (E + M)) & 1u;
  const uint32_t e = (c >> M) & ((1u << E) - 1u);
  const uint32_t m = c & ((1u << M) - 1u);
  const float sub = (float)m * __builtin_bit_cast(float, (uint32_t)(127 + 1 - BIAS - M) << 23);
  const float nor = __builtin_bit_cast(float, ((e + 127u - BIAS) << 23) | (m << (23 - M)));
  const float mag = e ? nor : sub;
  return s ? -mag : mag;
}

// ---- 8-bit FP: 4 codes per 32-bit word
template <int F>
__device__ __forceinline__ uint32_t fp8_pack4(float a, float b, float c, float d) {
  if constexpr ((F == LQ_E4M3 && LQ_NATIVE_E4M3) || (F == LQ_E5M2 && LQ_NATIVE_E5M2)) {
    int w;
    if constexpr (F == LQ_E4M3) {
      w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    } else {
      w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
      w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
    }
    return (uint32_t)w;
  } else {
    using T = Fmt<F>;
    return alu_encode<T::E, T::M, T::BIAS>(a) | (alu_encode<T::E, T::M, T::BIAS>(b) << 8) |
           (alu_encode<T::E, T::M, T::BIAS>(c) << 16) | (alu_encode<T::E, T::M, T::BIAS>(d) << 24);
  }
}

template <int F>
__device__ __forceinline__ void fp8_unpack4(uint32_t w, float out[4]) {
  if constexpr ((F == LQ_E4M3 && LQ_NATIVE_E4M3) || (F == LQ_E5M2 && LQ_NATIVE_E5M2)) {
    if constexpr (F == LQ_E4M3) {
      auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
      auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
      out[0] = lo[0]; out[1] = lo[1]; out[2] = hi[0]; out[3] = hi[1];
    } else {
      auto lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
      auto hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
      out[0] = lo[0]; out[1] = lo[1]; out[2] = hi[0]; out[3] = hi[1];
    }
  } else {
    using T = Fmt<F>;
#pragma unroll
    for (int i = 0; i < 4; i++) out[i] = alu_decode<T::E, T::M, T::BIAS>((w >> (8 * i)) & 0xFFu);
  }
}

// ---- E2M1: 8 codes per 32-bit word, element 2j in the low nibble of byte j
__device__ __forceinline__ uint32_t fp4_pack8(const float* v) {
#if LQ_NATIVE_E2M1
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
#else
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) w |= alu_encode<2, 1, 1>(v[i]) << (4 * i);
  return w;
#endif
}

__device__ __forceinline__ void fp4_unpack8(uint32_t w, float* out) {
#if LQ_NATIVE_E2M1
  auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  out[0] = p0[0]; out[1] = p0[1]; out[2] = p1[0]; out[3] = p1[1];
  out[4] = p2[0]; out[5] = p2[1]; out[6] = p3[0]; out[7] = p3[1];
#else
#pragma unroll
  for (int i = 0; i < 8; i++) out[i] = alu_decode<2, 1, 1>((w >> (4 * i)) & 0xFu);
#endif
}

// ---- FP6 (E2M3, E3M2): 6-bit codes, element i in bits 6i .. 6i+5.
// v_cvt_scalef32_2xpk16_{fp6,bf6}_f32 converts 32 binary32 values (two
// vectors of 16) to 32 codes in six dwords, taking the vectors' elements in
// turn (field 2k is the first vector's element k, field 2k+1 the second's);
// v_cvt_scalef32_pk32_f16_{fp6,bf6} gives the 32 values back, as fp16, in
// field order. With scale 1.0 both match the bit-level rule: round to
// nearest even, gradual underflow, a negative value that rounds to zero keeps
// its sign, and finite values beyond the largest code saturate to it (a
// structured sweep over every binary32 exponent, the rounding-relevant
// significands and the binary32 subnormals, both signs, against the CPU
// encoder: codes and values). A build can switch to the bit-manipulation
// encoder.
#ifndef LQ_NATIVE_FP6
#define LQ_NATIVE_FP6 1
#endif
typedef float lq_v16f __attribute__((ext_vector_type(16)));
typedef _Float16 lq_v32h __attribute__((ext_vector_type(32)));
typedef uint32_t lq_v6u __attribute__((ext_vector_type(6)));

template <int F>
__device__ __forceinline__ lq_v6u fp6_cvt32(lq_v16f even, lq_v16f odd) {
  if constexpr (F == LQ_E2M3) return __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(even, odd, 1.0f);
  else return __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(even, odd, 1.0f);
}
// The values of the 32 fields as fp16 (every FP6 value is exact in fp16, the
// sign of zero included), in field order.
template <int F>
__device__ __forceinline__ lq_v32h fp6_halves32(lq_v6u w) {
  if constexpr (F == LQ_E2M3) return __builtin_amdgcn_cvt_scalef32_pk32_f16_fp6(w, 1.0f);
  else return __builtin_amdgcn_cvt_scalef32_pk32_f16_bf6(w, 1.0f);
}

// The 16 codes of a tile's quotients v (96 bits in w0..w2) in one
// conversion; the vectors' upper halves feed fields 16..31 only, which are
// dropped, so they are left unspecified (no instructions).
template <int F>
__device__ __forceinline__ lq_v6u fp6_encode16(const float* v) {
  lq_v16f even = __builtin_nondeterministic_value(even), odd = __builtin_nondeterministic_value(odd);
#pragma unroll
  for (int k = 0; k < 8; k++) {
    even[k] = v[2 * k];
    odd[k] = v[2 * k + 1];
  }
  return fp6_cvt32<F>(even, odd);
}

// The values of 16 codes held in 96 bits (w0, w1, w2).
template <int F>
__device__ __forceinline__ void fp6_unpack16(uint32_t w0, uint32_t w1, uint32_t w2, float* d) {
  lq_v6u w = __builtin_nondeterministic_value(w);
  w[0] = w0;
  w[1] = w1;
  w[2] = w2;
  const lq_v32h h = fp6_halves32<F>(w);
#pragma unroll
  for (int i = 0; i < 16; i++) d[i] = (float)h[i];
}

// ---- scale storage formats
// fp16 (round to nearest even, saturating at 65504) and back
__device__ __forceinline__ uint32_t f16_bits_sat(float t) {
  _Float16 h = (_Float16)fminf(t, 65504.0f);
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_value(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
// E4M3 scale of a non-negative value (saturating at 448)
__device__ __forceinline__ uint32_t e4m3_scale_bits(float t) {
#if LQ_NATIVE_E4M3
  // byte 0 the code, byte 1 the code of +0 (0), bytes 2-3 the zero operand
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(t, 448.0f), 0.0f, 0, false);
#else
  return fp8_pack4<LQ_E4M3>(fminf(t, 448.0f), 0.f, 0.f, 0.f) & 0xFFu;
#endif
}
__device__ __forceinline__ float e4m3_scale_value(uint32_t c) {
  float o[4];
  fp8_unpack4<LQ_E4M3>(c, o);
  return o[0];
}

// ---------------------------------------------------------------- scales
// How an element is divided by the stored scale s.
enum : int { DIV_ZERO = 0, DIV_POW2 = 1, DIV_MARKSTEIN = 2, DIV_IEEE = 3 };

struct Scale {
  float s;        // stored scale as a binary32 value
  float r;        // 2^-e (DIV_POW2) or RN(1/s) (DIV_MARKSTEIN)
  float zp;       // zero point (asymmetric)
  uint32_t sbits; // stored scale bits
  uint32_t zbits; // stored zero-point bits
  int div;        // DIV_*
};

__device__ __forceinline__ void set_div(Scale& sc) {
  if (sc.s == 0.0f) {
    sc.div = DIV_ZERO;
    sc.r = 0.0f;
    return;
  }
  sc.r = 1.0f / sc.s;   // correctly rounded
  // Markstein's correction (q0 = x*r, rem = x - q0*s exactly, q = q0 + rem*r)
  // yields the correctly rounded quotient when r = RN(1/s) is finite. A scale
  // so small that 1/s overflows (below 2^-126) is DIV_IEEE: IEEE division, or
  // (scales computed from the data, |x| <= Qmax * s) the same correction on
  // x * 2^64 and s * 2^64, exact scalings that leave the quotient unchanged;
  // r then holds RN(1/(s * 2^64)).
  if (sc.r < __builtin_inff()) {
    sc.div = DIV_MARKSTEIN;
  } else {
    sc.div = DIV_IEEE;
    sc.r = 1.0f / (sc.s * 0x1p64f);
  }
}

// The divisions of a block scale stored as fp16 or E4M3, in a few VALU
// operations each and with the results of IEEE division:
//  - t = amax / Qmax by Markstein's correction around the constant
//    RN(1/Qmax). For each format's Qmax and every non-negative finite binary32
//    amax it equals the IEEE quotient wherever that is at least 2^-125; below
//    that both round to a zero fp16 or E4M3 scale. amax = +inf gives NaN
//    instead of +inf, and the saturating conversions take both to their
//    largest value.
//  - r = RN(1/s) by one Newton step from v_rcp_f32. For every positive fp16
//    and E4M3 value s, any start within 4 ulp of 1/s ends on RN(1/s) (an
//    exhaustive binary32 check), and v_rcp_f32 is within 1 ulp. Such an s
//    lies in [2^-24, 65504], so 1/s is a normal number.
template <int F>
__device__ __forceinline__ float amax_over_qmax(float amax) {
  constexpr float q = Fmt<F>::qmax;
  constexpr float r = 1.0f / Fmt<F>::qmax;
  const float q0 = amax * r;
  const float nrem = __builtin_fmaf(q0, q, -amax);
  return __builtin_fmaf(-nrem, r, q0);
}
__device__ __forceinline__ void set_div_narrow(Scale& sc) {
  const float r0 = __builtin_amdgcn_rcpf(sc.s);
  const float r = __builtin_fmaf(__builtin_fmaf(-sc.s, r0, 1.0f), r0, r0);
  const bool zero = sc.s == 0.0f;
  sc.r = zero ? 0.0f : r;
  sc.div = zero ? DIV_ZERO : DIV_MARKSTEIN;
}

// Symmetric AbsMax scale from a group's max |x|.
template <int F>
__device__ __forceinline__ Scale scale_sym(float amax, int scale_fmt) {
  using T = Fmt<F>;
  Scale sc;
  sc.zp = 0.0f;
  sc.zbits = 0u;
  if (scale_fmt == LQ_SCALE_UE8M0) {
    // smallest e with Qmax * 2^e >= amax: compare frexp() significands
    int e;
    if (amax == 0.0f) {
      e = -127;
    } else {
      int ex = __builtin_amdgcn_frexp_expf(amax);
      float m = __builtin_amdgcn_frexp_mantf(amax);
      e = ex - T::qexp + (m > T::qmant ? 1 : 0);
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
    }
    sc.sbits = (uint32_t)(e + 127);
    sc.s = __builtin_ldexpf(1.0f, e);
    sc.r = __builtin_ldexpf(1.0f, -e);
    sc.div = DIV_POW2;
    return sc;
  }
  if (scale_fmt == LQ_SCALE_F16 || scale_fmt == LQ_SCALE_E4M3) {
    const float t = amax_over_qmax<F>(amax);
    if (scale_fmt == LQ_SCALE_F16) {
      sc.sbits = f16_bits_sat(t);
      sc.s = f16_value(sc.sbits);
    } else {
      sc.sbits = e4m3_scale_bits(t);
      sc.s = e4m3_scale_value(sc.sbits);
    }
    set_div_narrow(sc);
    return sc;
  }
  const float t = amax / T::qmax;
  sc.s = t;
  sc.sbits = __float_as_uint(t);
  set_div(sc);
  return sc;
}

// Integer code range: symmetric INT8 [-127,127], otherwise [-128,127] / [-8,7].
template <int F>
__device__ __forceinline__ float qmin_of(bool sym) {
  if constexpr (F == LQ_INT8) return sym ? -127.0f : -128.0f;
  else return -8.0f;
}

__device__ __forceinline__ float round_int(float v, int rnd) {
  if (rnd == LQ_RNE) return __builtin_rintf(v);
  const float t = __builtin_truncf(v);
  return (fabsf(v - t) >= 0.5f) ? t + __builtin_copysignf(1.0f, v) : t;
}

// Asymmetric (zero-point) scale over [min(mn,0), max(mx,0)] (INT, F32/F16).
template <int F>
__device__ __forceinline__ Scale scale_asym(float mn, float mx, int scale_fmt, int rnd) {
  using T = Fmt<F>;
  const float qmin = qmin_of<F>(false);
  const float lo = fminf(mn, 0.0f), hi = fmaxf(mx, 0.0f);
  const float t = (hi - lo) / (T::qmax - qmin);
  Scale sc;
  if (scale_fmt == LQ_SCALE_F16) {
    sc.sbits = f16_bits_sat(t);
    sc.s = f16_value(sc.sbits);
  } else {
    sc.s = t;
    sc.sbits = __float_as_uint(t);
  }
  set_div(sc);
  float zp = 0.0f;
  if (sc.s != 0.0f) zp = clampf(qmin - round_int(lo / sc.s, rnd), qmin, T::qmax) + 0.0f;
  sc.zp = zp;
  sc.zbits = (scale_fmt == LQ_SCALE_F16) ? f16_bits_sat(zp) : __float_as_uint(zp);
  return sc;
}

// A scale read back from storage (caller-supplied, or for dequantization).
__device__ __forceinline__ Scale scale_load(const void* scales, const void* zeros, int64_t idx,
                                            int scale_fmt, bool sym, bool need_div) {
  Scale sc;
  switch (scale_fmt) {
    case LQ_SCALE_F32: sc.sbits = ((const uint32_t*)scales)[idx]; sc.s = __uint_as_float(sc.sbits); break;
    case LQ_SCALE_F16: sc.sbits = ((const uint16_t*)scales)[idx]; sc.s = f16_value(sc.sbits); break;
    case LQ_SCALE_UE8M0: sc.sbits = ((const uint8_t*)scales)[idx]; sc.s = __builtin_ldexpf(1.0f, (int)sc.sbits - 127); break;
    default: sc.sbits = ((const uint8_t*)scales)[idx]; sc.s = e4m3_scale_value(sc.sbits); break;
  }
  sc.zp = 0.0f;
  sc.zbits = 0u;
  if (!sym) {
    if (scale_fmt == LQ_SCALE_F16) { sc.zbits = ((const uint16_t*)zeros)[idx]; sc.zp = f16_value(sc.zbits); }
    else { sc.zbits = ((const uint32_t*)zeros)[idx]; sc.zp = __uint_as_float(sc.zbits); }
  }
  if (need_div) {
    if (scale_fmt == LQ_SCALE_UE8M0) {
      sc.r = __builtin_ldexpf(1.0f, 127 - (int)sc.sbits);
      sc.div = DIV_POW2;
    } else {
      set_div(sc);
    }
  }
  return sc;
}

__device__ __forceinline__ void scale_store(void* scales, void* zeros, int64_t idx, const Scale& sc,
                                            int scale_fmt, bool sym) {
  if (scales) {
    switch (scale_fmt) {
      case LQ_SCALE_F32: ((uint32_t*)scales)[idx] = sc.sbits; break;
      case LQ_SCALE_F16: ((uint16_t*)scales)[idx] = (uint16_t)sc.sbits; break;
      default: ((uint8_t*)scales)[idx] = (uint8_t)sc.sbits; break;
    }
  }
  if (zeros && !sym) {
    if (scale_fmt == LQ_SCALE_F16) ((uint16_t*)zeros)[idx] = (uint16_t)sc.zbits;
    else ((uint32_t*)zeros)[idx] = sc.zbits;
  }
}

// ---------------------------------------------------------------- lanes
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
// The two values of 16-lane rows 2k and 2k+1 combined, in every lane of both
// rows: v_permlane16_swap exchanges odd rows of one copy with even rows of
// the other, so the two results hold the pair's rows (every lane active).
template <bool MAX>
__device__ __forceinline__ float row_pair(float a) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  const float p = __uint_as_float(r[0]), q = __uint_as_float(r[1]);
  return MAX ? fmaxf(p, q) : fminf(p, q);
}

// Combine a value over groups of `lanes` neighbouring lanes (1..32), every
// lane of a group ending with the group result. Up to 16 lanes the partners
// come from DPP row permutations; the 32-lane step swaps row pairs.
__device__ __forceinline__ float group_max(float a, int lanes) {
  if (lanes >= 2) a = fmaxf(a, dpp<0xB1>(a));   // quad_perm [1,0,3,2]
  if (lanes >= 4) a = fmaxf(a, dpp<0x4E>(a));   // quad_perm [2,3,0,1]
  if (lanes >= 8) a = fmaxf(a, dpp<0x141>(a));  // row_half_mirror
  if (lanes >= 16) a = fmaxf(a, dpp<0x140>(a)); // row_mirror
  if (lanes >= 32) a = row_pair<true>(a);
  return a;
}
__device__ __forceinline__ float group_min(float a, int lanes) {
  if (lanes >= 2) a = fminf(a, dpp<0xB1>(a));
  if (lanes >= 4) a = fminf(a, dpp<0x4E>(a));
  if (lanes >= 8) a = fminf(a, dpp<0x141>(a));
  if (lanes >= 16) a = fminf(a, dpp<0x140>(a));
  if (lanes >= 32) a = row_pair<false>(a);
  return a;
}
// The same for two independent values at once (the two halves of a
// lane-contiguous tile): one branch on the group width, then both DPP chains
// in straight-line code so that each hides the other's latency.
template <bool MAX>
__device__ __forceinline__ float comb(float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); }
template <bool MAX, int LANES>
__device__ __forceinline__ void group2_fixed(float& a, float& b) {
  if (LANES >= 2) { a = comb<MAX>(a, dpp<0xB1>(a)); b = comb<MAX>(b, dpp<0xB1>(b)); }
  if (LANES >= 4) { a = comb<MAX>(a, dpp<0x4E>(a)); b = comb<MAX>(b, dpp<0x4E>(b)); }
  if (LANES >= 8) { a = comb<MAX>(a, dpp<0x141>(a)); b = comb<MAX>(b, dpp<0x141>(b)); }
  if (LANES >= 16) { a = comb<MAX>(a, dpp<0x140>(a)); b = comb<MAX>(b, dpp<0x140>(b)); }
  if (LANES >= 32) { a = row_pair<MAX>(a); b = row_pair<MAX>(b); }
}
template <bool MAX>
__device__ __forceinline__ void group2(float& a, float& b, int lanes) {
  switch (lanes) {
    case 2: group2_fixed<MAX, 2>(a, b); break;
    case 4: group2_fixed<MAX, 4>(a, b); break;
    case 8: group2_fixed<MAX, 8>(a, b); break;
    case 16: group2_fixed<MAX, 16>(a, b); break;
    case 32: group2_fixed<MAX, 32>(a, b); break;
    default: break;
  }
}
__device__ __forceinline__ float wave_max(float a) {
  a = group_max(a, 16);
  a = fmaxf(a, __shfl_xor(a, 16));
  return fmaxf(a, __shfl_xor(a, 32));
}
__device__ __forceinline__ float wave_min(float a) {
  a = group_min(a, 16);
  a = fminf(a, __shfl_xor(a, 16));
  return fminf(a, __shfl_xor(a, 32));
}

// ---------------------------------------------------------------- rotation
// Walsh-Hadamard rotation of aligned groups of n = 16..1024 columns
// (walkerchi.com playbook §5.3: QuaRot's randomized Hadamard, an orthogonal
// R = H_n D / sqrt(n) per group with D the random signs of its columns;
// cyqw.cn/news/1000169 §4.2, §7.2). A lane holds 16 consecutive columns, so a
// group is n/16 consecutive lanes (a whole wave for 1024; every rotating
// kernel gives consecutive lanes consecutive tiles from a 64-aligned start,
// with every lane of a wave active at each stage). Stages in Sylvester order,
// each (a, b) -> (a + b, a - b) in binary32: strides 1, 2, 4, 8 inside the
// lane, then lane strides 1 .. 32 (element strides 16..512), where the lower lane
// adds its partner's b to its a and the upper subtracts its b from the
// partner's a (the same two operations). Forward: signs, stages, * c;
// inverse: stages, * c, signs. c = 1/sqrt(n) rounded to binary32.
struct Rot {
  int n;           // 0: no rotation; else 16, 32, 64, 128, 256, 512 or 1024
  float c;         // 1/sqrt(n) in binary32
  uint32_t sbits;  // the signs of this lane's 16 columns (bit i set: column i negated)
  bool has_signs;  // the same for the whole launch: no sign work without signs
};

// sign bits of the 16 columns starting at `col` (a multiple of 16)
__device__ __forceinline__ uint32_t rot_signs(const uint32_t* signs, int64_t col) {
  return signs ? (signs[col >> 5] >> (col & 16)) & 0xFFFFu : 0u;
}

// The value of lane ^ D. D = 1, 2: one DPP quad permutation ([1,0,3,2],
// [2,3,0,1]). D = 4, 8, 16: ds_swizzle in bit mode (xor D, and-mask 31)
// through the LDS pipe, no address registers (lane ^ 4 and ^ 16 have no
// single DPP move; lane ^ 8 has one, row_ror:8, but the VALU move measured
// slower than the swizzle: 158.6-160.2 against 154.3-154.6 us per NVFP4 c4r
// call, NVINT4 and c4q no better, both orders on one box). Measured on
// C4's tensor under the 256-point rotation (NVFP4 / NVINT4 with signs), one
// box: 166.0 / 166.3 us per call with DPP for D = 1, 2 against 174.6 / 169.9
// us with the swizzle for every D (1024 points: 186.9 / 187.8 against 191.0
// / 193.8); with every D on DPP the 256-point kernels took 217-220 us against
// 192-197 us. Lane ^ 32 crosses the wave's halves through ds_bpermute
// (v_permlane32_swap on two copies of v measured 9 more VGPRs in the
// rotating kernels).
template <int D>
__device__ __forceinline__ float xor_lane(float v) {
  if constexpr (D == 32) return __shfl_xor(v, 32);
  else if constexpr (D == 1) return dpp<0xB1>(v);
  else if constexpr (D == 2) return dpp<0x4E>(v);
  else return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (D << 10)));
}

template <int D>
__device__ __forceinline__ void lane_stage(float* v) {
  // lower lane: own + partner; upper lane: partner - own; fma(±1, own,
  // partner) rounds once, so it is exactly either, in one VALU operation
  const float sgn = (threadIdx.x & D) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 16; i++) v[i] = __builtin_fmaf(sgn, v[i], xor_lane<D>(v[i]));
}

// MAXN: the largest n the caller can pass (16: no lane stages are compiled).
// STRAIGHT: when n == MAXN, the lane stages run straight through. Behind a
// branch each, every stage ends in a merge that copies the 16 values back
// into place (16 more VALU operations per stage); the second copy of the
// stages costs registers, so only kernels with room for it ask for it.
template <int MAXN = 1024, bool STRAIGHT = false>
__device__ __forceinline__ void rot_stages(float* v, int n) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  if (STRAIGHT && n == MAXN) {
    if constexpr (MAXN >= 32) lane_stage<1>(v);
    if constexpr (MAXN >= 64) lane_stage<2>(v);
    if constexpr (MAXN >= 128) lane_stage<4>(v);
    if constexpr (MAXN >= 256) lane_stage<8>(v);
    if constexpr (MAXN >= 512) lane_stage<16>(v);
    if constexpr (MAXN >= 1024) lane_stage<32>(v);
    return;
  }
  if (MAXN >= 32 && n >= 32) lane_stage<1>(v);
  if (MAXN >= 64 && n >= 64) lane_stage<2>(v);
  if (MAXN >= 128 && n >= 128) lane_stage<4>(v);
  if (MAXN >= 256 && n >= 256) lane_stage<8>(v);
  if (MAXN >= 512 && n >= 512) lane_stage<16>(v);
  if (MAXN >= 1024 && n >= 1024) lane_stage<32>(v);
}

__device__ __forceinline__ void rot_apply_signs(float* v, uint32_t sbits) {
#pragma unroll
  for (int i = 0; i < 16; i++) v[i] = __uint_as_float(__float_as_uint(v[i]) ^ (((sbits >> i) & 1u) << 31));
}

// The rotation of the 16 elements starting at element e0 (a row-major tensor
// of `cols` columns; signs may be null).
__device__ __forceinline__ Rot make_rot(int n, float c, const uint32_t* signs, int64_t e0, int64_t cols) {
  Rot r;
  r.n = n;
  r.c = c;
  r.has_signs = signs != nullptr;
  r.sbits = r.has_signs ? rot_signs(signs, e0 % cols) : 0u;
  return r;
}

template <int MAXN = 1024, bool STRAIGHT = false>
__device__ __forceinline__ void rot_forward(float* v, const Rot& r) {
  if (r.has_signs) rot_apply_signs(v, r.sbits);
  rot_stages<MAXN, STRAIGHT>(v, r.n);
#pragma unroll
  for (int i = 0; i < 16; i++) v[i] = v[i] * r.c;
}

template <int MAXN = 1024, bool STRAIGHT = false>
__device__ __forceinline__ void rot_inverse(float* v, const Rot& r) {
  rot_stages<MAXN, STRAIGHT>(v, r.n);
#pragma unroll
  for (int i = 0; i < 16; i++) v[i] = v[i] * r.c;
  if (r.has_signs) rot_apply_signs(v, r.sbits);
}

// 128-bit and 64-bit vectors for global loads and stores
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Outputs are written with non-temporal stores (streamed: they are not read
// back by this launch, and keeping them out of the caches leaves room for the
// inputs); loads are ordinary.
#ifndef LQ_NT_LOAD
#define LQ_NT_LOAD 0
#endif
#ifndef LQ_NT_STORE
#define LQ_NT_STORE 1
#endif
template <typename V>
__device__ __forceinline__ V gload(const V* p) {
#if LQ_NT_LOAD
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}
template <typename V>
__device__ __forceinline__ void gstore(V* p, V v) {
#if LQ_NT_STORE
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

// Raw bytes of one tile of input (16 elements of dtype DT).
template <int DT> struct Raw { u32x4 w[DT == LQ_F32 ? 4 : 2]; };

template <int DT>
__device__ __forceinline__ void raw_load(Raw<DT>& r, const void* x, int64_t e0) {
  constexpr int esz = (DT == LQ_F32) ? 4 : 2;
  const u32x4* p = (const u32x4*)((const char*)x + e0 * esz);
#pragma unroll
  for (int i = 0; i < (DT == LQ_F32 ? 4 : 2); i++) r.w[i] = gload(p + i);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maximum). Issued once
// after a loop's first prefetch: the first tile must land before the loop, and
// with the entry state drained the compiler's wait at the top of the loop only
// covers the prefetch, not the stores of the previous tile (on gfx9 stores
// count in vmcnt too).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int DT>
__device__ __forceinline__ void raw_to_float(const Raw<DT>& r, float* v) {
  const uint32_t* u = (const uint32_t*)r.w;
  if constexpr (DT == LQ_F32) {
#pragma unroll
    for (int i = 0; i < 16; i++) v[i] = __uint_as_float(u[i]);
  } else if constexpr (DT == LQ_BF16) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      v[2 * i] = f16_value(u[i] & 0xFFFFu);
      v[2 * i + 1] = f16_value(u[i] >> 16);
    }
  }
}

template <int DT>
__device__ __forceinline__ float load_one(const void* x, int64_t e) {
  if constexpr (DT == LQ_F32) return ((const float*)x)[e];
  else if constexpr (DT == LQ_BF16) return __uint_as_float((uint32_t)((const uint16_t*)x)[e] << 16);
  else return f16_value(((const uint16_t*)x)[e]);
}

// Load `cnt` (< 16) elements one by one; the rest read as 0.
template <int DT>
__device__ __forceinline__ void load_partial(const void* x, int64_t e0, int cnt, float* v) {
#pragma unroll
  for (int i = 0; i < 16; i++) v[i] = (i < cnt) ? load_one<DT>(x, e0 + i) : 0.0f;
}

// bf16/fp16 conversions of two floats, round to nearest even
typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){a, b}, bf2v));
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){a, b}, h2v));
}

// Store 16 fp32 values as out dtype: a full tile with 16-byte stores; a
// partial one element by element (unrolled with constant indices, so the
// values stay in registers).
__device__ __forceinline__ void store_y(void* y, int64_t e0, int cnt, const float* v, int out_dt) {
  if (cnt == 16) {
    if (out_dt == LQ_F32) {
      u32x4* p = (u32x4*)((float*)y + e0);
#pragma unroll
      for (int i = 0; i < 4; i++)
        gstore(p + i, (u32x4){__float_as_uint(v[4 * i]), __float_as_uint(v[4 * i + 1]),
                              __float_as_uint(v[4 * i + 2]), __float_as_uint(v[4 * i + 3])});
    } else {
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; i++)
        w[i] = (out_dt == LQ_BF16) ? pack_bf16x2(v[2 * i], v[2 * i + 1]) : pack_f16x2(v[2 * i], v[2 * i + 1]);
      u32x4* p = (u32x4*)((uint16_t*)y + e0);
      gstore(p, (u32x4){w[0], w[1], w[2], w[3]});
      gstore(p + 1, (u32x4){w[4], w[5], w[6], w[7]});
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      if (i < cnt) {
        if (out_dt == LQ_F32) {
          ((float*)y)[e0 + i] = v[i];
        } else {
          const uint32_t w = (out_dt == LQ_BF16) ? pack_bf16x2(v[i], 0.f) : pack_f16x2(v[i], 0.f);
          ((uint16_t*)y)[e0 + i] = (uint16_t)(w & 0xFFFFu);
        }
      }
    }
  }
}

// Codes of one tile: 16 bytes (8-bit formats) or 8 bytes (4-bit), little
// endian; element 2j of a 4-bit tile in the low nibble of byte j.
struct Codes { uint32_t w[4]; };

// FP6 codes of a tile: element i in bits 6i .. 6i+5 of words w[0..2] (96
// bits); in memory from byte 3 * e0 / 4 (e0 and cnt are multiples of 4, so a
// tile's codes are whole bytes; word stores when e0 is a multiple of 16, which
// makes them 4-byte aligned; per-row tiles of rows that are not may start
// anywhere).
template <int F>
__device__ __forceinline__ void store_codes(uint8_t* codes, int64_t e0, int cnt, const Codes& c) {
  if constexpr (Fmt<F>::six) {
    uint8_t* p = codes + e0 / 4 * 3;
    if (cnt == 16 && (e0 & 15) == 0) {
      uint32_t* q = (uint32_t*)p;
      gstore(q, c.w[0]);
      gstore(q + 1, c.w[1]);
      gstore(q + 2, c.w[2]);
    } else {
      // cnt is a multiple of 4 (rows hold a multiple of 4 elements): whole bytes
#pragma unroll
      for (int i = 0; i < 12; i++)
        if (4 * i < 3 * cnt) p[i] = (uint8_t)(c.w[i / 4] >> (8 * (i % 4)));
    }
  } else if constexpr (Fmt<F>::four) {
    if (cnt == 16) {
      gstore((u32x2*)(codes + e0 / 2), (u32x2){c.w[0], c.w[1]});
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++)
        if (2 * i < cnt) codes[e0 / 2 + i] = (uint8_t)(c.w[i / 4] >> (8 * (i % 4)));
    }
  } else {
    if (cnt == 16) {
      gstore((u32x4*)(codes + e0), (u32x4){c.w[0], c.w[1], c.w[2], c.w[3]});
    } else {
#pragma unroll
      for (int i = 0; i < 16; i++)
        if (i < cnt) codes[e0 + i] = (uint8_t)(c.w[i / 4] >> (8 * (i % 4)));
    }
  }
}

// Launch-wide choices: Mode holds them as kernel arguments (uniform across
// the grid; each picks one straight-line version of the tile pipeline with a
// scalar branch); ModeC fixes them at compile time for the specialised
// kernels. The tile pipeline is written once for both.
struct Mode {
  bool pow2;  // UE8M0 scales: dividing is an exact power-of-two scaling
  bool sym;   // AbsMax (no zero point)
  bool rna;   // integer rounding half away from zero (else half to even)
};
template <bool POW2, bool SYM, bool RNA>
struct ModeC {
  static constexpr bool pow2 = POW2;
  static constexpr bool sym = SYM;
  static constexpr bool rna = RNA;
};

// Element accessors of a tile: straight from the raw input registers (no
// 16-float copy is kept live), or from an fp32 array (rotated or partial tiles).
template <int DT>
struct RawX {
  static constexpr int dt = DT;   // the input dtype the values come from
  const Raw<DT>& r;
  __device__ __forceinline__ float operator()(int i) const {
    const uint32_t* u = (const uint32_t*)r.w;
    if constexpr (DT == LQ_F32) return __uint_as_float(u[i]);
    else if constexpr (DT == LQ_BF16) return __uint_as_float((i & 1) ? (u[i >> 1] & 0xFFFF0000u) : (u[i >> 1] << 16));
    else return f16_value((i & 1) ? (u[i >> 1] >> 16) : (u[i >> 1] & 0xFFFFu));
  }
};
struct ArrX {
  static constexpr int dt = -1;   // decoded already (fp32 values of any input)
  const float* x;
  __device__ __forceinline__ float operator()(int i) const { return x[i]; }
};

// Output words of one tile in the output dtype (bf16/fp16 pairs, or fp32).
template <int ODT> struct YW { uint32_t w[ODT == LQ_F32 ? 16 : 8]; };

template <int ODT>
__device__ __forceinline__ void put_y(YW<ODT>& y, int i, float a, float b) {
  if constexpr (ODT == LQ_F32) { y.w[i] = __float_as_uint(a); y.w[i + 1] = __float_as_uint(b); }
  else if constexpr (ODT == LQ_BF16) y.w[i >> 1] = pack_bf16x2(a, b);
  else y.w[i >> 1] = pack_f16x2(a, b);
}

template <int ODT>
__device__ __forceinline__ void store_yw(void* y, int64_t e0, int cnt, const YW<ODT>& yw) {
  if (cnt == 16) {
    u32x4* p = (u32x4*)((char*)y + e0 * (ODT == LQ_F32 ? 4 : 2));
#pragma unroll
    for (int j = 0; j < (ODT == LQ_F32 ? 4 : 2); j++)
      gstore(p + j, (u32x4){yw.w[4 * j], yw.w[4 * j + 1], yw.w[4 * j + 2], yw.w[4 * j + 3]});
  } else {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      if (i < cnt) {
        if constexpr (ODT == LQ_F32) ((uint32_t*)y)[e0 + i] = yw.w[i];
        else ((uint16_t*)y)[e0 + i] = (uint16_t)(yw.w[i >> 1] >> (16 * (i & 1)));
      }
    }
  }
}

// Division modes for v = x / s (all correctly rounded):
//  DIVM_MARKSTEIN: Markstein's correction around r = RN(1/s) (q0 = x*r,
//    rem = x - q0*s exactly, v = q0 + rem*r), for 1/s finite; an exact
//    multiply by 2^-e for power-of-two scales;
//  DIVM_IEEE: plain division (a scale whose 1/s overflows, any x);
//  DIVM_PRESCALED: the same correction on x * 2^64 and s * 2^64 (a scale
//    whose 1/s overflows, scales computed from the data so |x| <= Qmax * s and
//    the scaled x stays finite; both scalings are exact).
constexpr int DIVM_MARKSTEIN = 0, DIVM_IEEE = 1, DIVM_PRESCALED = 2;
// `sgn` gives the sign of a zero quotient (x itself, or the value x was
// derived from by a positive division).
template <bool FP, int DIVM>
__device__ __forceinline__ float divide(float x, const Scale& sc, bool pow2, float sgn) {
  if (DIVM == DIVM_IEEE) return x / sc.s;
  if (DIVM == DIVM_MARKSTEIN && pow2) return x * sc.r;
  const float xs = DIVM == DIVM_PRESCALED ? x * 0x1p64f : x;
  const float ss = DIVM == DIVM_PRESCALED ? sc.s * 0x1p64f : sc.s;
  const float q0 = xs * sc.r;
  const float rem = __builtin_fmaf(-q0, ss, xs);
  const float v = __builtin_fmaf(rem, sc.r, q0);
  return FP ? __builtin_copysignf(v, sgn) : v;   // x = -0 gives -0
}
template <bool FP, int DIVM>
__device__ __forceinline__ float divide(float x, const Scale& sc, bool pow2) {
  return divide<FP, DIVM>(x, sc, pow2, x);
}

// ---------------------------------------------------------------- two-level
// NVFP4-style two-level scaling (walkerchi.com quantization playbook §4.3.1
// "Tensor-level scale", §4.3.2): an FP32 tensor scale S above E4M3 block
// scales, x = x_q * s_block * S. S normalizes the whole tensor first: each
// value is divided by S, the quotients are block-quantized as usual, and
// the dequantized value is (value * s_block) * S (the first product is exact).
// S = max|x| / (448 * Qmax) (448: the largest E4M3 value), so the block
// holding the largest magnitude gets the largest block scale; an S of 0 (an
// all-zero tensor, or an underflowing quotient) becomes 1.
struct TScale {
  float s;    // S
  float r;    // RN(1 / (S * p))
  float sp;   // S * p
  float p;    // 1, or 2^64 when 1/S overflows: every |x| <= 448 * Qmax * S is
              // then tiny, so x * 2^64 is exact and finite
};

template <int F>
__device__ __forceinline__ float tensor_scale_of(float amax) {
  constexpr float kDen = 448.0f * Fmt<F>::qmax;   // exact
  const float S = amax / kDen;
  return S == 0.0f ? 1.0f : S;
}

__device__ __forceinline__ TScale tscale_make(float S) {
  TScale t;
  t.s = S;
  const float r = 1.0f / S;
  t.p = r < __builtin_inff() ? 1.0f : 0x1p64f;
  t.sp = S * t.p;
  t.r = 1.0f / t.sp;
  return t;
}

// The same in every lane: into scalar registers.
__device__ __forceinline__ TScale tscale_uniform(const TScale& t) {
  TScale u;
  u.s = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(t.s)));
  u.r = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(t.r)));
  u.sp = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(t.sp)));
  u.p = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(t.p)));
  return u;
}

// x / S correctly rounded: Markstein's correction on x * p and S * p
// (TL_FAST, for an S computed from the data), or IEEE division (TL_IEEE, for a
// given S of any size). TL_NONE: no tensor level. TL_FAST leaves the sign of
// a zero quotient open: only the element encoders look at it, and they take
// it from x (S > 0).
constexpr int TL_NONE = 0, TL_FAST = 1, TL_IEEE = 2;
template <int TL>
__device__ __forceinline__ float tdivide(float x, const TScale& t) {
  if constexpr (TL == TL_IEEE) {
    return x / t.s;
  } else {
    const float xs = x * t.p;
    const float q0 = xs * t.r;
    const float rem = __builtin_fmaf(-q0, t.sp, xs);
    return __builtin_fmaf(rem, t.r, q0);
  }
}

// Quantize group G (elements 8G..8G+7) of a tile under scale `sc`: codes
// into c (8-bit: words 2G, 2G+1; 4-bit: word G), output words (or the fp32
// dequantized values when XH, for a rotation back), and the group's fp32 terms
// of (x - xhat)^2 and x^2 added to ee and ss in element order. With a tensor
// level (TL != TL_NONE, *tl = S) the codes are those of x / S under sc and
// xhat is multiplied by S; the terms stay those of x.
template <int G, int F, int ODT, bool XH, int DIVM, int TL = TL_NONE, class X, class M>
__device__ __forceinline__ void quant_group(const X& xs, const Scale& sc, const M& m, Codes& c, YW<ODT>& yw,
                                            float* xh_out, float& ee, float& ss, const TScale* tl = nullptr) {
  using T = Fmt<F>;
  float x[8], v[8], xh[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    x[i] = xs(8 * G + i);
    const float xq = TL != TL_NONE ? tdivide<TL>(x[i], *tl) : x[i];
    v[i] = divide<!T::is_int, DIVM>(xq, sc, m.pow2, x[i]);
  }
  if constexpr (T::is_int) {
    const float qmin = qmin_of<F>(m.sym);
    int qi[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      float q;
      if (m.rna) {
        const float t = __builtin_truncf(v[i]);
        q = (fabsf(v[i] - t) >= 0.5f) ? t + __builtin_copysignf(1.0f, v[i]) : t;
      } else {
        q = __builtin_rintf(v[i]);
      }
      if (m.sym) {
        q = clampf(q, qmin, T::qmax);
        xh[i] = __builtin_fmaf(q, sc.s, 0.0f);   // the +0 turns a -0 into +0
      } else {
        q = clampf(q + sc.zp, qmin, T::qmax);
        xh[i] = sc.s * (q - sc.zp);
      }
      qi[i] = (int)q;
    }
    if constexpr (T::four) {
      uint32_t w = 0;
#pragma unroll
      for (int k = 0; k < 8; k++) w |= ((uint32_t)qi[k] & 0xFu) << (4 * k);
      c.w[G] = w;
    } else {
      // low bytes of four ints into one word: v_perm_b32 picks bytes of a pair
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const uint32_t lo = __builtin_amdgcn_perm((uint32_t)qi[4 * j + 1], (uint32_t)qi[4 * j], 0x0c0c0400u);
        const uint32_t hi = __builtin_amdgcn_perm((uint32_t)qi[4 * j + 3], (uint32_t)qi[4 * j + 2], 0x0c0c0400u);
        c.w[2 * G + j] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = clampf(v[i], -T::qmax, T::qmax);
    float d[8];
    if constexpr (T::six) {
      // bit-manipulation encoder; the group's eight 6-bit codes fill bits
      // 48G .. 48G+47 of the tile's 96 (group 1 after group 0)
      uint64_t u = 0;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        // the value from the encoder (4-5 us per MXFP6 call on C2's tensor in
        // the lane-contiguous kernels), except for fp32 raw tiles, whose
        // tile-per-lane kernels then pass 128 VGPRs: there the code is decoded
        uint32_t q;
        if constexpr (X::dt == LQ_F32) {
          q = alu_encode<T::E, T::M, T::BIAS>(v[i]);
          d[i] = alu_decode<T::E, T::M, T::BIAS>(q);
        } else {
          q = alu_encode_v<T::E, T::M, T::BIAS>(v[i], d[i]);
        }
        u |= (uint64_t)q << (6 * i);
      }
      if constexpr (G == 0) {
        c.w[0] = (uint32_t)u;
        c.w[1] = (uint32_t)(u >> 32);
      } else {
        c.w[1] |= (uint32_t)(u << 16);
        c.w[2] = (uint32_t)(u >> 16);
      }
    } else if constexpr (F == LQ_E2M1) {
      c.w[G] = fp4_pack8(v);
      fp4_unpack8(c.w[G], d);
    } else {
#pragma unroll
      for (int j = 0; j < 2; j++) {
        c.w[2 * G + j] = fp8_pack4<F>(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
        fp8_unpack4<F>(c.w[2 * G + j], d + 4 * j);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; i++) xh[i] = d[i] * sc.s;
  }
  if constexpr (TL != TL_NONE) {
#pragma unroll
    for (int i = 0; i < 8; i++) xh[i] = xh[i] * tl->s;
  }
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float dd = x[i] - xh[i];
    ee = __builtin_fmaf(dd, dd, ee);
    ss = __builtin_fmaf(x[i], x[i], ss);
  }
  if constexpr (XH) {
#pragma unroll
    for (int i = 0; i < 8; i++) xh_out[8 * G + i] = xh[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; i += 2) put_y<ODT>(yw, 8 * G + i, xh[i], xh[i + 1]);
  }
}

// FP6 with the native conversion: a tile's 16 quotients first (group G
// under its own scale), then all 16 codes in one conversion and their values
// in one decode (six_finish).
template <int G, int F, int DIVM, int TL = TL_NONE, class X, class M>
__device__ __forceinline__ void six_quotients(const X& xs, const Scale& sc, const M& m, float* v,
                                              const TScale* tl = nullptr) {
#pragma unroll
  for (int i = 8 * G; i < 8 * G + 8; i++) {
    const float x = xs(i);
    const float xq = TL != TL_NONE ? tdivide<TL>(x, *tl) : x;
    v[i] = divide<true, DIVM>(xq, sc, m.pow2, x);
  }
}

// Codes (c.w[0..2]), output words (or the fp32 dequantized values when XH)
// and fp32 terms of (x - xhat)^2 and x^2 of both groups (group G's into eG,
// sG, in element order; the same accumulators may be passed for both). The
// inputs are read from xs again rather than held across the conversion,
// whose two 16-register operands are the kernels' register peak.
template <int F, int ODT, bool XH, int TL = TL_NONE, class X>
__device__ __forceinline__ void six_finish(const X& xs, const float* v, const Scale& s0, const Scale& s1, Codes& c,
                                           YW<ODT>& yw, float* xh_out, float& e0, float& q0, float& e1, float& q1,
                                           const TScale* tl = nullptr) {
  float x[16];
  const lq_v6u w = fp6_encode16<F>(v);   // saturating: no clamp needed
  c.w[0] = w[0];
  c.w[1] = w[1];
  c.w[2] = w[2];
  const lq_v32h h = fp6_halves32<F>(w);
  float xh[16];
#pragma unroll
  for (int i = 0; i < 16; i++) {
    x[i] = xs(i);
    xh[i] = (float)h[i] * (i < 8 ? s0.s : s1.s);   // the value is exact in fp16: one rounding
    if constexpr (TL != TL_NONE) xh[i] = xh[i] * tl->s;
  }
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float dd = x[i] - xh[i];
    e0 = __builtin_fmaf(dd, dd, e0);
    q0 = __builtin_fmaf(x[i], x[i], q0);
  }
#pragma unroll
  for (int i = 8; i < 16; i++) {
    const float dd = x[i] - xh[i];
    e1 = __builtin_fmaf(dd, dd, e1);
    q1 = __builtin_fmaf(x[i], x[i], q1);
  }
  if constexpr (XH) {
#pragma unroll
    for (int i = 0; i < 16; i++) xh_out[i] = xh[i];
  } else {
#pragma unroll
    for (int i = 0; i < 16; i += 2) put_y<ODT>(yw, i, xh[i], xh[i + 1]);
  }
}

// Quantize one tile under one scale, 8 elements at a time: codes, output
// words (or the fp32 dequantized values when XH), and the tile's fp32 sums of
// (x - xhat)^2 and x^2.
template <int F, int ODT, bool XH, int DIVM, int TL = TL_NONE, class X, class M>
__device__ __forceinline__ void quant_stream(const X& xs, const Scale& sc, const M& m, Codes& c, YW<ODT>& yw,
                                             float* xh_out, float& e, float& s, const TScale* tl = nullptr) {
  float ee = 0.0f, ss = 0.0f;
  if constexpr (Fmt<F>::six && LQ_NATIVE_FP6) {
    float v[16];
    six_quotients<0, F, DIVM, TL>(xs, sc, m, v, tl);
    six_quotients<1, F, DIVM, TL>(xs, sc, m, v, tl);
    six_finish<F, ODT, XH, TL>(xs, v, sc, sc, c, yw, xh_out, ee, ss, ee, ss, tl);
  } else {
    quant_group<0, F, ODT, XH, DIVM, TL>(xs, sc, m, c, yw, xh_out, ee, ss, tl);
    quant_group<1, F, ODT, XH, DIVM, TL>(xs, sc, m, c, yw, xh_out, ee, ss, tl);
  }
  if (Fmt<F>::four) c.w[2] = c.w[3] = 0u;
  if (Fmt<F>::six) c.w[3] = 0u;
  e = ee;
  s = ss;
}

// Values of one tile of codes (dequantization), before the scale.
template <int F>
__device__ __forceinline__ void decode_tile(const Codes& c, float* d) {
  using T = Fmt<F>;
  if constexpr (F == LQ_INT8) {
#pragma unroll
    for (int i = 0; i < 16; i++) d[i] = (float)(int8_t)((c.w[i / 4] >> (8 * (i % 4))) & 0xFFu);
  } else if constexpr (F == LQ_INT4) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int n = (int)((c.w[i / 8] >> (4 * (i % 8))) & 0xFu);
      d[i] = (float)(n >= 8 ? n - 16 : n);
    }
  } else if constexpr (T::six && LQ_NATIVE_FP6) {
    fp6_unpack16<F>(c.w[0], c.w[1], c.w[2], d);
  } else if constexpr (T::six) {
    const uint64_t lo = (uint64_t)c.w[0] | ((uint64_t)(c.w[1] & 0xFFFFu) << 32);
    const uint64_t hi = (uint64_t)(c.w[1] >> 16) | ((uint64_t)c.w[2] << 16);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      d[i] = alu_decode<T::E, T::M, T::BIAS>((uint32_t)(lo >> (6 * i)) & 63u);
      d[8 + i] = alu_decode<T::E, T::M, T::BIAS>((uint32_t)(hi >> (6 * i)) & 63u);
    }
  } else if constexpr (F == LQ_E2M1) {
    fp4_unpack8(c.w[0], d);
    fp4_unpack8(c.w[1], d + 8);
  } else {
#pragma unroll
    for (int j = 0; j < 4; j++) fp8_unpack4<F>(c.w[j], d + 4 * j);
  }
  (void)sizeof(T);
}

}  // namespace lqd
