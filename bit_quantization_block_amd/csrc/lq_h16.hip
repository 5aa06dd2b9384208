// lq_h16.hip — NVFP4 / NVINT4 blocks under the 16-point Walsh-Hadamard
// rotation: bf16 in and out, 4-bit elements (E2M1, INT4), blocks of 16 with
// E4M3 scales from the data, each block one rotation group (16 columns, no
// random signs), round half to even, every output (walkerchi.com quantization
// playbook §4.3.1 NV blocks; cyqw.cn/news/1000169 §4.2 and §7.2, the rotation
// before NVINT4).
//
// Memory layout. Global loads and stores are lane-contiguous (a wave takes
// 1024 consecutive elements; lane L reads elements 8L..8L+7 and 512+8L..
// 512+8L+7, so each 16-byte instruction covers 1 KB of whole cache lines),
// and the wave's 128 sixteen-byte units are exchanged through LDS so that
// lane L holds the 16 consecutive elements 16L..16L+15 of the chunk (one
// rotation group and one block). Measured on C4's traffic: 119.6 us with each
// lane reading its 16 elements straight from memory (every instruction then
// touches twice the lines, half each), 108.0 us through LDS, 108.1 us for the
// lane-contiguous pattern itself. The dequantized values go back through LDS
// the same way; the 8 code bytes and the scale byte of a lane are stored
// directly (contiguous across the wave).
//
// Arithmetic (exactly the general path's results; the reasons):
//  - The butterflies give h = 4y, y the rotated values (y = h * 0.25 in
//    binary32). The block maximum max|y| is RN(max|h| * 0.25) (rounding is
//    monotone), so the stored E4M3 scale s is the general path's. The element
//    quotient is RN(h / 4s) instead of RN(RN(h * 0.25) / s): equal whenever
//    h * 0.25 is exact, and otherwise |y| < 2^-126 while an E4M3 scale is 0 or
//    at least 2^-9, so both quotients lie below the smallest nonzero code
//    and round to a zero code of h's sign (or the block's codes are all 0).
//  - Division: Markstein's correction around r = RN(1/4s) (= RN(1/s) / 4),
//    ordered as v = fma(-fma(q0, 4s, -h), r, q0) so that a zero quotient
//    keeps the sign of h without a separate copysign.
//  - Dequantization and the rotation back: with d the code values (E2M1 or
//    INT4), xhat = d * s exactly, every butterfly sum of 16 such products is
//    exact (at most 8 significant bits of d, 4 of s), and the sign of every
//    zero follows the same operations whatever the common positive factor.
//    So the rotated-back y equals RN(B * (s / 4)) with B the butterflies of d,
//    taken here on packed fp16 pairs (B is at most 128 in magnitude, a
//    multiple of 1/2: exact in fp16), then one mixed-precision multiply.
//  - QSNR: (y - xhat) = (h - d * 4s) / 4 and y^2 = h^2 / 16, so the fp32 tile
//    sums are taken on h and scaled by 1/16 (exact barring under- or
//    overflow, which the range check sends to the fp64 path).
//
// Two-level scaling (k_h16_two: an fp32 tensor scale S above the E4M3 block
// scales, walkerchi.com playbook §4.3.2) takes the general path's arithmetic
// step for step on the rotated values y = RN(h * 0.25): the block scale from
// RN(max|y| / S), each quotient RN(RN(y / S) / s), xhat = (d * s) * S (the
// product by S rounds, so nothing is folded), the fp32 terms of (y - xhat)^2
// and y^2, and the rotation back in binary32. Only the memory layout and the
// block-per-lane shape are this kernel's.
#include "lq_fast.h"

namespace lqd {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// (lo + hi, lo - hi) of one packed pair: the first butterfly stage of two
// neighbouring elements in one instruction
__device__ __forceinline__ h2 pair_stage(h2 v) {
  h2 out;
  asm volatile("v_pk_add_f16 %0, %1, %1 op_sel:[0,1] op_sel_hi:[0,1] neg_hi:[0,1]" : "=v"(out) : "v"(v));
  return out;
}

// RN(lo_or_hi(v) * s) as binary32, signs of zeros kept (the addend is -0)
template <int HI>
__device__ __forceinline__ float mix_mul(h2 v, float s, float negzero) {
  float out;
  if constexpr (HI)
    asm volatile("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
                 : "=v"(out) : "v"(v), "v"(s), "s"(negzero));
  else
    asm volatile("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[1,0,0]"
                 : "=v"(out) : "v"(v), "v"(s), "s"(negzero));
  return out;
}

// Sylvester butterflies of 16 values in binary32, strides 1, 2, 4, 8
__device__ __forceinline__ void butterflies16(float* v) {
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
}

// The same on 8 packed fp16 pairs (element 2j in the low half of p[j])
__device__ __forceinline__ void butterflies16_h2(h2* p) {
#pragma unroll
  for (int j = 0; j < 8; j++) p[j] = pair_stage(p[j]);
#pragma unroll
  for (int s = 1; s < 8; s <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; j++) {
      if ((j & s) == 0) {
        const h2 a = p[j], b = p[j + s];
        p[j] = a + b;
        p[j + s] = a - b;
      }
    }
  }
}

// Markstein's correction for h / 4s (see above): a zero quotient keeps h's sign
__device__ __forceinline__ float div4s(float h, float s4, float r4) {
  const float q0 = h * r4;
  const float nrem = __builtin_fmaf(q0, s4, -h);
  return __builtin_fmaf(-nrem, r4, q0);
}

// One lane's block: codes (2 words), the scale, the output words, the fp32
// QSNR terms. h holds the butterflies of the block's 16 inputs (4y). Pairs of
// elements are finished one after the other (quotients, codes, code values,
// QSNR terms), so each pair's registers are free again before the next.
template <int F>
__device__ __forceinline__ void h16_block(const float* h, bool unrotate, float negzero, uint32_t* code, Scale& sc,
                                          uint32_t* yw, float& te, float& ts) {
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i++) am = fmaxf(am, fabsf(h[i]));
  sc = scale_sym<F>(am * 0.25f, LQ_SCALE_E4M3);     // max|y| = RN(max|h| / 4)
  const float s4 = sc.s * 4.0f, r4 = sc.r * 0.25f;    // r = RN(1/s); 0 with a zero scale
  float ee = 0.0f, ss = 0.0f;
  h2 d[8];
  uint32_t b[8];
  code[0] = code[1] = 0u;
  static_for<8>([&](auto j) __attribute__((always_inline)) {
    const float h0 = h[2 * j], h1 = h[2 * j + 1];
    float v0 = div4s(h0, s4, r4), v1 = div4s(h1, s4, r4);
    if constexpr (F == LQ_E2M1) {
      v0 = clampf(v0, -6.0f, 6.0f);
      v1 = clampf(v1, -6.0f, 6.0f);
      uint32_t& w = code[j / 4];
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v0, v1, 1.0f, j % 4);
      d[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, j % 4);
    } else {
      // round half to even by the binary32 addition of 1.5 * 2^23 (the sum's
      // low mantissa bits hold the integer, two's complement in the low
      // nibble), clamp in that domain, and the integer back as an exact
      // float (x - x = +0: a zero code has the value +0)
      constexpr float kMagic = 12582912.0f;
      const float u0 = clampf(v0 + kMagic, kMagic - 8.0f, kMagic + 7.0f);
      const float u1 = clampf(v1 + kMagic, kMagic - 8.0f, kMagic + 7.0f);
      b[j] = (__float_as_uint(u1) << 4) | (__float_as_uint(u0) & 0xFu);
      d[j] = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(u0 - kMagic, u1 - kMagic));
    }
    // QSNR terms on the 4y scale: (h - d * 4s)^2 and h^2
    const float dd0 = __builtin_fmaf(-(float)d[j].x, s4, h0);
    const float dd1 = __builtin_fmaf(-(float)d[j].y, s4, h1);
    ee = __builtin_fmaf(dd0, dd0, ee);
    ee = __builtin_fmaf(dd1, dd1, ee);
    ss = __builtin_fmaf(h0, h0, ss);
    ss = __builtin_fmaf(h1, h1, ss);
  });
  if constexpr (F != LQ_E2M1) {
#pragma unroll
    for (int w = 0; w < 2; w++) {
      const uint32_t lo = __builtin_amdgcn_perm(b[4 * w + 1], b[4 * w], 0x0c0c0400u);
      const uint32_t hi = __builtin_amdgcn_perm(b[4 * w + 3], b[4 * w + 2], 0x0c0c0400u);
      code[w] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
  }
  if (sc.div == DIV_ZERO) {
    // a zero scale (an E4M3 scale is 0 or at least 2^-9): codes 0 and values
    // +0, not the signs of the zero quotients; the terms above are already
    // right (d * 4s = 0)
    code[0] = code[1] = 0u;
#pragma unroll
    for (int j = 0; j < 8; j++) d[j] = (h2){(_Float16)0.0f, (_Float16)0.0f};
  }
  te = ee * 0.0625f;
  ts = ss * 0.0625f;
  // the output: the rotation of xhat back, or xhat itself
  float m = sc.s;
  if (unrotate) {
    butterflies16_h2(d);
    m = sc.s * 0.25f;
  }
#pragma unroll
  for (int j = 0; j < 8; j++) yw[j] = pack_bf16x2(mix_mul<0>(d[j], m, negzero), mix_mul<1>(d[j], m, negzero));
}

// One lane's block under two-level scaling (see above). h holds the
// butterflies of the block's inputs; it is left holding xhat, rotated back
// when `unrotate`, and the output words are packed from it.
template <int F>
__device__ __forceinline__ void h16_block_two(float* h, bool unrotate, const TScale& tl, uint32_t* code, Scale& sc,
                                              uint32_t* yw, float& te, float& ts) {
  constexpr bool kFp = !Fmt<F>::is_int;
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    h[i] = h[i] * 0.25f;                 // the forward rotation's 1/sqrt(16)
    am = fmaxf(am, fabsf(h[i]));
  }
  sc = scale_sym<F>(fabsf(tdivide<TL_FAST>(am, tl)), LQ_SCALE_E4M3);
  float ee = 0.0f, ss = 0.0f;
  uint32_t b[8];
  code[0] = code[1] = 0u;
  static_for<8>([&](auto j) __attribute__((always_inline)) {
    const float y0 = h[2 * j], y1 = h[2 * j + 1];
    float v0 = divide<kFp, DIVM_MARKSTEIN>(tdivide<TL_FAST>(y0, tl), sc, false, y0);
    float v1 = divide<kFp, DIVM_MARKSTEIN>(tdivide<TL_FAST>(y1, tl), sc, false, y1);
    float xh0, xh1;
    if constexpr (F == LQ_E2M1) {
      v0 = clampf(v0, -6.0f, 6.0f);
      v1 = clampf(v1, -6.0f, 6.0f);
      uint32_t& w = code[j / 4];
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v0, v1, 1.0f, j % 4);
      const auto d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, j % 4);
      xh0 = d[0] * sc.s;
      xh1 = d[1] * sc.s;
    } else {
      // round half to even and clamp by the magic-number sum, as in
      // h16_block; the +0 addend turns a -0 product into +0
      constexpr float kMagic = 12582912.0f;
      const float u0 = clampf(v0 + kMagic, kMagic - 8.0f, kMagic + 7.0f);
      const float u1 = clampf(v1 + kMagic, kMagic - 8.0f, kMagic + 7.0f);
      b[j] = (__float_as_uint(u1) << 4) | (__float_as_uint(u0) & 0xFu);
      xh0 = __builtin_fmaf(u0 - kMagic, sc.s, 0.0f);
      xh1 = __builtin_fmaf(u1 - kMagic, sc.s, 0.0f);
    }
    xh0 = xh0 * tl.s;
    xh1 = xh1 * tl.s;
    const float dd0 = y0 - xh0, dd1 = y1 - xh1;
    ee = __builtin_fmaf(dd0, dd0, ee);
    ss = __builtin_fmaf(y0, y0, ss);
    ee = __builtin_fmaf(dd1, dd1, ee);
    ss = __builtin_fmaf(y1, y1, ss);
    h[2 * j] = xh0;
    h[2 * j + 1] = xh1;
  });
  if constexpr (F != LQ_E2M1) {
#pragma unroll
    for (int w = 0; w < 2; w++) {
      const uint32_t lo = __builtin_amdgcn_perm(b[4 * w + 1], b[4 * w], 0x0c0c0400u);
      const uint32_t hi = __builtin_amdgcn_perm(b[4 * w + 3], b[4 * w + 2], 0x0c0c0400u);
      code[w] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
  }
  te = ee;
  ts = ss;
  if (sc.div == DIV_ZERO) {
    // a zero block scale: codes 0, xhat +0, the error is the signal
    code[0] = code[1] = 0u;
#pragma unroll
    for (int i = 0; i < 16; i++) h[i] = 0.0f;
    te = ss;
  }
  if (unrotate) {
    butterflies16(h);
#pragma unroll
    for (int i = 0; i < 16; i++) h[i] = h[i] * 0.25f;
  }
#pragma unroll
  for (int j = 0; j < 8; j++) yw[j] = pack_bf16x2(h[2 * j], h[2 * j + 1]);
}

// The kernels' body. TWO: two-level scaling, the tensor scale combined from
// the statistic pass's partials by every workgroup.
template <int F, bool TWO>
__device__ __forceinline__ void h16_body(const FastArgs& a) {
  constexpr int kWaves = kThreads / 64;
  __shared__ u32x4 sh[kWaves][kLxSlots];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  u32x4* s = sh[wave];
  const bool unrotate = a.unrotate != 0;
  const float negzero = __builtin_bit_cast(float, 0x80000000u);
  double acc_e = 0.0, acc_s = 0.0;
  uint32_t bad = 0, slow = 0;
  const int64_t w0 = (int64_t)blockIdx.x * kWaves + wave;
  const int64_t wstride = (int64_t)gridDim.x * kWaves;
  Raw<LQ_BF16> r;
  if (w0 < a.ntiles) lx_load(r, a.x, w0, lane);
  TScale tl;
  if constexpr (TWO) tl = tscale_from_stat<F, kThreads>(a);   // while the first loads are in flight
  else tl.s = tl.r = tl.sp = tl.p = 1.0f;
  wait_vmem_all();
  int k = 0;
  for (int64_t chunk = w0; chunk < a.ntiles; chunk += wstride, k++) {
    const Raw<LQ_BF16> cur = r;
    if (chunk + wstride < a.ntiles) lx_load(r, a.x, chunk + wstride, lane);
    // lane-contiguous units -> this lane's block of 16 consecutive elements
    const Raw<LQ_BF16> t = lx_gather(s, cur, lane);
    float h[16];
    raw_to_float<LQ_BF16>(t, h);
    butterflies16(h);
    uint32_t code[2], yw[8];
    Scale sc;
    float te, ts;
    if constexpr (TWO) h16_block_two<F>(h, unrotate, tl, code, sc, yw, te, ts);
    else h16_block<F>(h, unrotate, negzero, code, sc, yw, te, ts);
    // codes and the scale of block (chunk * 64 + lane) straight out
    gstore((u32x2*)(a.codes + chunk * 512 + 8 * lane), (u32x2){code[0], code[1]});
    ((uint8_t*)a.scales)[chunk * 64 + lane] = (uint8_t)sc.sbits;
    // the output words back to the lane-contiguous layout
    lx_store(s, a.y, chunk, lane, yw);
    if (sums_in_range(te, ts)) {
      acc_e += (double)te;
      acc_s += (double)ts;
    } else {
      slow |= 1u << k;
    }
  }
  if (__any(slow != 0u)) {
    // blocks of tiny, huge or non-finite values: their terms in fp64 by the
    // general path's arithmetic (block index chunk * 64 + lane)
    for (int j = 0; j < kFastMaxIters; j++) {
      const bool marked = ((slow >> j) & 1u) != 0u;
      if (!__any(marked)) continue;
      const int64_t chunk = w0 + (int64_t)j * wstride;
      if (chunk >= a.ntiles || !marked) continue;
      const int64_t tile = chunk * 64 + lane;
      Raw<LQ_BF16> raw;
      raw_load<LQ_BF16>(raw, a.x, tile << 4);
      float x[16];
      raw_to_float<LQ_BF16>(raw, x);
      bad += count_nonfinite(x);
      rot_forward<16>(x, Rot{16, 0.25f, 0u, false});
      const ArrX xs{x};
      constexpr int TL = TWO ? TL_FAST : TL_NONE;
      const Scale sc = TWO ? scale_sym<F>(fabsf(tdivide<TL_FAST>(tile_absmax_x(xs), tl)), LQ_SCALE_E4M3)
                           : scale_sym<F>(tile_absmax_x(xs), LQ_SCALE_E4M3);
      Codes c;
      YW<LQ_BF16> yw;
      float te, ts;
      fast_quant<F, LQ_BF16, LQ_SCALE_E4M3, true, false, TL>(xs, sc, c, yw, nullptr, te, ts, &tl);
      uint32_t rotated_bad = 0;   // the count is of the inputs (above), not of the rotated values
      tile_sums_f64<F, true>(xs, c, sc, acc_e, acc_s, rotated_bad, TWO ? tl.s : 1.0f);
    }
  }
  if (a.finish_inline) {
    qsnr_publish<kThreads>(a.ws, a.epoch, acc_e, acc_s, bad);
    qsnr_finish<kThreads>(a.ws, a.epoch, gridDim.x, a.res);
  } else {
    qsnr_partial_ws(a.ws, acc_e, acc_s, bad);
  }
}

template <int F>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(6))) k_h16(FastArgs a) {
  h16_body<F, false>(a);
}
// (two-level: the division by S and the fp32 xhat need more registers; the
// INT4 kernel spills at 5 or 6 waves per SIMD, and takes 103 VGPRs at 4)
template <int F>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) k_h16_two(FastArgs a) {
  h16_body<F, true>(a);
}

template <int F>
static hipError_t launch_h16(const FastArgs& a, int nwg, hipStream_t s) {
  if (g_plan) return plan_add(nwg, kThreads, "void lqd::k_h16<%d>(lqd::FastArgs)", F);
  hipLaunchKernelGGL((k_h16<F>), dim3(nwg), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}
template <int F>
static hipError_t launch_h16_two(const FastArgs& a, int nwg, hipStream_t s) {
  if (g_plan) return plan_add(nwg, kThreads, "void lqd::k_h16_two<%d>(lqd::FastArgs)", F);
  hipLaunchKernelGGL((k_h16_two<F>), dim3(nwg), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

void h16_kernels(fast_fn* k, fast_fn* two) {
  for (int f = 0; f < kFormats; f++) k[f] = two[f] = nullptr;
  k[LQ_INT4] = &launch_h16<LQ_INT4>;
  k[LQ_E2M1] = &launch_h16<LQ_E2M1>;
  two[LQ_INT4] = &launch_h16_two<LQ_INT4>;
  two[LQ_E2M1] = &launch_h16_two<LQ_E2M1>;
}

}  // namespace lqd
