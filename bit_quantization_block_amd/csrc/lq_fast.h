// lq_fast.h — specialised per-block fake-quant kernels for the common
// configuration: block scales computed from the data, round half to even,
// codes, scales (zeros), dequantized output and QSNR all produced. Format,
// scale format, zero point, input/output dtype and rotation are template
// parameters, so the tile loop is one straight-line path with few live
// registers; every other combination runs through k_flat.
//
// Two launch shapes:
//  - without rotation: 1024-thread workgroups (16 waves) at <= 64 VGPRs, so two
//    workgroups share a CU (8 waves per SIMD); the grid's last workgroup
//    collects the tagged partials of the others and writes the QSNR itself, so
//    the call is one kernel;
//  - with rotation (about 90 VGPRs): 256-thread workgroups, which keep 5 waves
//    per SIMD resident, and the one-workgroup k_finish after the kernel.
#pragma once
#include "lq_kernels.h"

namespace lqd {

struct FastArgs {
  const void* x;
  uint8_t* codes;
  void* scales;
  void* zeros;
  void* y;
  Workspace* ws;
  lq_result* res;
  uint32_t epoch;        // tag of this call's partials (never 0)
  int64_t ntiles;        // tiles of 16 elements (the element count is a multiple of the block)
  int32_t block_lanes;   // block / 16
  int32_t block_shift;   // log2(block_lanes)
  int32_t unrotate;      // rotation: write y back in the original domain
  int32_t stat_parts;    // per-tensor and two-level: k_stat partials to combine
  float* tscale;         // two-level: where S is stored (may be null)
  int32_t had;           // rotation size n (with HAD), its 1/sqrt(n), the random signs
  float rot_c;           // (one bit per column; may be null) and the columns of x
  const uint32_t* signs;
  int64_t cols;
  int32_t finish_inline;  // the kernel finishes the QSNR itself (tagged records, qsnr_finish)
  int32_t nwork;          // > 0: workgroups [0, nwork) do the work and publish their records; the
                          // grid's one further workgroup only collects them (qsnr_collect_only)
};

// Workgroups of the work (the grid without a collector of its own).
__device__ __forceinline__ int work_groups(const FastArgs& a) { return a.nwork > 0 ? a.nwork : (int)gridDim.x; }

__device__ __forceinline__ Rot rot_of(const FastArgs& a, int64_t e0) {
  return make_rot(a.had, a.rot_c, a.signs, e0, a.cols);
}

// Launch shapes of k_fast. Wide: 1024-thread workgroups at <= 64 VGPRs (two
// per CU, 8 waves per SIMD) whose last workgroup writes the QSNR itself, for
// 16-bit inputs without rotation when the grid covers the tensor in one pass
// (measured: the single kernel saves the finishing launch, about 2 us, but
// over several passes the coarse workgroups cost more than that). Narrow:
// 256-thread workgroups and the k_finish kernel after them, with the waves per
// SIMD that the register need leaves (fp32 raw tiles and their prefetch take
// 32 VGPRs, the rotation about 30 more).
// (FP6's bit-manipulation encoder and 6-bit packing do not fit the wide
// shape's 64 VGPRs without spilling: narrow only.)
constexpr bool fast_can_be_wide(int dt, bool had, int fmt) {
  return dt != LQ_F32 && !had && fmt != LQ_E2M3 && fmt != LQ_E3M2;
}
constexpr int fast_threads(bool wide) { return wide ? 1024 : 256; }
// Largest rotation k_fast takes: lane stages up to lane ^ 8. The two stages
// more that 512 and 1024 need cost 6 VGPRs, which took C4's rotated INT4
// kernel from 5 to 4 waves per SIMD; those sizes take k_fast_wrot.
constexpr int kFastMaxRot = 256;
// Waves per SIMD the kernels are compiled for (their VGPR budget). Rotating
// kernels with INT4 or FP6 codes get 3 (168 VGPRs): at 4 they spill. Measured
// on C4's tensor under signed rotations, one box: INT4 166.6 us (256 columns)
// and 199.2 us (1024) at 3 waves, against 170.7 / 193.4 us spilling 48 / 64
// bytes at 4; E2M1 fits 4 (164.8 / 186.7 us, 168.8 / 195.0 at 3). FP6
// kernels without rotation get 4 (a budget of 128 VGPRs): the native
// conversion's two 16-register operands do not fit the 80 VGPRs of 6; they
// take 84-97, which still leaves 5 waves per SIMD for most of them.
constexpr int fast_waves_per_simd(int dt, int fmt, bool had, bool wide) {
  return wide ? 8
         : had ? ((fmt == LQ_INT4 || fmt == LQ_E2M3 || fmt == LQ_E3M2) ? 3 : 4)
         : (dt == LQ_F32 || fmt == LQ_E2M3 || fmt == LQ_E3M2) ? 4
                                                               : 6;
}

// Wave-wide max as a wave-uniform value: DPP within each row of 16 lanes,
// then the four row results read out (no lane shuffles, whose address
// arithmetic the compiler would otherwise share with the kernel's final
// reductions and keep live across the main loop).
__device__ __forceinline__ float wave_max_uniform(float v) {
  v = group_max(v, 16);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Workgroup-wide max over NT threads (every thread gets it).
template <int NT>
__device__ __forceinline__ float block_max_nt(float v) {
  __shared__ float sh[NT / 64];
  v = wave_max_uniform(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = sh[0];
#pragma unroll
  for (int i = 1; i < NT / 64; i++) m = fmaxf(m, sh[i]);
  return m;
}

// Two-level: the tensor scale from k_stat's partials (every workgroup
// combines them; max does not depend on the order), stored by workgroup 0,
// returned in scalar registers.
template <int F, int NT>
__device__ __forceinline__ TScale tscale_from_stat(const FastArgs& a) {
  float am = 0.0f;
  for (int i = threadIdx.x; i < a.stat_parts; i += NT) am = fmaxf(am, a.ws->part_amax[i]);
  const float S = tensor_scale_of<F>(block_max_nt<NT>(am));
  if (a.tscale && blockIdx.x == 0 && threadIdx.x == 0) *a.tscale = S;
  return tscale_uniform(tscale_make(S));
}

// Codes and fp32 QSNR terms of one tile under its block scale; a zero stored
// scale gives code 0 and xhat = +0, so the error is the signal.
template <int F, int ODT, int SF, bool SYM, bool XH, int TL = TL_NONE, class X>
__device__ __forceinline__ void fast_quant(const X& xs, const Scale& sc, Codes& c, YW<ODT>& yw, float* xh,
                                           float& te, float& ts, const TScale* tl = nullptr) {
  using M = ModeC<SF == LQ_SCALE_UE8M0, SYM, false>;
  // only an fp32 scale can be so small that 1/s overflows; the scales here
  // come from the data, so the pre-scaled correction applies
  constexpr bool kTiny = SF == LQ_SCALE_F32;
  if (kTiny && sc.div == DIV_IEEE) quant_stream<F, ODT, XH, DIVM_PRESCALED, TL>(xs, sc, M{}, c, yw, xh, te, ts, tl);
  else quant_stream<F, ODT, XH, DIVM_MARKSTEIN, TL>(xs, sc, M{}, c, yw, xh, te, ts, tl);
  if (SF != LQ_SCALE_UE8M0 && sc.div == DIV_ZERO) {
#pragma unroll
    for (int j = 0; j < 4; j++) c.w[j] = 0u;
    te = ts;
  }
}

// Block scale of the tile's block (the lanes of a block reduce together).
// Two-level: the block's max|x| divided by S (the max of the quotients, as
// correctly rounded division is monotone) under an E4M3 scale.
template <int F, int SF, bool SYM, int TL = TL_NONE, class X>
__device__ __forceinline__ Scale fast_scale(const FastArgs& a, const X& xs, const TScale* tl = nullptr) {
  if constexpr (TL != TL_NONE) {
    return scale_sym<F>(fabsf(tdivide<TL>(group_max(tile_absmax_x(xs), a.block_lanes), *tl)), SF);
  } else if constexpr (SYM) {
    return scale_sym<F>(group_max(tile_absmax_x(xs), a.block_lanes), SF);
  } else {
    float mn = xs(0), mx = xs(0);
#pragma unroll
    for (int i = 1; i < 16; i++) { mn = fminf(mn, xs(i)); mx = fmaxf(mx, xs(i)); }
    return scale_asym<F>(group_min(mn, a.block_lanes), group_max(mx, a.block_lanes), SF, LQ_RNE);
  }
}

// The fp32 tile sums are used when both lie in [2^-100, inf); otherwise
// (tiny, huge or non-finite values) the tile is summed again in fp64.
__device__ __forceinline__ bool sums_in_range(float te, float ts) {
  const float lo = 0x1p-100f, hi = __builtin_inff();
  return te >= lo && te < hi && ts >= lo && ts < hi;
}

// ---- lane-contiguous access of a wave's 64 tiles (one chunk of 1024
// elements) for bf16 inputs and outputs. Lane L loads the chunk's 16-byte
// units L and 64 + L, so each load instruction covers 1 KB of whole cache
// lines, and the units are exchanged through LDS so that lane L holds its
// tile (units 2L and 2L + 1, elements 16L .. 16L + 15); the dequantized words
// go back the same way before the store. A lane reading its own 16 elements
// makes every instruction touch twice the lines, half of each: measured on
// C4's traffic 119.6 us that way, 108.0 us through LDS, 108.1 us for the
// lane-contiguous pattern itself.
// LDS slot of unit u: u/2 (u even) or kOddSlot + u/2 (u odd). Lane L's tile
// units then sit at slots L and kOddSlot + L, and the units L and 64 + L of a
// lane-contiguous access spread over both halves; the 8-slot gap puts the two
// halves in different LDS banks.
constexpr int kOddSlot = 72;
constexpr int kLxSlots = kOddSlot + 64;

__device__ __forceinline__ int unit_slot(int u) { return (u & 1) ? kOddSlot + (u >> 1) : (u >> 1); }

// lane L's two lane-contiguous units of chunk c
__device__ __forceinline__ void lx_load(Raw<LQ_BF16>& r, const void* x, int64_t c, int lane) {
  const char* p = (const char*)x + (c * 1024 + 8 * lane) * 2;
  r.w[0] = gload((const u32x4*)p);
  r.w[1] = gload((const u32x4*)(p + 1024));
}

// lane-contiguous units -> this lane's tile (s: the wave's kLxSlots slots)
__device__ __forceinline__ Raw<LQ_BF16> lx_gather(u32x4* s, const Raw<LQ_BF16>& r, int lane) {
  s[unit_slot(lane)] = r.w[0];
  s[unit_slot(64 + lane)] = r.w[1];
  Raw<LQ_BF16> t;
  t.w[0] = s[lane];
  t.w[1] = s[kOddSlot + lane];
  return t;
}

// this lane's 8 output words (its tile) -> lane-contiguous stores of chunk c
__device__ __forceinline__ void lx_store(u32x4* s, void* y, int64_t c, int lane, const uint32_t* w) {
  s[lane] = (u32x4){w[0], w[1], w[2], w[3]};
  s[kOddSlot + lane] = (u32x4){w[4], w[5], w[6], w[7]};
  const u32x4 ya = s[unit_slot(lane)], yb = s[unit_slot(64 + lane)];
  u32x4* q = (u32x4*)((char*)y + (c * 1024 + 8 * lane) * 2);
  gstore(q, ya);
  gstore(q + 64, yb);
}

// The exchange state of one wave: on when the wave's current chunk is whole
// (the same for all its lanes), then outputs go through s.
struct Lx {
  u32x4* s;
  int lane;
  bool on;
};

// Rotating kernels that take the largest compiled rotation size straight
// through (see rot_stages): bf16 inputs, 4- and 8-bit codes, one level of
// scales. The others are near their register budget without the second copy
// of the lane stages. Measured on C4's tensor under the 256-column rotation
// (NVFP4 / NVINT4 with random signs): SQ_INSTS_VALU 844 per 16-element tile
// with the branches.
template <int DT, int F, int TL>
constexpr bool kStraight = DT == LQ_BF16 && !Fmt<F>::six && TL == TL_NONE;

// One tile: scale, codes, dequantized values, stores. Returns false when the
// tile's sums must be redone in fp64 (nothing was added then).
template <int DT, int F, int ODT, int SF, bool SYM, bool HAD, int TL, int RMAX, class X>
__device__ __forceinline__ bool fast_tile(const FastArgs& a, int64_t t, const X& xs, double& acc_e, double& acc_s,
                                          const TScale& tl, const Lx& lx, const Rot& rot) {
  const Scale sc = fast_scale<F, SF, SYM, TL>(a, xs, &tl);
  const int64_t bidx = t >> a.block_shift;
  if ((threadIdx.x & (a.block_lanes - 1)) == 0) scale_store(a.scales, a.zeros, bidx, sc, SF, SYM);
  Codes c;
  YW<ODT> yw;
  float te, ts;
  const bool zero = SF != LQ_SCALE_UE8M0 && sc.div == DIV_ZERO;
  if (HAD && a.unrotate) {
    float xh[16];
    fast_quant<F, ODT, SF, SYM, true, TL>(xs, sc, c, yw, xh, te, ts, &tl);
    if (zero) {
#pragma unroll
      for (int i = 0; i < 16; i++) xh[i] = 0.0f;
    }
    // the sign masks are rebuilt from the bits rather than kept in 16
    // registers across the quantization (the empty asm hides that they are
    // the forward rotation's)
    Rot back = rot;
    asm volatile("" : "+v"(back.sbits));
    rot_inverse<RMAX, kStraight<DT, F, TL>>(xh, back);
#pragma unroll
    for (int i = 0; i < 16; i += 2) put_y<ODT>(yw, i, xh[i], xh[i + 1]);
  } else {
    fast_quant<F, ODT, SF, SYM, false, TL>(xs, sc, c, yw, nullptr, te, ts, &tl);
    if (zero) {
#pragma unroll
      for (int i = 0; i < (ODT == LQ_F32 ? 16 : 8); i++) yw.w[i] = 0u;
    }
  }
  const int64_t e0 = t << 4;
  store_codes<F>(a.codes, e0, 16, c);
  if constexpr (ODT == LQ_BF16) {
    if (lx.on) lx_store(lx.s, a.y, t >> 6, lx.lane, yw.w);
    else store_yw<ODT>(a.y, e0, 16, yw);
  } else {
    store_yw<ODT>(a.y, e0, 16, yw);
  }
  if (!sums_in_range(te, ts)) return false;
  acc_e += (double)te;
  acc_s += (double)ts;
  return true;
}

// fp64 QSNR terms of one tile from its values and codes (the oracle's
// arithmetic: the difference of the two values and the squares taken in fp64;
// xhat as the quantizer forms it), one element at a time: a rare path, kept
// from raising the kernel's register count.
// tls: the two-level tensor scale S that multiplies xhat (1 without one).
template <int F, bool SYM, class X>
__device__ __forceinline__ void tile_sums_f64(const X& xs, const Codes& c, const Scale& sc, double& acc_e,
                                              double& acc_s, uint32_t& bad, float tls = 1.0f) {
  float d[16];
  decode_tile<F>(c, d);
  const bool zero = sc.div == DIV_ZERO;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const float x = xs(i);
    const float xh = zero ? 0.0f : (SYM ? d[i] * sc.s : sc.s * (d[i] - sc.zp)) * tls;
    const double e = (double)x - (double)xh;
    acc_e += e * e;
    acc_s += (double)x * (double)x;
    bad += ((__float_as_uint(x) & 0x7F800000u) == 0x7F800000u) ? 1u : 0u;
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Iterations of the tile loop per lane that the record of out-of-range tiles
// covers (one bit each); the host sends larger tensors to k_flat.
constexpr int kFastMaxIters = 32;

// Tiles whose fp32 sums left the range are summed after the main loop, when
// its registers are free: bit k of `slow` marks this lane's tile of iteration
// k. Each such tile is read again and its scale and codes recomputed with the
// same arithmetic (the lanes of a block take every step together, as in the
// loop); a lane adds the fp64 terms of its own marked tiles only, and counts
// their non-finite inputs (only such tiles can hold any). With rotation the
// terms are of the rotated values and the count is of the inputs.
template <int DT, int F, int SF, bool SYM, bool HAD, int TL, int RMAX>
__device__ void fast_redo(const FastArgs& a, int64_t t0, int64_t stride, uint32_t slow, double& acc_e,
                          double& acc_s, uint32_t& bad, const TScale& tl) {
  const float tls = TL != TL_NONE ? tl.s : 1.0f;
  for (int k = 0; k < kFastMaxIters; k++) {
    const bool marked = ((slow >> k) & 1u) != 0u;
    if (!__any(marked)) continue;
    const int64_t t = t0 + (int64_t)k * stride;
    if (t >= a.ntiles) continue;
    Raw<DT> r;
    raw_load<DT>(r, a.x, t << 4);
    Codes c;
    YW<DT> yw;
    float te, ts;
    if constexpr (HAD) {
      float x[16];
      raw_to_float<DT>(r, x);
      const uint32_t b = count_nonfinite(x);
      rot_forward<RMAX>(x, rot_of(a, t << 4));
      const ArrX xs{x};
      const Scale sc = fast_scale<F, SF, SYM, TL>(a, xs, &tl);
      fast_quant<F, DT, SF, SYM, false, TL>(xs, sc, c, yw, nullptr, te, ts, &tl);
      if (marked) {
        uint32_t unused = 0;
        tile_sums_f64<F, SYM>(xs, c, sc, acc_e, acc_s, unused, tls);
        bad += b;
      }
    } else {
      const RawX<DT> xs{r};
      const Scale sc = fast_scale<F, SF, SYM, TL>(a, xs, &tl);
      fast_quant<F, DT, SF, SYM, false, TL>(xs, sc, c, yw, nullptr, te, ts, &tl);
      if (marked) tile_sums_f64<F, SYM>(xs, c, sc, acc_e, acc_s, bad, tls);
    }
  }
}

template <int DT, int F, int ODT, int SF, bool SYM, bool HAD, int TL, int RMAX>
__device__ __forceinline__ bool fast_body(const FastArgs& a, int64_t t, const Raw<DT>& cur, double& acc_e,
                                          double& acc_s, const TScale& tl, const Lx& lx, const Rot& rot) {
  if constexpr (HAD) {
    float x[16];
    raw_to_float<DT>(cur, x);
    // the lane's sign bits are the same every pass: the empty asm keeps the
    // compiler from hoisting their 16 masks out of the loop into registers
    Rot fwd = rot;
    asm volatile("" : "+v"(fwd.sbits));
    rot_forward<RMAX, kStraight<DT, F, TL>>(x, fwd);
    return fast_tile<DT, F, ODT, SF, SYM, HAD, TL, RMAX>(a, t, ArrX{x}, acc_e, acc_s, tl, lx, rot);
  } else {
    return fast_tile<DT, F, ODT, SF, SYM, HAD, TL, RMAX>(a, t, RawX<DT>{cur}, acc_e, acc_s, tl, lx, rot);
  }
}

// TWO: two-level scaling (E4M3 block scales, symmetric) under the tensor
// scale that every workgroup combines from k_stat's partials. RMAX: the
// largest rotation the lane stages are compiled for.
template <int DT, int F, int ODT, int SF, bool SYM, bool HAD, bool WIDE, bool TWO, int RMAX>
__device__ __forceinline__ void fast_kernel_body(const FastArgs& a) {
  constexpr int NT = fast_threads(WIDE);
  constexpr int TL = TWO ? TL_FAST : TL_NONE;
  static_assert(!TWO || (SF == LQ_SCALE_E4M3 && SYM), "two-level scaling has symmetric E4M3 block scales");
  double acc_e = 0.0, acc_s = 0.0;
  uint32_t bad = 0, slow = 0;
  const int64_t stride = (int64_t)gridDim.x * NT;
  const int64_t t0 = (int64_t)blockIdx.x * NT + threadIdx.x;
  // bf16 in and out: whole chunks (a wave's 64 tiles, from a 64-aligned
  // start) are loaded lane-contiguously and exchanged through LDS; a partial
  // last chunk is read tile by tile. Not in the wide shape (held to 64 VGPRs)
  // nor for FP6 codes: the exchange's registers make those spill. Not under a
  // rotation either: those kernels are bound by their arithmetic, and on one
  // box the 256-point NVFP4 / NVINT4 calls on C4's tensor took 185 / 199 us
  // with the exchange against 171 / 177 us without (C3's INT4 group-128
  // zero-point call: 41.4-42.0 us with, 44.4 us without).
  constexpr bool LX = DT == LQ_BF16 && ODT == LQ_BF16 && !WIDE && !Fmt<F>::six && !HAD;
  __shared__ u32x4 lx_sh[LX ? NT / 64 : 1][LX ? kLxSlots : 1];
  Lx lx;
  lx.lane = threadIdx.x & 63;
  lx.s = lx_sh[LX ? (threadIdx.x >> 6) : 0];
  lx.on = false;
  const int64_t whole = LX ? (a.ntiles & ~(int64_t)63) : 0;   // tiles of whole chunks
  auto load = [&](Raw<DT>& r, int64_t t) __attribute__((always_inline)) {
    if constexpr (LX) {
      if (t < whole) {
        lx_load(r, a.x, t >> 6, lx.lane);
        return;
      }
    }
    raw_load<DT>(r, a.x, t << 4);
  };
  // rotation signs: the host gives a signed rotation a grid that covers the
  // tensor in one pass or whose stride is a multiple of cols, so all of a
  // lane's tiles sit at one column and its 16 sign bits are read once, here.
  // (Read per tile, after the prefetch, they made every pass wait for all
  // loads in flight and cost a 64-bit remainder: 25-35 us of a 170-178 us
  // 256-point call on C4's tensor.)
  const bool has_signs = HAD && a.signs != nullptr;
  uint32_t sb = 0;
  if (has_signs && t0 < a.ntiles) sb = rot_signs(a.signs, (t0 << 4) % a.cols);
  const Rot rot{a.had, a.rot_c, sb, has_signs};
  // software pipeline: the next tile's loads are issued as soon as this
  // tile's registers are copied; lanes past the end load nothing (rather than
  // all re-reading one tile, a hot spot in one L2 channel)
  Raw<DT> r;
  if (t0 < a.ntiles) load(r, t0);
  TScale tl;
  if constexpr (TWO) tl = tscale_from_stat<F, NT>(a);   // while the first loads are in flight
  else tl.s = tl.r = tl.sp = tl.p = 1.0f;
  wait_vmem_all();
  int k = 0;
  for (int64_t t = t0; t < a.ntiles; t += stride, k++) {
    Raw<DT> cur = r;
    const int64_t tn = t + stride;
    if (tn < a.ntiles) load(r, tn);
    if constexpr (LX) {
      lx.on = __builtin_amdgcn_readfirstlane(t < whole ? 1 : 0) != 0;
      if (lx.on) cur = lx_gather(lx.s, cur, lx.lane);
    }
    if (!fast_body<DT, F, ODT, SF, SYM, HAD, TL, RMAX>(a, t, cur, acc_e, acc_s, tl, lx, rot)) slow |= 1u << k;
  }
  if (__any(slow != 0u)) fast_redo<DT, F, SF, SYM, HAD, TL, RMAX>(a, t0, stride, slow, acc_e, acc_s, bad, tl);
  if (WIDE || a.finish_inline) {
    qsnr_publish<NT>(a.ws, a.epoch, acc_e, acc_s, bad);
    qsnr_finish<NT>(a.ws, a.epoch, gridDim.x, a.res);
  } else {
    qsnr_partial_ws(a.ws, acc_e, acc_s, bad);
  }
}

template <int DT, int F, int ODT, int SF, bool SYM, bool HAD, bool WIDE, bool TWO = false>
__global__ void __launch_bounds__(fast_threads(WIDE))
    __attribute__((amdgpu_waves_per_eu(fast_waves_per_simd(DT, F, HAD, WIDE)))) k_fast(FastArgs a) {
  fast_kernel_body<DT, F, ODT, SF, SYM, HAD, WIDE, TWO, kFastMaxRot>(a);
}

// The same with the lane stages of 512- and 1024-column rotations compiled
// in (narrow, rotation only): a separate kernel, so the 16..256 ones keep
// their registers.
template <int DT, int F, int ODT, int SF, bool SYM, bool TWO = false>
__global__ void __launch_bounds__(fast_threads(false))
    __attribute__((amdgpu_waves_per_eu(fast_waves_per_simd(DT, F, true, false)))) k_fast_wrot(FastArgs a) {
  fast_kernel_body<DT, F, ODT, SF, SYM, true, false, TWO, 1024>(a);
}

// ---- 2-D tiles (walkerchi.com playbook §4.4, DeepSeek-V3 per-tile scaling):
// the specialised path for symmetric scales from the data, round half to
// even, every output in the input dtype, no rotation. A workgroup owns a
// tile of tile_rows x tile_cols elements (the last band of rows may be
// shorter). The tile is read as groups of 8 consecutive elements (16 bytes
// of bf16), consecutive lanes taking consecutive groups of a tile row, so
// each 16-byte load or store instruction covers whole rows of the tile; a
// lane pairs two such groups into one 16-element unit (first 8 elements:
// group tid + 512k, last 8: group tid + 512k + 256), and its NCH units stay
// in raw input registers between the tile's max|x| and the quantization.
// Measured on 128x128 bf16 E4M3 tiles of an 11008x4096 tensor: 49.5 us per
// call in this layout (164 VGPRs, 3 waves per SIMD; capping it at 128 spills),
// 55 us with one 16-element run per lane (each load instruction then touches
// twice the cache lines, half each), 62 us with the next tile double-buffered
// in registers, 81-85 us in the general group kernel (k_row).

template <int DT>
__device__ __forceinline__ void group_load(u32x4* w, const void* x, int64_t e) {
  const u32x4* p = (const u32x4*)((const char*)x + e * (DT == LQ_F32 ? 4 : 2));
  w[0] = gload(p);
  if constexpr (DT == LQ_F32) w[1] = gload(p + 1);
}

// Codes and outputs of 8 elements (half h of a unit) at element e.
template <int DT, int F>
__device__ __forceinline__ void group_store(const Args& a, int64_t e, int h, const Codes& c, const YW<DT>& yw) {
  if constexpr (Fmt<F>::four) {
    gstore((uint32_t*)(a.codes + e / 2), c.w[h]);
  } else {
    gstore((u32x2*)(a.codes + e), (u32x2){c.w[2 * h], c.w[2 * h + 1]});
  }
  if constexpr (DT == LQ_F32) {
    u32x4* q = (u32x4*)((char*)a.y + e * 4);
    gstore(q, (u32x4){yw.w[8 * h], yw.w[8 * h + 1], yw.w[8 * h + 2], yw.w[8 * h + 3]});
    gstore(q + 1, (u32x4){yw.w[8 * h + 4], yw.w[8 * h + 5], yw.w[8 * h + 6], yw.w[8 * h + 7]});
  } else {
    gstore((u32x4*)((char*)a.y + e * 2), (u32x4){yw.w[4 * h], yw.w[4 * h + 1], yw.w[4 * h + 2], yw.w[4 * h + 3]});
  }
}

template <int DT, int F, int SF, int NCH>
__global__ void __launch_bounds__(kThreads) k_tile(Args a) {
  constexpr int kHalf = DT == LQ_F32 ? 2 : 1;            // 16-byte words per group of 8
  __shared__ float sh[4];
  const int tid = threadIdx.x;
  const int64_t seg = a.tile_cols;
  const int gshift = a.unit_shift + 1;                   // log2(groups of 8 per tile row)
  const int64_t tpb = a.cols / seg;                      // tiles per band of rows
  const int64_t ngroups = (a.rows + a.tile_rows - 1) / a.tile_rows * tpb;
  double acc_e = 0.0, acc_s = 0.0;
  uint32_t bad = 0;
  for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
    const int64_t band = g / tpb;
    const int64_t row0 = band * a.tile_rows;
    const int64_t col0 = (g - band * tpb) * seg;
    const int64_t nseg = a.rows - row0 < a.tile_rows ? a.rows - row0 : a.tile_rows;
    // group j of this lane (j = 2k + h): row lrow + j * jrows of the tile,
    // the same 8 columns (a tile row holds 2..32 groups, which divide the 256
    // lanes); one base element and a constant row stride
    const int lrow = tid >> gshift;
    const int jrows = kThreads >> gshift;
    const int64_t base = (row0 + lrow) * a.cols + col0 + ((tid & ((1 << gshift) - 1)) << 3);
    const int64_t jstride = (int64_t)jrows * a.cols;
    auto valid = [&](int j) __attribute__((always_inline)) { return lrow + j * jrows < nseg; };
    Raw<DT> r[NCH];
    float am = 0.0f;
    static_for<NCH>([&](auto k) __attribute__((always_inline)) {
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int j = 2 * k + h;
        if (valid(j)) {
          group_load<DT>(&r[k].w[h * kHalf], a.x, base + j * jstride);
        } else {
#pragma unroll
          for (int i = 0; i < kHalf; i++) r[k].w[h * kHalf + i] = (u32x4){0u, 0u, 0u, 0u};
        }
      }
      am = fmaxf(am, tile_absmax_x(RawX<DT>{r[k]}));
    });
    const Scale sc = scale_sym<F>(block_reduce_max(am, sh), SF);
    if (tid == 0) scale_store(a.scales, a.zeros, g, sc, SF, true);
    const bool zero = SF != LQ_SCALE_UE8M0 && sc.div == DIV_ZERO;
    static_for<NCH>([&](auto k) __attribute__((always_inline)) {
      if (valid(2 * k)) {
        const RawX<DT> xs{r[k]};
        Codes c;
        YW<DT> yw;
        float te, ts;
        fast_quant<F, DT, SF, true, false>(xs, sc, c, yw, nullptr, te, ts);
        if (zero) {
#pragma unroll
          for (int i = 0; i < (DT == LQ_F32 ? 16 : 8); i++) yw.w[i] = 0u;
        }
        group_store<DT, F>(a, base + (2 * k) * jstride, 0, c, yw);
        if (valid(2 * k + 1)) group_store<DT, F>(a, base + (2 * k + 1) * jstride, 1, c, yw);
        // a missing second group is zeros: it adds nothing to either sum
        if (sums_in_range(te, ts)) {
          acc_e += (double)te;
          acc_s += (double)ts;
        } else {
          tile_sums_f64<F, true>(xs, c, sc, acc_e, acc_s, bad);
        }
      }
    });
  }
  if (a.finish_inline) {
    qsnr_publish<kThreads>(a.ws, a.epoch, acc_e, acc_s, bad);
    qsnr_finish<kThreads>(a.ws, a.epoch, gridDim.x, a.res);
  } else {
    qsnr_partial(a, acc_e, acc_s, bad);
  }
}

template <int DT, int F, int SF, int NCH>
hipError_t launch_tile(const Args& a, int nwg, hipStream_t s) {
  if (g_plan) return plan_add(nwg, kThreads, "void lqd::k_tile<%d, %d, %d, %d>(lqd::Args)", DT, F, SF, NCH);
  hipLaunchKernelGGL((k_tile<DT, F, SF, NCH>), dim3(nwg), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int DT, int F, int ODT, int SF, bool SYM, bool HAD, bool WIDE, bool TWO = false>
hipError_t launch_fast(const FastArgs& a, int nwg, hipStream_t s) {
  if (g_plan)
    return plan_add(nwg, fast_threads(WIDE), "void lqd::k_fast<%d, %d, %d, %d, %s, %s, %s, %s>(lqd::FastArgs)", DT, F, ODT, SF, tf(SYM),
                    tf(HAD), tf(WIDE), tf(TWO));
  hipLaunchKernelGGL((k_fast<DT, F, ODT, SF, SYM, HAD, WIDE, TWO>), dim3(nwg), dim3(fast_threads(WIDE)), 0, s, a);
  return hipGetLastError();
}

template <int DT, int F, int ODT, int SF, bool SYM, bool TWO = false>
hipError_t launch_fast_wrot(const FastArgs& a, int nwg, hipStream_t s) {
  if (g_plan)
    return plan_add(nwg, fast_threads(false), "void lqd::k_fast_wrot<%d, %d, %d, %d, %s, %s>(lqd::FastArgs)", DT, F, ODT, SF, tf(SYM),
                    tf(TWO));
  hipLaunchKernelGGL((k_fast_wrot<DT, F, ODT, SF, SYM, TWO>), dim3(nwg), dim3(fast_threads(false)), 0, s, a);
  return hipGetLastError();
}

typedef hipError_t (*fast_fn)(const FastArgs&, int, hipStream_t);

// k: [format][scale format][asymmetric][rotation][wide];
// two: two-level (E4M3 block scales, symmetric) [format][rotation][wide];
// wrot: rotations of 512 and 1024 columns [format][scale format], and
// two-level under them, wrot_two[format]
struct FastSet {
  fast_fn k[kFormats][4][2][2][2];
  fast_fn two[kFormats][2][2];
  fast_fn wrot[kFormats][4];
  fast_fn wrot_two[kFormats];
  flat_fn tile[kFormats][4][3];   // 2-D tiles: [format][scale format][1, 2 or 4 units per lane]
};

// Lane-contiguous kernels (lq_lc.hip: bf16 in and out, symmetric scales, no
// rotation, element count a multiple of 1024): [format][scale format]
// [per-tensor][wide]. Their FastArgs carry chunks of 1024 elements in
// `ntiles`, block / 8 in `block_lanes` and log2(block) in `block_shift`
// (per-block and two-level), and k_stat's partial count in `stat_parts`
// (per-tensor and two-level).
// FP6 has none of these (6-bit codes of 8 elements are not 16-byte pieces).
struct LcSet {
  fast_fn k[kFormats][4][2][2];
  fast_fn row[kFormats][4];   // per-channel, symmetric: [format][scale format]
  fast_fn two[kFormats][2];   // two-level, E4M3 block scales: [format][wide]
};
void lc_kernels(LcSet& k);

// 4-bit blocks of 16 with E4M3 scales under the 16-point rotation without
// signs (lq_h16.hip: bf16 in and out, element count a multiple of 1024),
// [format]; FastArgs as the lane-contiguous kernels' (chunks of 1024 in
// `ntiles`).
void h16_kernels(fast_fn* k, fast_fn* two);

}  // namespace lqd
