// lq_lc.hip — the specialised per-block kernels for bf16 input and output
// without rotation, in the lane-contiguous layout.
//
// A wave takes 1024 consecutive elements (a chunk): lane L holds elements
// 8L..8L+7 (half A) and 512+8L..512+8L+7 (half B). Every 16-byte load and
// store instruction then covers 1 KB of consecutive bytes (512 B for 8-bit
// codes, 256 B for 4-bit codes), whole cache lines, where a lane owning 16
// consecutive elements makes each instruction touch twice as many lines half
// each (measured on the C2 memory pattern: 30.0 us against 33.5 us). A block
// of B elements is B/8 neighbouring lanes inside one half (B divides 512), so
// a lane computes two block scales, one per half, and quantizes each group of
// 8 under its own. Used for symmetric scales when the element count is a
// multiple of 1024; other shapes and zero-point variants take k_fast / k_flat
// (a zero point makes the scale computation the larger part of the work, and
// two per lane measured slower than the strided layout's one). FP6 codes: a
// half's eight are 48 bits, bytes 6L..6L+5 of the half's 384, written as a
// dword and a short (even lanes dword first, odd lanes short first, so both
// are naturally aligned).
#include "lq_fast.h"

namespace lqd {

// Scales of k_lc: per block, one per tensor (fp32, from k_stat's partials),
// or two-level (E4M3 block scales of the values divided by the tensor scale).
constexpr int LC_BLOCK = 0, LC_TENSOR = 1, LC_TWO = 2;

// Tile of one lane in one chunk: element i < 8 is half A's i, i >= 8 is half
// B's i - 8; the two 16-byte loads fill Raw words 0-3 and 4-7.
__device__ __forceinline__ void lc_load(Raw<LQ_BF16>& r, const void* x, int64_t chunk, int lane) {
  const char* p = (const char*)x + (chunk * 1024 + 8 * lane) * 2;
  r.w[0] = gload((const u32x4*)p);
  r.w[1] = gload((const u32x4*)(p + 1024));
}

// Codes of a lane's two halves in one chunk (1024 elements): 8-bit codes 8
// bytes per half, 4-bit codes 4, 6-bit codes 6 (a dword and a short at
// naturally aligned addresses, in the element order of the whole stream).
template <int F>
__device__ __forceinline__ void lc_store_codes(uint8_t* codes, int64_t chunk, int lane, const Codes& c) {
  if constexpr (Fmt<F>::six) {
    uint8_t* p = codes + chunk * 768 + 6 * lane;
    const uint64_t ha = (uint64_t)c.w[0] | ((uint64_t)(c.w[1] & 0xFFFFu) << 32);
    const uint64_t hb = (uint64_t)(c.w[1] >> 16) | ((uint64_t)c.w[2] << 16);
    const bool odd = (lane & 1) != 0;
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const uint64_t v = h == 0 ? ha : hb;
      uint8_t* q = p + 384 * h;                                 // 512 elements on: 384 bytes
      gstore((uint32_t*)(q + (odd ? 2 : 0)), (uint32_t)(odd ? v >> 16 : v));
      gstore((uint16_t*)(q + (odd ? 0 : 4)), (uint16_t)(odd ? v : v >> 32));
    }
  } else if constexpr (Fmt<F>::four) {
    uint32_t* p = (uint32_t*)(codes + (chunk * 1024 + 8 * lane) / 2);
    gstore(p, c.w[0]);
    gstore(p + 64, c.w[1]);                       // 512 elements on: 256 bytes
  } else {
    u32x2* p = (u32x2*)(codes + chunk * 1024 + 8 * lane);
    gstore(p, (u32x2){c.w[0], c.w[1]});
    gstore(p + 64, (u32x2){c.w[2], c.w[3]});      // 512 bytes on
  }
}

// Block scales of the two halves (lanes of a block reduce together).
// Two-level: of each block's max|x| divided by S (the max of the quotients,
// as correctly rounded division is monotone).
template <int F, int SF, int TL, class X>
__device__ __forceinline__ void lc_scales(const FastArgs& a, const X& xs, Scale& sa, Scale& sb, const TScale& tl) {
  float ma = 0.0f, mb = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    ma = fmaxf(ma, fabsf(xs(i)));
    mb = fmaxf(mb, fabsf(xs(8 + i)));
  }
  group2<true>(ma, mb, a.block_lanes);
  if constexpr (TL != TL_NONE) {
    ma = fabsf(tdivide<TL>(ma, tl));   // a zero quotient as +0
    mb = fabsf(tdivide<TL>(mb, tl));
  }
  sa = scale_sym<F>(ma, SF);
  sb = scale_sym<F>(mb, SF);
}

// Codes and fp32 QSNR terms of a lane's two groups, each under its half's
// scale; a zero stored scale gives codes 0 and xhat = +0 for its group (the
// group's error is then its signal, and YW words are cleared by the caller).
template <int F, int SF, int TL, class X>
__device__ __forceinline__ void lc_quant(const X& xs, const Scale& sa, const Scale& sb, Codes& c, YW<LQ_BF16>& yw,
                                         float& te, float& ts, const TScale* tl = nullptr) {
  using M = ModeC<SF == LQ_SCALE_UE8M0, true, false>;
  // only an fp32 scale can make 1/s overflow; scales from the data allow the
  // pre-scaled correction there. Each group takes the mode its own scale needs.
  constexpr bool kTiny = SF == LQ_SCALE_F32;
  float ea = 0.0f, sa_ = 0.0f, eb = 0.0f, sb_ = 0.0f;
  if constexpr (Fmt<F>::six && LQ_NATIVE_FP6) {
    float v[16];
    if (kTiny && sa.div == DIV_IEEE) six_quotients<0, F, DIVM_PRESCALED, TL>(xs, sa, M{}, v, tl);
    else six_quotients<0, F, DIVM_MARKSTEIN, TL>(xs, sa, M{}, v, tl);
    if (kTiny && sb.div == DIV_IEEE) six_quotients<1, F, DIVM_PRESCALED, TL>(xs, sb, M{}, v, tl);
    else six_quotients<1, F, DIVM_MARKSTEIN, TL>(xs, sb, M{}, v, tl);
    six_finish<F, LQ_BF16, false, TL>(xs, v, sa, sb, c, yw, nullptr, ea, sa_, eb, sb_, tl);
  } else {
    if (kTiny && sa.div == DIV_IEEE)
      quant_group<0, F, LQ_BF16, false, DIVM_PRESCALED, TL>(xs, sa, M{}, c, yw, nullptr, ea, sa_, tl);
    else
      quant_group<0, F, LQ_BF16, false, DIVM_MARKSTEIN, TL>(xs, sa, M{}, c, yw, nullptr, ea, sa_, tl);
    if (kTiny && sb.div == DIV_IEEE)
      quant_group<1, F, LQ_BF16, false, DIVM_PRESCALED, TL>(xs, sb, M{}, c, yw, nullptr, eb, sb_, tl);
    else
      quant_group<1, F, LQ_BF16, false, DIVM_MARKSTEIN, TL>(xs, sb, M{}, c, yw, nullptr, eb, sb_, tl);
  }
  if (SF != LQ_SCALE_UE8M0) {
    if (sa.div == DIV_ZERO) {
      if (Fmt<F>::four) c.w[0] = 0u;
      else if (Fmt<F>::six) { c.w[0] = 0u; c.w[1] &= 0xFFFF0000u; }
      else c.w[0] = c.w[1] = 0u;
#pragma unroll
      for (int i = 0; i < 4; i++) yw.w[i] = 0u;
      ea = sa_;
    }
    if (sb.div == DIV_ZERO) {
      if (Fmt<F>::four) c.w[1] = 0u;
      else if (Fmt<F>::six) { c.w[1] &= 0xFFFFu; c.w[2] = 0u; }
      else c.w[2] = c.w[3] = 0u;
#pragma unroll
      for (int i = 4; i < 8; i++) yw.w[i] = 0u;
      eb = sb_;
    }
  }
  te = ea + eb;
  ts = sa_ + sb_;
}

// One lane's tile of one chunk: scales, codes, dequantized values, stores.
// Returns false when its sums must be redone in fp64 (nothing added then).
template <int F, int SF, int MODE>
__device__ __forceinline__ bool lc_tile(const FastArgs& a, int64_t chunk, int lane, const Raw<LQ_BF16>& r,
                                        const Scale& tsc, const TScale& tl, double& acc_e, double& acc_s) {
  constexpr int TL = MODE == LC_TWO ? TL_FAST : TL_NONE;
  const RawX<LQ_BF16> xs{r};
  Scale sa, sb;
  const int64_t e0 = chunk * 1024 + 8 * lane;
  if constexpr (MODE == LC_TENSOR) {
    sa = tsc;
    sb = tsc;
  } else {
    lc_scales<F, SF, TL>(a, xs, sa, sb, tl);
    if ((lane & (a.block_lanes - 1)) == 0) {
      scale_store(a.scales, a.zeros, e0 >> a.block_shift, sa, SF, true);
      scale_store(a.scales, a.zeros, (e0 + 512) >> a.block_shift, sb, SF, true);
    }
  }
  Codes c;
  YW<LQ_BF16> yw;
  float te, ts;
  lc_quant<F, SF, TL>(xs, sa, sb, c, yw, te, ts, &tl);
  lc_store_codes<F>(a.codes, chunk, lane, c);
  u32x4* q = (u32x4*)((char*)a.y + e0 * 2);
  gstore(q, (u32x4){yw.w[0], yw.w[1], yw.w[2], yw.w[3]});
  gstore(q + 64, (u32x4){yw.w[4], yw.w[5], yw.w[6], yw.w[7]});   // 1024 bytes on
  if (!sums_in_range(te, ts)) return false;
  acc_e += (double)te;
  acc_s += (double)ts;
  return true;
}

// fp64 QSNR terms of the lane tiles marked in `slow` (bit k: the chunk of
// pass k), after the main loop: re-read, scales and codes recomputed with the
// same arithmetic (every lane of the wave takes each step, as in the loop),
// and the terms added one element at a time.
template <int F, int SF, int MODE>
__device__ void lc_redo(const FastArgs& a, int64_t w0, int64_t wstride, int lane, uint32_t slow, const Scale& tsc,
                        const TScale& tl, double& acc_e, double& acc_s, uint32_t& bad) {
  constexpr int TL = MODE == LC_TWO ? TL_FAST : TL_NONE;
  for (int k = 0; k < kFastMaxIters; k++) {
    const bool marked = ((slow >> k) & 1u) != 0u;
    if (!__any(marked)) continue;
    const int64_t chunk = w0 + (int64_t)k * wstride;
    if (chunk >= a.ntiles) continue;              // uniform over the wave
    Raw<LQ_BF16> r;
    lc_load(r, a.x, chunk, lane);
    const RawX<LQ_BF16> xs{r};
    Scale sa = tsc, sb = tsc;
    if constexpr (MODE != LC_TENSOR) lc_scales<F, SF, TL>(a, xs, sa, sb, tl);
    Codes c;
    YW<LQ_BF16> yw;
    float te, ts;
    lc_quant<F, SF, TL>(xs, sa, sb, c, yw, te, ts, &tl);
    if (marked) {
      float d[16];
      decode_tile<F>(c, d);                       // element order: group 0, then group 1
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const Scale& sc = i < 8 ? sa : sb;
        const float x = xs(i);
        float xh = sc.div == DIV_ZERO ? 0.0f : d[i] * sc.s;
        if constexpr (TL != TL_NONE) xh = xh * tl.s;
        const double e = (double)x - (double)xh;
        acc_e += e * e;
        acc_s += (double)x * (double)x;
        bad += ((__float_as_uint(x) & 0x7F800000u) == 0x7F800000u) ? 1u : 0u;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// LC_TENSOR: one scale for the whole tensor from max|x|, combined by every
// workgroup from k_stat's partials (order-free); workgroup 0 stores it.
// LC_TWO: the tensor scale S the same way, and E4M3 block scales.
template <int F, int SF, int MODE, bool WIDE>
__global__ void __launch_bounds__(fast_threads(WIDE))
    __attribute__((amdgpu_waves_per_eu(fast_waves_per_simd(LQ_BF16, F, false, WIDE)))) k_lc(FastArgs a) {
  constexpr bool TENSOR = MODE == LC_TENSOR;
  static_assert(MODE != LC_TWO || SF == LQ_SCALE_E4M3, "two-level scaling has E4M3 block scales");
  constexpr int NT = fast_threads(WIDE);
  constexpr int kWaves = NT / 64;
  if (WIDE && a.nwork > 0 && (int)blockIdx.x >= a.nwork) {
    qsnr_collect_only<NT>(a.ws, a.epoch, a.nwork, a.res);
    return;
  }
  double acc_e = 0.0, acc_s = 0.0;
  uint32_t bad = 0, slow = 0;
  const int lane = threadIdx.x & 63;
  // this wave's first chunk; wave-uniform, so held in scalar registers with
  // the whole chunk loop
  const int64_t w0 = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t wstride = (int64_t)work_groups(a) * kWaves;
  // software pipeline as in k_fast: the next chunk's loads are issued as soon
  // as this chunk's registers are copied (a wave-uniform branch: a wave past
  // the end loads nothing, rather than every such wave re-reading one chunk)
  Raw<LQ_BF16> r;
  if (w0 < a.ntiles) lc_load(r, a.x, w0, lane);
  // the tensor scale: the statistic partials are read while the first
  // chunk's loads are in flight
  Scale tsc;
  if constexpr (TENSOR) {
    float am = 0.0f;
    for (int i = threadIdx.x; i < a.stat_parts; i += NT) am = fmaxf(am, a.ws->part_amax[i]);
    tsc = scale_sym<F>(block_max_nt<NT>(am), SF);
    if (blockIdx.x == 0 && threadIdx.x == 0) scale_store(a.scales, a.zeros, 0, tsc, SF, true);
    // the same in every lane: keep it in scalar registers for the loop
    tsc.s = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(tsc.s)));
    tsc.r = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(tsc.r)));
    tsc.zp = 0.0f;
    tsc.sbits = __builtin_amdgcn_readfirstlane(tsc.sbits);
    tsc.zbits = 0u;
    tsc.div = __builtin_amdgcn_readfirstlane(tsc.div);
  } else {
    tsc.s = tsc.r = tsc.zp = 0.0f;
    tsc.sbits = tsc.zbits = 0u;
    tsc.div = DIV_ZERO;
  }
  TScale tl;
  if constexpr (MODE == LC_TWO) tl = tscale_from_stat<F, NT>(a);
  else tl.s = tl.r = tl.sp = tl.p = 1.0f;
  wait_vmem_all();
  int k = 0;
  for (int64_t chunk = w0; chunk < a.ntiles; chunk += wstride, k++) {
    const Raw<LQ_BF16> cur = r;
    const int64_t cn = chunk + wstride;
    if (cn < a.ntiles) lc_load(r, a.x, cn, lane);
    if (!lc_tile<F, SF, MODE>(a, chunk, lane, cur, tsc, tl, acc_e, acc_s)) slow |= 1u << k;
  }
  if (__any(slow != 0u)) lc_redo<F, SF, MODE>(a, w0, wstride, lane, slow, tsc, tl, acc_e, acc_s, bad);
  if (WIDE || a.finish_inline) {
    qsnr_publish<NT>(a.ws, a.epoch, acc_e, acc_s, bad);
    if (a.nwork == 0) qsnr_finish<NT>(a.ws, a.epoch, gridDim.x, a.res);
  } else {
    qsnr_partial_ws(a.ws, acc_e, acc_s, bad);
  }
}

// ---- per-channel: one wave per row, rows of 1024..4096 elements (a
// multiple of 1024) held in registers as 1..4 lane-contiguous chunks; the row
// scale comes from a wave-wide max; 256-thread workgroups (4 rows each) over
// a grid the host keeps within kInlineFinishMaxWG, rows strided over it; the
// QSNR is finished in-kernel. FastArgs: `ntiles` = rows, `block_lanes` =
// chunks per row.
constexpr int kRowMaxChunks = 4;

template <int F, int SF>
__global__ void __launch_bounds__(kThreads) k_row_lc(FastArgs a) {
  constexpr int kWaves = kThreads / 64;
  double acc_e = 0.0, acc_s = 0.0;
  uint32_t bad = 0;
  const int lane = threadIdx.x & 63;
  const int cpr = a.block_lanes;
  const int64_t wave = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int64_t row = wave; row < a.ntiles; row += (int64_t)gridDim.x * kWaves) {
    Raw<LQ_BF16> r[kRowMaxChunks];
#pragma unroll
    for (int j = 0; j < kRowMaxChunks; j++)
      if (j < cpr) lc_load(r[j], a.x, row * cpr + j, lane);
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < kRowMaxChunks; j++) {
      if (j < cpr) {
        const RawX<LQ_BF16> xs{r[j]};
#pragma unroll
        for (int i = 0; i < 16; i++) am = fmaxf(am, fabsf(xs(i)));
      }
    }
    const Scale sc = scale_sym<F>(wave_max(am), SF);
    if (lane == 0) scale_store(a.scales, a.zeros, row, sc, SF, true);
#pragma unroll
    for (int j = 0; j < kRowMaxChunks; j++) {
      if (j < cpr) {
        const RawX<LQ_BF16> xs{r[j]};
        Codes c;
        YW<LQ_BF16> yw;
        float te, ts;
        lc_quant<F, SF, TL_NONE>(xs, sc, sc, c, yw, te, ts);
        const int64_t e0 = (row * cpr + j) * 1024 + 8 * lane;
        lc_store_codes<F>(a.codes, row * cpr + j, lane, c);
        u32x4* q = (u32x4*)((char*)a.y + e0 * 2);
        gstore(q, (u32x4){yw.w[0], yw.w[1], yw.w[2], yw.w[3]});
        gstore(q + 64, (u32x4){yw.w[4], yw.w[5], yw.w[6], yw.w[7]});
        if (sums_in_range(te, ts)) {
          acc_e += (double)te;
          acc_s += (double)ts;
        } else {
          // tiny, huge or non-finite values: the chunk's terms in fp64 from
          // its codes, one element at a time
          float d[16];
          decode_tile<F>(c, d);
#pragma unroll
          for (int i = 0; i < 16; i++) {
            const float x = xs(i);
            const float xh = sc.div == DIV_ZERO ? 0.0f : d[i] * sc.s;
            const double e = (double)x - (double)xh;
            acc_e += e * e;
            acc_s += (double)x * (double)x;
            bad += ((__float_as_uint(x) & 0x7F800000u) == 0x7F800000u) ? 1u : 0u;
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
  }
  qsnr_publish<kThreads>(a.ws, a.epoch, acc_e, acc_s, bad);
  qsnr_finish<kThreads>(a.ws, a.epoch, gridDim.x, a.res);
}

template <int F, int SF>
static hipError_t launch_row_lc(const FastArgs& a, int nwg, hipStream_t s) {
  if (g_plan) return plan_add(nwg, kThreads, "void lqd::k_row_lc<%d, %d>(lqd::FastArgs)", F, SF);
  hipLaunchKernelGGL((k_row_lc<F, SF>), dim3(nwg), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// The wide shape (one pass) gets a collecting workgroup of its own after its
// nwg working ones (qsnr_collect_only).
template <int F, int SF, int MODE, bool WIDE>
static hipError_t launch_lc(const FastArgs& a0, int nwg, hipStream_t s) {
  FastArgs a = a0;
  int grid = nwg;
  if (WIDE) {
    a.nwork = nwg;
    grid = nwg + 1;
  }
  if (g_plan) return plan_add(grid, fast_threads(WIDE), "void lqd::k_lc<%d, %d, %d, %s>(lqd::FastArgs)", F, SF, MODE, tf(WIDE));
  hipLaunchKernelGGL((k_lc<F, SF, MODE, WIDE>), dim3(grid), dim3(fast_threads(WIDE)), 0, s, a);
  return hipGetLastError();
}

// Only the narrow shape for fp32 block scales (their two divisions per lane)
// and for FP6 (its encoder and 48-bit packing): neither fits the wide shape's
// 64 VGPRs without spilling. A missing wide entry sends the call to the
// narrow one.
template <int F>
constexpr bool lc_wide_fits(int sf) {
  return sf != LQ_SCALE_F32 && !Fmt<F>::six;
}

template <int F, int SF>
static void put(LcSet& k) {
  k.k[F][SF][0][0] = &launch_lc<F, SF, LC_BLOCK, false>;
  if constexpr (lc_wide_fits<F>(SF)) k.k[F][SF][0][1] = &launch_lc<F, SF, LC_BLOCK, true>;
}

template <int F>
static void put_all_scales(LcSet& k) {
  put<F, LQ_SCALE_F32>(k);
  put<F, LQ_SCALE_F16>(k);
  put<F, LQ_SCALE_UE8M0>(k);
  put<F, LQ_SCALE_E4M3>(k);
  // per-tensor scales are fp32 (the other formats go through k_flat)
  k.k[F][LQ_SCALE_F32][1][0] = &launch_lc<F, LQ_SCALE_F32, LC_TENSOR, false>;
  if constexpr (!Fmt<F>::six) k.k[F][LQ_SCALE_F32][1][1] = &launch_lc<F, LQ_SCALE_F32, LC_TENSOR, true>;
  k.two[F][0] = &launch_lc<F, LQ_SCALE_E4M3, LC_TWO, false>;
  if constexpr (!Fmt<F>::six) k.two[F][1] = &launch_lc<F, LQ_SCALE_E4M3, LC_TWO, true>;
}

template <int F>
static void put_rows(LcSet& k) {
  k.row[F][LQ_SCALE_F32] = &launch_row_lc<F, LQ_SCALE_F32>;
  k.row[F][LQ_SCALE_F16] = &launch_row_lc<F, LQ_SCALE_F16>;
  k.row[F][LQ_SCALE_UE8M0] = &launch_row_lc<F, LQ_SCALE_UE8M0>;
  k.row[F][LQ_SCALE_E4M3] = &launch_row_lc<F, LQ_SCALE_E4M3>;
}

void lc_kernels(LcSet& k) {
  for (auto& a : k.k)
    for (auto& b : a)
      for (auto& c : b)
        for (auto& d : c) d = nullptr;
  for (auto& a : k.row)
    for (auto& b : a) b = nullptr;
  for (auto& a : k.two)
    for (auto& b : a) b = nullptr;
  put_rows<LQ_INT8>(k);
  put_rows<LQ_INT4>(k);
  put_rows<LQ_E4M3>(k);
  put_rows<LQ_E5M2>(k);
  put_rows<LQ_E2M1>(k);
  put_all_scales<LQ_INT8>(k);
  put_all_scales<LQ_INT4>(k);
  put_all_scales<LQ_E4M3>(k);
  put_all_scales<LQ_E5M2>(k);
  put_all_scales<LQ_E2M1>(k);
  put_rows<LQ_E2M3>(k);
  put_rows<LQ_E3M2>(k);
  put_all_scales<LQ_E2M3>(k);
  put_all_scales<LQ_E3M2>(k);
}

}  // namespace lqd
