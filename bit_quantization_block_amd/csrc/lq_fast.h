// lq_fast.h — specialised per-block fake-quant kernels for the common
// configuration: block scales computed from the data, round half to even,
// codes, scales (zeros), dequantized output and QSNR all produced. Format,
// scale format, zero point, input/output dtype and rotation are template
// parameters, so the tile loop is one straight-line path with few live
// registers; every other combination runs through k_flat.
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
  int64_t ntiles;        // tiles of 16 elements (the element count is a multiple of the block)
  int32_t block_lanes;   // block / 16
  int32_t block_shift;   // log2(block_lanes)
  int32_t unrotate;      // rotation: write y back in the original domain
};

template <int DT, int F, int ODT, int SF, bool SYM, bool HAD, class X>
__device__ __forceinline__ void fast_tile(const FastArgs& a, int64_t t, const X& xs, double& acc_e, double& acc_s,
                                          uint32_t& bad) {
  using M = ModeC<SF == LQ_SCALE_UE8M0, SYM, false>;
  const M md{};
  Scale sc;
  if constexpr (SYM) {
    sc = scale_sym<F>(group_max(tile_absmax_x(xs), a.block_lanes), SF);
  } else {
    float mn = xs(0), mx = xs(0);
#pragma unroll
    for (int i = 1; i < 16; i++) { mn = fminf(mn, xs(i)); mx = fmaxf(mx, xs(i)); }
    sc = scale_asym<F>(group_min(mn, a.block_lanes), group_max(mx, a.block_lanes), SF, LQ_RNE);
  }
  const int64_t bidx = t >> a.block_shift;
  if ((threadIdx.x & (a.block_lanes - 1)) == 0) scale_store(a.scales, a.zeros, bidx, sc, SF, SYM);
  Codes c;
  YW<ODT> yw;
  float te, ts;
  // only an fp32 scale can be so small that 1/s overflows
  constexpr bool kIeee = SF == LQ_SCALE_F32;
  if (HAD && a.unrotate) {
    float xh[16];
    if (kIeee && sc.div == DIV_IEEE) quant_stream<F, ODT, true, true>(xs, sc, md, c, yw, xh, te, ts);
    else quant_stream<F, ODT, true, false>(xs, sc, md, c, yw, xh, te, ts);
    if (SF != LQ_SCALE_UE8M0 && sc.div == DIV_ZERO) {
#pragma unroll
      for (int i = 0; i < 16; i++) xh[i] = 0.0f;
    }
    hadamard16(xh);
#pragma unroll
    for (int i = 0; i < 16; i += 2) put_y<ODT>(yw, i, xh[i], xh[i + 1]);
  } else {
    if (kIeee && sc.div == DIV_IEEE) quant_stream<F, ODT, false, true>(xs, sc, md, c, yw, nullptr, te, ts);
    else quant_stream<F, ODT, false, false>(xs, sc, md, c, yw, nullptr, te, ts);
    if (SF != LQ_SCALE_UE8M0 && sc.div == DIV_ZERO) {
#pragma unroll
      for (int i = 0; i < (ODT == LQ_F32 ? 16 : 8); i++) yw.w[i] = 0u;
    }
  }
  if (SF != LQ_SCALE_UE8M0 && sc.div == DIV_ZERO) {
    // zero stored scale: code 0, xhat = +0, so the error is the signal
#pragma unroll
    for (int j = 0; j < 4; j++) c.w[j] = 0u;
    te = ts;
  }
  const int64_t e0 = t << 4;
  store_codes<F>(a.codes, e0, 16, c);
  store_yw<ODT>(a.y, e0, 16, yw);
  tile_sums<F>(xs, c, sc, SYM, te, ts, acc_e, acc_s, bad);
}

#ifndef LQ_FAST_PIPE
#define LQ_FAST_PIPE 1
#endif

template <int DT, int F, int ODT, int SF, bool SYM, bool HAD>
__device__ __forceinline__ void fast_body(const FastArgs& a, int64_t t, const Raw<DT>& cur, double& acc_e,
                                          double& acc_s, uint32_t& bad) {
  if constexpr (HAD) {
    float x[16];
    raw_to_float<DT>(cur, x);
    hadamard16(x);
    fast_tile<DT, F, ODT, SF, SYM, HAD>(a, t, ArrX{x}, acc_e, acc_s, bad);
  } else {
    fast_tile<DT, F, ODT, SF, SYM, HAD>(a, t, RawX<DT>{cur}, acc_e, acc_s, bad);
  }
}

template <int DT, int F, int ODT, int SF, bool SYM, bool HAD>
__global__ void __launch_bounds__(kThreads) k_fast(FastArgs a) {
  double acc_e = 0.0, acc_s = 0.0;
  uint32_t bad = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
#if LQ_FAST_PIPE == 0
  for (; t < a.ntiles; t += stride) {
    Raw<DT> cur;
    raw_load<DT>(cur, a.x, t << 4);
    fast_body<DT, F, ODT, SF, SYM, HAD>(a, t, cur, acc_e, acc_s, bad);
  }
#elif LQ_FAST_PIPE == 1
  const int64_t last = a.ntiles - 1;           // the host launches only with ntiles >= 1
  // software pipeline: the next tile's loads are issued as soon as this
  // tile's registers are copied; past the end the load repeats the last tile
  Raw<DT> r;
  raw_load<DT>(r, a.x, (t < last ? t : last) << 4);
  wait_vmem_all();
  for (; t < a.ntiles; t += stride) {
    const Raw<DT> cur = r;
    const int64_t tn = t + stride;
    raw_load<DT>(r, a.x, (tn < last ? tn : last) << 4);
    fast_body<DT, F, ODT, SF, SYM, HAD>(a, t, cur, acc_e, acc_s, bad);
  }
#else
  // software pipeline without the trailing load: a lane loads its next tile
  // only when it has one
  if (t < a.ntiles) {
    Raw<DT> r;
    raw_load<DT>(r, a.x, t << 4);
    wait_vmem_all();
    for (;;) {
      const Raw<DT> cur = r;
      const int64_t tn = t + stride;
      const bool more = tn < a.ntiles;
      if (more) raw_load<DT>(r, a.x, tn << 4);
      fast_body<DT, F, ODT, SF, SYM, HAD>(a, t, cur, acc_e, acc_s, bad);
      if (!more) break;
      t = tn;
    }
  }
#endif
  qsnr_partial_ws(a.ws, acc_e, acc_s, bad);
}

template <int DT, int F, int ODT, int SF, bool SYM, bool HAD>
hipError_t launch_fast(const FastArgs& a, int nwg, hipStream_t s) {
  hipLaunchKernelGGL((k_fast<DT, F, ODT, SF, SYM, HAD>), dim3(nwg), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

typedef hipError_t (*fast_fn)(const FastArgs&, int, hipStream_t);

// [format][scale format][asymmetric][rotation]
struct FastSet {
  fast_fn k[5][4][2][2];
};

}  // namespace lqd
