// lq_kernels.h — gfx950 kernels of liblq (templates; instantiated in lq_inst.hip).
//
// Data layout in HBM: x, codes and y are row-major; one lane owns 16
// consecutive elements (one "tile"); a workgroup of 256 lanes walks 4096
// consecutive elements per step and strides over the tensor (grid-stride), so
// every wave reads and writes contiguous runs and every block of
// 16..256 elements lives in 1..16 neighbouring lanes.
#pragma once
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <utility>

#include "lq_device.h"

namespace lqd {

struct Args {
  const void* x;
  uint8_t* codes;
  void* scales;
  void* zeros;
  void* y;
  int64_t rows, cols, n;   // n = rows * cols
  int32_t block_lanes;     // per-block granularity: block / 16 (1..16)
  int32_t block_shift;     // log2(block_lanes)
  int32_t scale_fmt, sym, rnd, out_dt;
  int32_t had, unrotate, given, qsnr;   // had: rotation size n (0: none)
  int32_t pow2;            // scale_fmt == UE8M0 (or a given power-of-two scale)
  int32_t maybe_ieee;      // scales may be so small that 1/s overflows (fp32 or given scales)
  Workspace* ws;
  lq_result* res;
  int32_t stat_parts;      // per-tensor with data-driven scale: k_stat partials to combine first
  int32_t finish_inline;   // the grid's last workgroup writes *res (tagged partials, no k_finish)
  uint32_t epoch;          // tag of this call's partials when finish_inline
  float* tscale;           // two-level: where S is stored (written, or read when given); may be null
  int32_t tile_rows;       // 2-D tiles: rows and columns of a tile (0: no tiles), and
  int32_t tile_cols;       // log2(tile_cols / 16)
  int32_t unit_shift;
  float rot_c;             // rotation: 1/sqrt(had) in binary32
  const uint32_t* signs;   // rotation: the random signs, one bit per column (may be null)
};

__device__ __forceinline__ Rot rot_of(const Args& a, int64_t e0) {
  return make_rot(a.had, a.rot_c, a.signs, e0, a.cols);
}

// k_flat modes: one scale per block, one per tensor, or two-level (E4M3
// block scales under an FP32 tensor scale).
constexpr int FLAT_BLOCK = 0, FLAT_TENSOR = 1, FLAT_TWO = 2;

// Per-channel kernel (one wave per row, rows strided over the grid): grids
// of at most this many workgroups.
constexpr int kInlineFinishMaxWG = 1024;

// ---------------------------------------------------------------- reductions
// Wave sums in a fixed order: inside each row of 16 lanes by DPP moves (swap
// neighbours, swap pairs, mirror the half-row, mirror the row), then the four
// row sums read from lanes 0, 16, 32 and 48 and added pairwise. All 64 lanes
// must be active; the result is uniform.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t r = ((uint64_t)dpp32<CTRL>((uint32_t)(u >> 32)) << 32) | dpp32<CTRL>((uint32_t)u);
  return __longlong_as_double((long long)r);
}
__device__ __forceinline__ double lane64(double v, int lane) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t r = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane) << 32) |
                     (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  return __longlong_as_double((long long)r);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
__device__ __forceinline__ double wave_sum(double v) {
  v += dpp64<kDppXor1>(v);
  v += dpp64<kDppXor2>(v);
  v += dpp64<kDppHalfMirror>(v);
  v += dpp64<kDppMirror>(v);
  return (lane64(v, 0) + lane64(v, 16)) + (lane64(v, 32) + lane64(v, 48));
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  v += dpp32<kDppXor1>(v);
  v += dpp32<kDppXor2>(v);
  v += dpp32<kDppHalfMirror>(v);
  v += dpp32<kDppMirror>(v);
  return ((uint32_t)__builtin_amdgcn_readlane((int)v, 0) + (uint32_t)__builtin_amdgcn_readlane((int)v, 16)) +
         ((uint32_t)__builtin_amdgcn_readlane((int)v, 32) + (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
}

// Sums over an NT-thread workgroup of every thread's (e, s, b), in a fixed
// order, valid in wave 0 (uniform there). The fp64 terms go through LDS and
// only wave 0 adds them up (each lane its NT/64 entries in order, then across
// lanes), so the lane reduction, some 50 VALU operations, runs in one wave of
// the workgroup rather than in each. The non-finite count is reduced only in
// a wave where some lane has one.
template <int NT>
__device__ __forceinline__ void block_sums(double e, double s, uint32_t b, double& E, double& S, uint32_t& B) {
  constexpr int NW = NT / 64;
  __shared__ double sh_e[NT], sh_s[NT];
  __shared__ uint32_t sh_b[NW];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  sh_e[tid] = e;
  sh_s[tid] = s;
  const uint32_t wb = __any(b != 0u) ? wave_sum(b) : 0u;
  if (lane == 0) sh_b[wave] = wb;
  __syncthreads();
  if (wave == 0) {
    double pe = sh_e[lane], ps = sh_s[lane];
#pragma unroll
    for (int w = 1; w < NW; w++) {
      pe += sh_e[lane + 64 * w];
      ps += sh_s[lane + 64 * w];
    }
    E = wave_sum(pe);
    S = wave_sum(ps);
    uint32_t nb = 0;
#pragma unroll
    for (int w = 0; w < NW; w++) nb += sh_b[w];
    B = nb;
  }
}

// Partial QSNR sums of one 256-thread workgroup into the workspace.
__device__ inline void qsnr_partial_ws(Workspace* ws, double e, double s, uint32_t b) {
  double E, S;
  uint32_t B;
  block_sums<256>(e, s, b, E, S, B);
  if (threadIdx.x == 0) {
    ws->part_err[blockIdx.x] = E;
    ws->part_sig[blockIdx.x] = S;
    ws->part_bad[blockIdx.x] = B;
  }
}
__device__ inline void qsnr_partial(const Args& a, double e, double s, uint32_t b) {
  qsnr_partial_ws(a.ws, e, s, b);
}

// Last step of the QSNR sum, shared by both finishing routes: each thread of
// an NT-thread workgroup holds the sequential sum of partials tid, tid + NT,
// ...; lanes and waves are combined in a fixed order and thread 0 writes the
// result. `failed` marks a sum whose partials did not all arrive (the result
// then reads NaN with reserved = 1).
template <int NT>
__device__ __forceinline__ double sum_waves(const double* v) {
  if constexpr (NT == 256) return (v[0] + v[1]) + (v[2] + v[3]);
  double t[NT / 128];
#pragma unroll
  for (int i = 0; i < NT / 128; i++) t[i] = v[2 * i] + v[2 * i + 1];
#pragma unroll
  for (int w = NT / 256; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; i++) t[i] = t[2 * i] + t[2 * i + 1];
  return t[0];
}

// The workgroup's totals of per-thread sums, in a fixed order (lanes by DPP,
// then waves pairwise), valid in thread 0; `failed` is set there when any
// thread's was.
template <int NT = kThreads>
__device__ inline void block_totals(double& E, double& S, uint32_t& B, bool& failed) {
  constexpr int NW = NT / 64;
  __shared__ double sh_e[NW], sh_s[NW];
  __shared__ uint32_t sh_b[NW], sh_f[NW];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  E = wave_sum(E);
  S = wave_sum(S);
  B = wave_sum(B);
  const uint32_t f = wave_sum(failed ? 1u : 0u);
  if (lane == 0) { sh_e[wave] = E; sh_s[wave] = S; sh_b[wave] = B; sh_f[wave] = f; }
  __syncthreads();
  if (tid == 0) {
    uint32_t nb = 0, nf = 0;
#pragma unroll
    for (int w = 0; w < NW; w++) { nb += sh_b[w]; nf += sh_f[w]; }
    E = sum_waves<NT>(sh_e);
    S = sum_waves<NT>(sh_s);
    B = nb;
    failed = nf != 0u;
  }
}

__device__ inline void write_result(double E, double S, uint32_t B, bool failed, lq_result* res) {
  if (failed) {
    res->err2 = __builtin_nan("");
    res->sig2 = __builtin_nan("");
    res->qsnr_db = __builtin_nan("");
    res->nonfinite = 0xFFFFFFFFu;
    res->reserved = 1u;
    return;
  }
  res->err2 = E;
  res->sig2 = S;
  res->qsnr_db = (E == 0.0) ? __builtin_inf() : -10.0 * log10(E / S);
  res->nonfinite = B;
  res->reserved = 0u;
}

template <int NT = kThreads>
__device__ inline void finish_write(double E, double S, uint32_t B, bool failed, lq_result* res) {
  block_totals<NT>(E, S, B, failed);
  if (threadIdx.x == 0) write_result(E, S, B, failed, res);
}

// Second stage of the QSNR sum: one workgroup adds the `parts` partials in a
// fixed order (deterministic for a given grid) and writes the result. The
// partials are read 16 bytes per lane (two sums or four counts): one
// workgroup's load issue is what this kernel waits on, and 8-byte loads took
// 2.4 times as many instructions. Lanes past `parts` add zeros (the words
// there, inside the arrays, may hold an older call's partials).
__device__ __forceinline__ double f64_of(uint32_t lo, uint32_t hi) {
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
static __global__ void __launch_bounds__(kThreads) k_finish(const Workspace* ws, int parts, lq_result* res) {
  constexpr int K2 = kMaxWG / 2 / kThreads, K4 = kMaxWG / 4 / kThreads;
  const int tid = threadIdx.x;
  const u32x4* pe = (const u32x4*)ws->part_err;
  const u32x4* ps = (const u32x4*)ws->part_sig;
  const u32x4* pb = (const u32x4*)ws->part_bad;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  // every load is issued before the first is used
  u32x4 we[K2], ws2[K2], wb[K4];
#pragma unroll
  for (int k = 0; k < K2; k++) {
    const int j = tid + k * kThreads;
    we[k] = 2 * j < parts ? pe[j] : zero;
    ws2[k] = 2 * j < parts ? ps[j] : zero;
  }
#pragma unroll
  for (int k = 0; k < K4; k++) {
    const int j = tid + k * kThreads;
    wb[k] = 4 * j < parts ? pb[j] : zero;
  }
  double E = 0.0, S = 0.0;
  uint32_t B = 0;
#pragma unroll
  for (int k = 0; k < K2; k++) {
    const bool second = 2 * (tid + k * kThreads) + 1 < parts;
    E += f64_of(we[k][0], we[k][1]);
    E += second ? f64_of(we[k][2], we[k][3]) : 0.0;
    S += f64_of(ws2[k][0], ws2[k][1]);
    S += second ? f64_of(ws2[k][2], ws2[k][3]) : 0.0;
  }
#pragma unroll
  for (int k = 0; k < K4; k++) {
    const int i0 = 4 * (tid + k * kThreads);
#pragma unroll
    for (int c = 0; c < 4; c++) B += i0 + c < parts ? wb[k][c] : 0u;
  }
  finish_write(E, S, B, false, res);
}

// ---- in-kernel finish (tagged partials, see Workspace)
__device__ __forceinline__ void tag_store(uint64_t* p, uint64_t tag, uint32_t payload) {
  __hip_atomic_store(p, tag | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tag_load(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void tag_record(uint64_t* r, uint32_t epoch, double E, double S, uint32_t B);

// Workgroup partials of an NT-thread workgroup, published tagged.
template <int NT>
__device__ inline void qsnr_publish(Workspace* ws, uint32_t epoch, double e, double s, uint32_t b) {
  double E, S;
  uint32_t B;
  block_sums<NT>(e, s, b, E, S, B);
  if (threadIdx.x == 0) tag_record(ws->tagged[blockIdx.x], epoch, E, S, B);
}

// Polls of one record before the collecting workgroup gives up (each poll
// sleeps about 0.1 us; every other workgroup publishes unconditionally, so
// only a lost write could exhaust this).
constexpr int kPollLimit = 1 << 22;
// Non-finite count of a group record whose sum could not be completed.
constexpr uint32_t kFailedCount = 0xFFFFFFFFu;

// Per-thread sums of the tagged records [i0, i1) of `rec`: thread tid takes
// records i0 + tid, i0 + tid + NT, ... in order, CHUNK at a time with all
// their loads in flight together, polling each until its five words carry
// `epoch`. `failed` on a record that never arrived or that reports a failed
// sum. The callers pick CHUNK so that one round of loads covers the range:
// the collection is a chain of memory round trips at the end of the kernel
// (measured on C3's lane-contiguous group-64 call: 45.1 us with the
// collection, 39.6 us without it, when it took two rounds of two per thread).
// Four records per thread would raise the kernels' registers: the
// collection's share decides the whole kernel's budget.
template <int NT, int CHUNK>
__device__ inline void collect_range(const uint64_t (*rec)[kTagWords], uint32_t epoch, int i0, int i1, double& E,
                                     double& S, uint32_t& B, bool& failed) {
  constexpr int kChunk = CHUNK;
  const int tid = threadIdx.x;
  for (int k0 = i0; k0 < i1; k0 += kChunk * NT) {
    uint64_t w[kChunk][kTagWords];
#pragma unroll
    for (int k = 0; k < kChunk; k++) {
      const int i = k0 + tid + k * NT;
#pragma unroll
      for (int j = 0; j < kTagWords; j++) w[k][j] = (i < i1) ? tag_load(&rec[i][j]) : 0;
    }
#pragma unroll
    for (int k = 0; k < kChunk; k++) {
      const int i = k0 + tid + k * NT;
      if (i >= i1 || failed) continue;
      for (int polls = 0;; polls++) {
        bool ready = true;
#pragma unroll
        for (int j = 0; j < kTagWords; j++) ready &= (uint32_t)(w[k][j] >> 32) == epoch;
        if (ready) break;
        if (polls == kPollLimit) { failed = true; break; }
        __builtin_amdgcn_s_sleep(4);
#pragma unroll
        for (int j = 0; j < kTagWords; j++) w[k][j] = tag_load(&rec[i][j]);
      }
      if (failed) continue;
      E += __longlong_as_double((long long)((w[k][1] << 32) | (w[k][0] & 0xFFFFFFFFull)));
      S += __longlong_as_double((long long)((w[k][3] << 32) | (w[k][2] & 0xFFFFFFFFull)));
      const uint32_t b = (uint32_t)w[k][4];
      if (b == kFailedCount) failed = true;
      else B += b;
    }
  }
}

__device__ __forceinline__ void tag_record(uint64_t* r, uint32_t epoch, double E, double S, uint32_t B) {
  const uint64_t tag = (uint64_t)epoch << 32;
  const uint64_t e = (uint64_t)__double_as_longlong(E), s = (uint64_t)__double_as_longlong(S);
  tag_store(&r[0], tag, (uint32_t)e);
  tag_store(&r[1], tag, (uint32_t)(e >> 32));
  tag_store(&r[2], tag, (uint32_t)s);
  tag_store(&r[3], tag, (uint32_t)(s >> 32));
  tag_store(&r[4], tag, B);
}

// After every workgroup's qsnr_publish: the grid's last K = ceil(nwg /
// kGroupRecords) workgroups each sum one range of kGroupRecords records and
// publish a group record; the last workgroup then sums the K group records
// and writes the result (with K = 1 it writes straight away). The collectors
// are the last workgroups dispatched and only they wait, so every record they
// wait for comes from a workgroup already running or finished; the sums are
// taken in a fixed order (deterministic for a given grid).
// (1024-thread workgroups, held to 64 VGPRs, come in grids of at most 2048:
// one workgroup collects every record, two per thread, as one group: the
// last working one here, or one of its own in qsnr_collect_only.)
template <int NT>
__host__ __device__ constexpr int qsnr_collectors(int nwg) {
  return NT >= 1024 ? 1 : (nwg + kGroupRecords - 1) / kGroupRecords;
}

// Collector j of K over the records of workgroups [0, nwg).
template <int NT>
__device__ inline void qsnr_collect(Workspace* ws, uint32_t epoch, int nwg, int K, int j, lq_result* res) {
  double E = 0.0, S = 0.0;
  uint32_t B = 0;
  bool failed = false;
  if constexpr (NT >= 1024) {
    collect_range<NT, 2>(ws->tagged, epoch, 0, nwg, E, S, B, failed);
    finish_write<NT>(E, S, B, failed, res);
    return;
  }
  const int i0 = j * kGroupRecords, i1 = i0 + kGroupRecords < nwg ? i0 + kGroupRecords : nwg;
  static_assert(kGroupRecords <= 2 * NT || NT >= 1024, "one round of two records per thread");
  collect_range<NT, (kGroupRecords + NT - 1) / NT>(ws->tagged, epoch, i0, i1, E, S, B, failed);
  if (K == 1) {
    finish_write<NT>(E, S, B, failed, res);
    return;
  }
  block_totals<NT>(E, S, B, failed);
  if (threadIdx.x == 0) tag_record(ws->group[j], epoch, E, S, failed ? kFailedCount : B);
  if (j != K - 1) return;
  E = S = 0.0;
  B = 0;
  failed = false;
  collect_range<NT, (kMaxGroups + NT - 1) / NT>(ws->group, epoch, 0, K, E, S, B, failed);
  finish_write<NT>(E, S, B, failed, res);
}

template <int NT>
__device__ inline void qsnr_finish(Workspace* ws, uint32_t epoch, int nwg, lq_result* res) {
  const int K = qsnr_collectors<NT>(nwg);
  const int j = (int)blockIdx.x - (nwg - K);
  if (j >= 0) qsnr_collect<NT>(ws, epoch, nwg, K, j, res);
}

// A collector of its own: a one-pass grid of nwork 1024-thread workgroups
// that only publish, then one more workgroup that only collects. It is
// dispatched after every publishing workgroup and polls at once, with no
// stores of its own outstanding (a wave's memory counter also counts its
// stores, so a collector that first streamed a chunk waits for those writes
// before its first poll returns). Measured on C2's MX calls (one pass over
// 2048 workgroups): 32.0-32.4 us per call against 32.7-33.1 us with the last
// working workgroup collecting, both load orders on one box. Grids of several
// passes keep their collectors among the working workgroups: there a
// collector of its own starts with the first pass and polls through the whole
// kernel (c7, capped at 1024 workgroups: 44.2-44.5 against 37.4-37.8 us).
template <int NT>
__device__ inline void qsnr_collect_only(Workspace* ws, uint32_t epoch, int nwork, lq_result* res) {
  qsnr_collect<NT>(ws, epoch, nwork, qsnr_collectors<NT>(nwork), (int)blockIdx.x - nwork, res);
}

__device__ __forceinline__ uint32_t count_nonfinite(const float* x) {
  uint32_t b = 0;
#pragma unroll
  for (int i = 0; i < 16; i++) b += ((__float_as_uint(x[i]) & 0x7F800000u) == 0x7F800000u) ? 1u : 0u;
  return b;
}

// Add a tile's fp32 sums to the fp64 accumulators. They are kept when both
// lie in [2^-100, +inf), where no term that matters can have overflowed or
// underflowed. Otherwise (huge or tiny values, an exact tile, non-finite
// inputs) the tile is summed again: xhat is rebuilt from the codes exactly as
// dequantization does, each sum is taken in fp32 after scaling by a power of
// two from its own tile maximum (max|x|, max|x - xhat|), returned to scale
// exactly in fp64, and non-finite inputs are counted.
template <int F, class X>
__device__ __forceinline__ void tile_sums_slow(const X& xs, const Codes& c, const Scale& sc, bool sym,
                                               double& acc_e, double& acc_s, uint32_t& bad, float tls) {
  float d[16], x[16];
  decode_tile<F>(c, d);
  float dmax = 0.0f, amax = 0.0f;
  uint32_t b = 0;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    x[i] = xs(i);
    const float xh = (sc.s == 0.0f) ? 0.0f : (sym ? d[i] * sc.s : sc.s * (d[i] - sc.zp)) * tls;
    d[i] = x[i] - xh;
    dmax = fmaxf(dmax, fabsf(d[i]));
    amax = fmaxf(amax, fabsf(x[i]));
    b += ((__float_as_uint(x[i]) & 0x7F800000u) == 0x7F800000u) ? 1u : 0u;
  }
  int ks = __builtin_amdgcn_frexp_expf(amax);
  int ke = __builtin_amdgcn_frexp_expf(dmax);
  ks = ks < -125 ? -125 : ks;
  ke = ke < -125 ? -125 : ke;
  const float fs = __builtin_ldexpf(1.0f, -ks), fe = __builtin_ldexpf(1.0f, -ke);
  float e = 0.0f, s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const float dd = d[i] * fe;
    const float xs_ = x[i] * fs;
    e = __builtin_fmaf(dd, dd, e);
    s = __builtin_fmaf(xs_, xs_, s);
  }
  acc_e += (double)e * __builtin_ldexp(1.0, 2 * ke);
  acc_s += (double)s * __builtin_ldexp(1.0, 2 * ks);
  bad += b;
}

// tls: the two-level tensor scale S that multiplies xhat (1 without one).
template <int F, class X>
__device__ __forceinline__ void tile_sums(const X& xs, const Codes& c, const Scale& sc, bool sym, float e, float s,
                                          double& acc_e, double& acc_s, uint32_t& bad, float tls = 1.0f) {
  const float lo = 0x1p-100f, hi = __builtin_inff();
  if (e >= lo && e < hi && s >= lo && s < hi) {
    acc_e += (double)e;
    acc_s += (double)s;
  } else {
    tile_sums_slow<F>(xs, c, sc, sym, acc_e, acc_s, bad, tls);
  }
}

__device__ __forceinline__ float tile_absmax(const float* x) {
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i++) am = fmaxf(am, fabsf(x[i]));
  return am;
}

// Workgroup-wide max / min (every thread gets the result).
__device__ __forceinline__ float block_reduce_max(float v, float* sh) {
  const int tid = threadIdx.x;
  v = wave_max(v);
  __syncthreads();
  if ((tid & 63) == 0) sh[tid >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}
__device__ __forceinline__ float block_reduce_min(float v, float* sh) {
  const int tid = threadIdx.x;
  v = wave_min(v);
  __syncthreads();
  if ((tid & 63) == 0) sh[tid >> 6] = v;
  __syncthreads();
  return fminf(fminf(sh[0], sh[1]), fminf(sh[2], sh[3]));
}

// ---------------------------------------------------------------- flat kernel
// Per-block (TENSOR = false) or per-tensor (TENSOR = true, scale from the
// statistic pass) fake-quant over the flattened tensor.
#ifndef LQ_WAVES_PER_EU
#define LQ_WAVES_PER_EU 0
#endif
#if LQ_WAVES_PER_EU > 0
#define LQ_OCCUPANCY __attribute__((amdgpu_waves_per_eu(LQ_WAVES_PER_EU)))
#else
#define LQ_OCCUPANCY
#endif

template <class X>
__device__ __forceinline__ float tile_absmax_x(const X& xs) {
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i++) am = fmaxf(am, fabsf(xs(i)));
  return am;
}

// Quantize a tile whose scale is known, store its codes and dequantized
// values, and add its QSNR terms (TL: under the tensor level *tl as well).
template <int F, int ODT, int TL, class X>
__device__ __forceinline__ void tile_quant_store(const Args& a, const Mode md, const Scale& sc, int64_t e0, int cnt,
                                                 const X& xs, double& acc_e, double& acc_s, uint32_t& bad,
                                                 const TScale* tl, const Rot& rot) {
  Codes c;
  YW<ODT> yw;
  float te, ts;
  // Given scales take IEEE division: Markstein's correction assumes
  // |x / s| <= Qmax (1 + 2^-23), true of scales from the data, but a given
  // scale far below |x| / Qmax makes x * RN(1/s) overflow and the corrected
  // quotient NaN (IEEE division returns the saturating infinity instead).
  const bool ieee = a.given || (a.maybe_ieee && sc.div == DIV_IEEE);
  if (a.had && a.unrotate) {
    float xh[16];
    if (ieee)
      quant_stream<F, ODT, true, DIVM_IEEE, TL>(xs, sc, md, c, yw, xh, te, ts, tl);
    else
      quant_stream<F, ODT, true, DIVM_MARKSTEIN, TL>(xs, sc, md, c, yw, xh, te, ts, tl);
    if (sc.div == DIV_ZERO) {
#pragma unroll
      for (int i = 0; i < 16; i++) xh[i] = 0.0f;
    }
    rot_inverse(xh, rot);
#pragma unroll
    for (int i = 0; i < 16; i += 2) put_y<ODT>(yw, i, xh[i], xh[i + 1]);
  } else {
    if (ieee)
      quant_stream<F, ODT, false, DIVM_IEEE, TL>(xs, sc, md, c, yw, nullptr, te, ts, tl);
    else
      quant_stream<F, ODT, false, DIVM_MARKSTEIN, TL>(xs, sc, md, c, yw, nullptr, te, ts, tl);
    if (sc.div == DIV_ZERO) {
#pragma unroll
      for (int i = 0; i < (ODT == LQ_F32 ? 16 : 8); i++) yw.w[i] = 0u;
    }
  }
  if (sc.div == DIV_ZERO) {
    // zero stored scale: code 0, xhat = +0, so the error is the signal
#pragma unroll
    for (int j = 0; j < 4; j++) c.w[j] = 0u;
    te = ts;
  }
  if (a.codes) store_codes<F>(a.codes, e0, cnt, c);
  if (a.y) store_yw<ODT>(a.y, e0, cnt, yw);
  if (a.qsnr) tile_sums<F>(xs, c, sc, md.sym, te, ts, acc_e, acc_s, bad, TL != TL_NONE ? tl->s : 1.0f);
}

// One tile of the flat kernel (per-block scale from the tile's lanes, or the
// per-tensor scale; two-level: the block scale of the tile's values divided
// by S, which is max|x| / S since correctly rounded division is monotone).
template <int F, int ODT, int MODE, class X>
__device__ __forceinline__ void flat_tile(const Args& a, const Mode md, const Scale& tsc, const TScale& tl, int64_t t,
                                          int cnt, const X& xs, double& acc_e, double& acc_s, uint32_t& bad,
                                          const Rot& rot) {
  constexpr int TL = MODE == FLAT_TWO ? TL_IEEE : TL_NONE;
  Scale sc;
  if constexpr (MODE == FLAT_TENSOR) {
    sc = tsc;
  } else {
    const int64_t bidx = t >> a.block_shift;
    if (a.given) {
      sc = scale_load(a.scales, a.zeros, bidx, a.scale_fmt, md.sym, true);
    } else {
      if (MODE == FLAT_TWO) {
        sc = scale_sym<F>(tdivide<TL_IEEE>(group_max(tile_absmax_x(xs), a.block_lanes), tl), LQ_SCALE_E4M3);
      } else if (md.sym) {
        sc = scale_sym<F>(group_max(tile_absmax_x(xs), a.block_lanes), a.scale_fmt);
      } else {
        float mn = xs(0), mx = xs(0);
#pragma unroll
        for (int i = 1; i < 16; i++) { mn = fminf(mn, xs(i)); mx = fmaxf(mx, xs(i)); }
        sc = scale_asym<F>(group_min(mn, a.block_lanes), group_max(mx, a.block_lanes), a.scale_fmt, a.rnd);
      }
      if ((threadIdx.x & (a.block_lanes - 1)) == 0) scale_store(a.scales, a.zeros, bidx, sc, a.scale_fmt, md.sym);
    }
  }
  tile_quant_store<F, ODT, TL>(a, md, sc, t << 4, cnt, xs, acc_e, acc_s, bad, &tl, rot);
}

#ifndef LQ_WAVES_PER_EU
#define LQ_WAVES_PER_EU 0
#endif
#if LQ_WAVES_PER_EU > 0
#define LQ_OCCUPANCY __attribute__((amdgpu_waves_per_eu(LQ_WAVES_PER_EU)))
#else
#define LQ_OCCUPANCY
#endif

// Per-block, per-tensor (scale from the statistic pass) or two-level (tensor
// scale from the statistic pass, or given) fake-quant over the flattened tensor.
template <int DT, int F, int ODT, int MODE>
__global__ void __launch_bounds__(kThreads) LQ_OCCUPANCY k_flat(Args a) {
  constexpr bool TENSOR = MODE == FLAT_TENSOR;
  const bool sym = a.sym != 0;
  const Mode md{a.pow2 != 0, sym, a.rnd == LQ_RNA};
  const int64_t ntiles = (a.n + 15) >> 4;
  const int64_t nfull = a.n >> 4;                 // tiles with 16 valid elements
  const int tid = threadIdx.x;
  double acc_e = 0.0, acc_s = 0.0;
  uint32_t bad = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t t = (int64_t)blockIdx.x * kThreads + tid;
  // Software pipeline: a tile's raw registers are copied once its loads have
  // landed and immediately receive the next tile's loads, which stay in
  // flight while this tile is processed. Only full tiles are loaded this way
  // (a partial tile is read element by element); lanes past them load nothing.
  Raw<DT> r;
  if (t < nfull) raw_load<DT>(r, a.x, t << 4);
  // the scale (per-tensor: the statistic partials are read while the first
  // tile's loads are in flight)
  Scale tsc;
  if constexpr (TENSOR) {
    float st[3] = {0.0f, 0.0f, 0.0f};
    if (!a.given) {
      // every workgroup combines k_stat's partials itself (a finishing
      // launch would cost more); max and min do not depend on the order
      __shared__ float sh[3][4];
      float am = 0.0f, mn = __builtin_inff(), mx = -__builtin_inff();
      for (int i = tid; i < a.stat_parts; i += kThreads) {
        am = fmaxf(am, a.ws->part_amax[i]);
        mn = fminf(mn, a.ws->part_min[i]);
        mx = fmaxf(mx, a.ws->part_max[i]);
      }
      st[0] = block_reduce_max(am, sh[0]);
      st[1] = block_reduce_min(mn, sh[1]);
      st[2] = block_reduce_max(mx, sh[2]);
    }
    if (a.given) tsc = scale_load(a.scales, a.zeros, 0, a.scale_fmt, sym, true);
    else if (sym) tsc = scale_sym<F>(st[0], a.scale_fmt);
    else tsc = scale_asym<F>(st[1], st[2], a.scale_fmt, a.rnd);
    if (!a.given && blockIdx.x == 0 && tid == 0) scale_store(a.scales, a.zeros, 0, tsc, a.scale_fmt, sym);
  } else {
    tsc.s = tsc.r = tsc.zp = 0.0f;
    tsc.sbits = tsc.zbits = 0u;
    tsc.div = DIV_ZERO;
  }
  TScale tl;
  tl.s = tl.r = tl.sp = tl.p = 1.0f;
  if constexpr (MODE == FLAT_TWO) {
    if (a.given) {
      tl.s = *a.tscale;
    } else {
      __shared__ float sh2[4];
      float am = 0.0f;
      for (int i = tid; i < a.stat_parts; i += kThreads) am = fmaxf(am, a.ws->part_amax[i]);
      tl.s = tensor_scale_of<F>(block_reduce_max(am, sh2));
      if (a.tscale && blockIdx.x == 0 && tid == 0) *a.tscale = tl.s;
    }
  }
  wait_vmem_all();
  for (; t < ntiles; t += stride) {
    const Raw<DT> cur = r;
    const int64_t tn = t + stride;
    if (tn < nfull) raw_load<DT>(r, a.x, tn << 4);
    const int cnt = (t < nfull) ? 16 : (int)(a.n - (t << 4));
    if (a.had || cnt < 16) {
      // a rotation group spans whole tiles of consecutive lanes (cols is a
      // multiple of the group, so every tile is full and the lanes of a group
      // leave the loop together)
      float x[16];
      const Rot rot = rot_of(a, t << 4);
      if (cnt < 16) load_partial<DT>(a.x, t << 4, cnt, x);
      else raw_to_float<DT>(cur, x);
      if (a.had) rot_forward(x, rot);
      flat_tile<F, ODT, MODE>(a, md, tsc, tl, t, cnt, ArrX{x}, acc_e, acc_s, bad, rot);
    } else {
      flat_tile<F, ODT, MODE>(a, md, tsc, tl, t, 16, RawX<DT>{cur}, acc_e, acc_s, bad, Rot{0, 1.0f, 0u, false});
    }
  }
  if (a.qsnr) {
    if (a.finish_inline) {
      qsnr_publish<kThreads>(a.ws, a.epoch, acc_e, acc_s, bad);
      qsnr_finish<kThreads>(a.ws, a.epoch, gridDim.x, a.res);
    } else {
      qsnr_partial(a, acc_e, acc_s, bad);
    }
  }
}

// ---------------------------------------------------------------- group kernel
// One scale per group of row segments: per-channel (a group is one row) or
// 2-D tiles (tile_rows segments of tile_cols elements; the last band of rows
// may be shorter). A workgroup owns a group; NCH 16-element units per lane
// stay in registers between the group statistic and the quantization (NCH =
// 0: groups too large for registers are read twice, the second time from L2).

// f(integral_constant<int, k>) for k = 0 .. N-1, expanded at compile time (an
// unroll pragma alone can leave the loop rolled, and a register array indexed
// by a loop variable then lives in scratch memory).
template <class Fn, int... K>
__device__ __forceinline__ void static_for_seq(Fn&& f, std::integer_sequence<int, K...>) {
  (f(std::integral_constant<int, K>{}), ...);
}
template <int N, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

template <int DT>
__device__ __forceinline__ void load_tile(const void* x, int64_t e0, int cnt, bool full, float* v) {
  if (full) {
    Raw<DT> r;
    raw_load<DT>(r, x, e0);
    raw_to_float<DT>(r, v);
  } else {
    load_partial<DT>(x, e0, cnt, v);
  }
}

template <int DT, int F, int ODT, int NCH>
__global__ void __launch_bounds__(kThreads) k_row(Args a) {
  __shared__ float sh[2][4];
  const bool sym = a.sym != 0;
  const Mode md{a.pow2 != 0, sym, a.rnd == LQ_RNA};
  const int tid = threadIdx.x;
  const bool vec = (a.cols & 15) == 0;
  const bool tiles = a.tile_rows > 0;
  const int64_t seg = tiles ? a.tile_cols : a.cols;          // elements per segment
  const int64_t nsu = (seg + 15) >> 4;                       // units per segment
  const int64_t tpb = tiles ? a.cols / seg : 1;              // groups per band of rows
  const int64_t ngroups = tiles ? (a.rows + a.tile_rows - 1) / a.tile_rows * tpb : a.rows;
  constexpr int R = NCH > 0 ? NCH : 1;
  double acc_e = 0.0, acc_s = 0.0;
  uint32_t bad = 0;
  for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
    int64_t row0 = g, col0 = 0, nseg = 1;
    if (tiles) {
      const int64_t band = g / tpb;
      row0 = band * a.tile_rows;
      col0 = (g - band * tpb) * seg;
      nseg = a.rows - row0 < a.tile_rows ? a.rows - row0 : a.tile_rows;
    }
    const int64_t nu = nseg * nsu;
    // unit tt: segment tt / nsu (a power of two with tiles), 16 elements at
    // offset 16 * (tt % nsu) inside it
    auto unit = [&](int64_t tt, int64_t& e0, int& cnt) __attribute__((always_inline)) {
      // (a rotation group is n / 16 consecutive units of one row segment)
      const int64_t s = tiles ? (tt >> a.unit_shift) : 0;
      const int64_t off = (tiles ? (tt & (nsu - 1)) : tt) << 4;
      e0 = (row0 + s) * a.cols + col0 + off;
      cnt = (int)(seg - off >= 16 ? 16 : seg - off);
    };
    float x[R][16];
    float am = 0.0f, mn = __builtin_inff(), mx = -__builtin_inff();
    // pass 1: statistic of the group
    auto stat_unit = [&](int64_t tt, float* v) __attribute__((always_inline)) {
      int64_t e0 = 0;
      int cnt = 0;
      if (tt < nu) unit(tt, e0, cnt);
      load_tile<DT>(a.x, e0, cnt, vec && cnt == 16, v);   // cnt = 0: zeros, no access
      if (a.had) rot_forward(v, rot_of(a, e0));
#pragma unroll
      for (int i = 0; i < 16; i++) {
        if (i < cnt) {
          am = fmaxf(am, fabsf(v[i]));
          mn = fminf(mn, v[i]);
          mx = fmaxf(mx, v[i]);
        }
      }
    };
    if constexpr (NCH > 0) {
      // expanded at compile time, so x stays in registers
      static_for<NCH>([&](auto k) __attribute__((always_inline)) { stat_unit(tid + (int64_t)k * kThreads, x[k]); });
    } else {
      for (int64_t tt = tid; tt < nu; tt += kThreads) stat_unit(tt, x[0]);
    }
    Scale sc;
    if (a.given) {
      sc = scale_load(a.scales, a.zeros, g, a.scale_fmt, sym, true);
    } else {
      if (sym) {
        sc = scale_sym<F>(block_reduce_max(am, sh[0]), a.scale_fmt);
      } else {
        const float rmx = block_reduce_max(mx, sh[0]);
        const float rmn = block_reduce_min(mn, sh[1]);
        sc = scale_asym<F>(rmn, rmx, a.scale_fmt, a.rnd);
      }
      if (tid == 0) scale_store(a.scales, a.zeros, g, sc, a.scale_fmt, sym);
    }
    // pass 2: quantize
    auto quant_unit = [&](int64_t tt, float* v, bool loaded) __attribute__((always_inline)) {
      int64_t e0;
      int cnt;
      unit(tt, e0, cnt);
      const bool full = vec && cnt == 16;
      const Rot rot = rot_of(a, e0);
      if (!loaded) {
        load_tile<DT>(a.x, e0, cnt, full, v);
        if (a.had) rot_forward(v, rot);
      }
      tile_quant_store<F, ODT, TL_NONE>(a, md, sc, e0, full ? 16 : cnt, ArrX{v}, acc_e, acc_s, bad, nullptr, rot);
    };
    if constexpr (NCH > 0) {
      static_for<NCH>([&](auto k) __attribute__((always_inline)) {
        if (tid + (int64_t)k * kThreads < nu) quant_unit(tid + (int64_t)k * kThreads, x[k], true);
      });
    } else {
      for (int64_t tt = tid; tt < nu; tt += kThreads) quant_unit(tt, x[0], false);
    }
  }
  if (a.qsnr) qsnr_partial(a, acc_e, acc_s, bad);
}

// ---------------------------------------------------------------- statistic
// Per-tensor max|x| (and min, max) of the (rotated) tensor: per-workgroup
// partials (at most kStatParts), combined by each workgroup of the kernel
// that quantizes. A pure read stream in 1024-thread workgroups, each lane
// with kStatUnroll 16-byte loads in flight. Without rotation the tensor is
// read as consecutive 16-byte vectors, consecutive lanes taking consecutive
// vectors (each load instruction covers 1 KB of whole cache lines); under a
// rotation, whose groups must sit in one lane, as 16-element tiles, one per
// lane. Two loads per lane rather than eight: on C4's bf16 tensor the
// two-level calls took 148-149 us against 154-155 with eight loads of tiles
// (both load orders of a one-box A/B), in line with a read-only probe that
// streamed fastest with few loads in flight per lane (6.25 TB/s with one,
// 5.4 with eight). Elements past the last whole tile or vector are read one
// by one; slots past the end of the tensor read as zeros, which move neither
// max|x| nor the [min(min x, 0), max(max x, 0)] range the scales use.
constexpr int kStatThreads = 1024;
constexpr int kStatUnroll = 2;

__device__ __forceinline__ void stat_add(float v, float& am, float& mn, float& mx) {
  am = fmaxf(am, fabsf(v));
  mn = fminf(mn, v);
  mx = fmaxf(mx, v);
}
// The values of one 32-bit word of the input: one fp32, or two 16-bit values.
template <int DT>
__device__ __forceinline__ void stat_add_word(uint32_t w, float& am, float& mn, float& mx) {
  if constexpr (DT == LQ_F32) {
    stat_add(__uint_as_float(w), am, mn, mx);
  } else if constexpr (DT == LQ_BF16) {
    stat_add(__uint_as_float(w << 16), am, mn, mx);
    stat_add(__uint_as_float(w & 0xFFFF0000u), am, mn, mx);
  } else {
    stat_add((float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)), am, mn, mx);
    stat_add((float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)), am, mn, mx);
  }
}

// Wave-wide max / min as a wave-uniform value (DPP within rows of 16 lanes,
// then the four row results read out).
template <bool MAX>
__device__ __forceinline__ float wave_reduce_uniform(float v) {
  v = MAX ? group_max(v, 16) : group_min(v, 16);
  float r[4];
#pragma unroll
  for (int i = 0; i < 4; i++) r[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * i));
  return MAX ? fmaxf(fmaxf(r[0], r[1]), fmaxf(r[2], r[3])) : fminf(fminf(r[0], r[1]), fminf(r[2], r[3]));
}

// ROT: 0 no rotation, 16 the 16-point rotation (in-lane only), 1024 any size.
// The grid walks the tensor from its end to its start: the quantizing kernel
// that follows reads it from the start, so its first reads find the part this
// pass read last still in the Infinity Cache (a tensor larger than that cache
// is otherwise read twice from HBM). Measured on c4t (NVFP4 / NVINT4
// two-level on C4's tensor): 155.8-156.9 us per call this way, 173.7-174.4
// us walking forward. The extrema do not depend on the order.
template <int DT, int ROT>
__global__ void __launch_bounds__(kStatThreads) k_stat(Args a) {
  constexpr bool HAD = ROT != 0;
  constexpr int esz = DT == LQ_F32 ? 4 : 2;
  constexpr bool kVectors = !HAD;
  constexpr int kWaves = kStatThreads / 64;
  __shared__ float sh[3][kWaves];
  const int tid = threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kStatThreads;
  const int64_t g = (int64_t)blockIdx.x * kStatThreads + tid;
  float am = 0.0f, mn = __builtin_inff(), mx = -__builtin_inff();
  int64_t done;   // elements covered by whole vectors or tiles
  if constexpr (kVectors) {
    const u32x4* p = (const u32x4*)a.x;
    const int64_t nvec = a.n * esz / 16;
    done = nvec * 16 / esz;
    for (int64_t base = g; base < nvec; base += kStatUnroll * stride) {
      u32x4 w[kStatUnroll];
#pragma unroll
      for (int j = 0; j < kStatUnroll; j++) {
        const int64_t v = base + j * stride;
        if (v < nvec) w[j] = gload(p + (nvec - 1 - v));
        else w[j] = (u32x4){0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < kStatUnroll; j++)
#pragma unroll
        for (int k = 0; k < 4; k++) stat_add_word<DT>(w[j][k], am, mn, mx);
    }
  } else {
    constexpr int kTiles = kStatUnroll / (DT == LQ_F32 ? 4 : 2) > 0 ? kStatUnroll / (DT == LQ_F32 ? 4 : 2) : 1;
    const int64_t ntiles = a.n >> 4;
    // whole rows of 64 tiles are walked backwards, the lanes of a row in
    // ascending order, so that a rotation group wider than one tile sits in
    // its lanes as the forward pass places it
    const int64_t nrows = (ntiles + 63) >> 6;
    const int64_t span = nrows << 6;
    done = ntiles << 4;
    for (int64_t base = g; base < span; base += kTiles * stride) {
      Raw<DT> r[kTiles];
      int64_t tile[kTiles];   // the tile a lane takes, or -1 past the end
#pragma unroll
      for (int j = 0; j < kTiles; j++) {
        const int64_t t = base + j * stride;
        const int64_t rt = ((nrows - 1 - (t >> 6)) << 6) | (t & 63);
        tile[j] = (t < span && rt < ntiles) ? rt : -1;
        if (tile[j] >= 0) raw_load<DT>(r[j], a.x, tile[j] << 4);
        else
#pragma unroll
          for (int i = 0; i < (DT == LQ_F32 ? 4 : 2); i++) r[j].w[i] = (u32x4){0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < kTiles; j++) {
        float x[16];
        raw_to_float<DT>(r[j], x);
        if (HAD) rot_forward<ROT>(x, rot_of(a, tile[j] >= 0 ? tile[j] << 4 : 0));   // zeros past the end
#pragma unroll
        for (int i = 0; i < 16; i++) stat_add(x[i], am, mn, mx);
      }
    }
  }
  // the rotation needs whole groups of 16 (n is then a multiple of 16)
  if (!HAD && done + g < a.n) stat_add(load_one<DT>(a.x, done + g), am, mn, mx);
  am = wave_reduce_uniform<true>(am);
  mn = wave_reduce_uniform<false>(mn);
  mx = wave_reduce_uniform<true>(mx);
  if ((tid & 63) == 0) {
    sh[0][tid >> 6] = am;
    sh[1][tid >> 6] = mn;
    sh[2][tid >> 6] = mx;
  }
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int i = 1; i < kWaves; i++) {
      am = fmaxf(am, sh[0][i]);
      mn = fminf(mn, sh[1][i]);
      mx = fmaxf(mx, sh[2][i]);
    }
    a.ws->part_amax[blockIdx.x] = am;
    a.ws->part_min[blockIdx.x] = mn;
    a.ws->part_max[blockIdx.x] = mx;
  }
}

// Workgroups of k_stat for n elements: two 16-byte loads per lane (a finer
// grid than one full round of kStatUnroll measured faster on small tensors),
// at most kStatParts.
inline int stat_grid(int64_t n, int dt) {
  const int64_t vecs = n * (dt == LQ_F32 ? 4 : 2) / 16 + 1;
  const int64_t per_wg = (int64_t)kStatThreads * 2;
  const int64_t wg = (vecs + per_wg - 1) / per_wg;
  return (int)(wg < kStatParts ? wg : kStatParts);
}

// ---------------------------------------------------------------- dequantize
// gran: 0 tensor, 1 channel, 2 block (block = 16 << block_shift), 3 2-D tile.
template <int F>
__global__ void __launch_bounds__(kThreads) k_dequant(Args a, int gran) {
  const bool sym = a.sym != 0;
  const int64_t ntiles = (a.n + 15) >> 4;
  const bool row_tiles = (a.cols & 15) == 0;  // channel: a tile never spans two rows
  for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < ntiles; t += (int64_t)gridDim.x * kThreads) {
    const int64_t e0 = t << 4;
    const int cnt = (a.n - e0 >= 16) ? 16 : (int)(a.n - e0);
    Codes c;
    c.w[0] = c.w[1] = c.w[2] = c.w[3] = 0u;
    if (Fmt<F>::six) {
      const uint8_t* p = a.codes + e0 / 4 * 3;   // e0 is a multiple of 16 here
      if (cnt == 16) {
        const uint32_t* q = (const uint32_t*)p;
        c.w[0] = q[0]; c.w[1] = q[1]; c.w[2] = q[2];
      } else {
#pragma unroll
        for (int i = 0; i < 12; i++)
          if (4 * i < 3 * cnt) c.w[i / 4] |= (uint32_t)p[i] << (8 * (i % 4));
      }
    } else if (Fmt<F>::four) {
      if (cnt == 16) {
        const u32x2 u = *(const u32x2*)(a.codes + e0 / 2);
        c.w[0] = u[0]; c.w[1] = u[1];
      } else {
#pragma unroll
        for (int i = 0; i < 8; i++)
          if (2 * i < cnt) c.w[i / 4] |= (uint32_t)a.codes[e0 / 2 + i] << (8 * (i % 4));
      }
    } else {
      if (cnt == 16) {
        const u32x4 u = *(const u32x4*)(a.codes + e0);
        c.w[0] = u[0]; c.w[1] = u[1]; c.w[2] = u[2]; c.w[3] = u[3];
      } else {
#pragma unroll
        for (int i = 0; i < 16; i++)
          if (i < cnt) c.w[i / 4] |= (uint32_t)a.codes[e0 + i] << (8 * (i % 4));
      }
    }
    float d[16], xh[16];
    decode_tile<F>(c, d);
    const float tls = a.tscale ? *a.tscale : 1.0f;   // two-level: x = (value * s_block) * S
    if (gran != 1 || row_tiles) {
      int64_t idx = (gran == 2) ? (t >> a.block_shift) : (gran == 1 ? e0 / a.cols : 0);
      if (gran == 3) {
        // 2-D tiles: a unit of 16 never crosses a tile (tile_cols >= 16, cols % 16 == 0)
        const int64_t row = e0 / a.cols;
        idx = row / a.tile_rows * (a.cols / a.tile_cols) + (e0 - row * a.cols) / a.tile_cols;
      }
      const Scale sc = scale_load(a.scales, a.zeros, idx, a.scale_fmt, sym, false);
#pragma unroll
      for (int i = 0; i < 16; i++)
        xh[i] = (sc.s == 0.0f) ? 0.0f : (sym ? d[i] * sc.s : sc.s * (d[i] - sc.zp));
      if (a.tscale) {
#pragma unroll
        for (int i = 0; i < 16; i++) xh[i] = xh[i] * tls;
      }
    } else {
      for (int i = 0; i < 16; i++) {
        const int64_t ei = e0 + (i < cnt ? i : 0);   // lanes past the end read a valid scale
        const Scale sc = scale_load(a.scales, a.zeros, ei / a.cols, a.scale_fmt, sym, false);
        xh[i] = (i >= cnt || sc.s == 0.0f) ? 0.0f : (sym ? d[i] * sc.s : sc.s * (d[i] - sc.zp));
      }
    }
    if (a.had) rot_inverse(xh, rot_of(a, e0));
    store_y(a.y, e0, cnt, xh, a.out_dt);
  }
}

// ---------------------------------------------------------------- helpers
static __global__ void k_fill_zero(uint32_t* p, int64_t nwords) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

static __global__ void k_empty_result(lq_result* res) {
  if (threadIdx.x == 0) {
    res->err2 = 0.0;
    res->sig2 = 0.0;
    res->qsnr_db = __builtin_inf();
    res->nonfinite = 0u;
    res->reserved = 0u;
  }
}

// ---------------------------------------------------------------- launchers
// Launch plans: while a host thread has a PlanRecorder installed, every
// launch wrapper appends the name of the kernel it would launch (as the HIP
// runtime's demangler prints it, the name profilers report) and the grid
// and block sizes, instead of launching. lq_call_kernels uses it to report the kernels
// of a call from this dispatch code itself.
struct PlanRecorder {
  char* buf;      // may be null (count only)
  size_t cap;     // bytes at buf
  size_t len;     // bytes written, without the terminating NUL
  int count;      // kernels recorded
};
extern thread_local PlanRecorder* g_plan;

__attribute__((format(printf, 3, 4))) inline hipError_t plan_add(int nwg, int nthreads, const char* fmt, ...) {
  PlanRecorder* r = g_plan;
  char line[256];
  va_list ap;
  va_start(ap, fmt);
  int n = vsnprintf(line, sizeof line, fmt, ap);
  va_end(ap);
  if (n < 0) n = 0;
  char grid[32];
  const int g = snprintf(grid, sizeof grid, "\t%d\t%d\n", nwg, nthreads);
  if (r->buf && r->len + (size_t)n + (size_t)g < r->cap) {
    memcpy(r->buf + r->len, line, (size_t)n);
    memcpy(r->buf + r->len + n, grid, (size_t)g);
    r->len += (size_t)n + (size_t)g;
    r->buf[r->len] = '\0';
  }
  r->count++;
  return hipSuccess;
}
inline const char* tf(bool b) { return b ? "true" : "false"; }

template <int DT, int F, int ODT, int MODE>
hipError_t launch_flat(const Args& a, int nwg, hipStream_t s) {
  if (g_plan) return plan_add(nwg, kThreads, "void lqd::k_flat<%d, %d, %d, %d>(lqd::Args)", DT, F, ODT, MODE);
  hipLaunchKernelGGL((k_flat<DT, F, ODT, MODE>), dim3(nwg), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}
template <int DT, int F, int ODT, int NCH>
hipError_t launch_row(const Args& a, int nwg, hipStream_t s) {
  if (g_plan) return plan_add(nwg, kThreads, "void lqd::k_row<%d, %d, %d, %d>(lqd::Args)", DT, F, ODT, NCH);
  hipLaunchKernelGGL((k_row<DT, F, ODT, NCH>), dim3(nwg), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}
template <int DT>
hipError_t launch_stat(const Args& a, int nwg, hipStream_t s) {
  const int rot = a.had > 16 ? 1024 : a.had ? 16 : 0;
  if (g_plan) return plan_add(nwg, kStatThreads, "void lqd::k_stat<%d, %d>(lqd::Args)", DT, rot);
  if (rot == 1024) hipLaunchKernelGGL((k_stat<DT, 1024>), dim3(nwg), dim3(kStatThreads), 0, s, a);
  else if (rot == 16) hipLaunchKernelGGL((k_stat<DT, 16>), dim3(nwg), dim3(kStatThreads), 0, s, a);
  else hipLaunchKernelGGL((k_stat<DT, 0>), dim3(nwg), dim3(kStatThreads), 0, s, a);
  return hipGetLastError();
}
template <int F>
hipError_t launch_dequant(const Args& a, int gran, int nwg, hipStream_t s) {
  if (g_plan) return plan_add(nwg, kThreads, "void lqd::k_dequant<%d>(lqd::Args, int)", F);
  hipLaunchKernelGGL((k_dequant<F>), dim3(nwg), dim3(kThreads), 0, s, a, gran);
  return hipGetLastError();
}
inline hipError_t launch_finish(const Workspace* ws, int parts, lq_result* res, hipStream_t s) {
  if (g_plan) return plan_add(1, kThreads, "lqd::k_finish(lqd::Workspace const*, int, lq_result*)");
  hipLaunchKernelGGL(k_finish, dim3(1), dim3(kThreads), 0, s, ws, parts, res);
  return hipGetLastError();
}
inline hipError_t launch_empty_result(lq_result* res, hipStream_t s) {
  if (g_plan) return plan_add(1, 64, "lqd::k_empty_result(lq_result*)");
  hipLaunchKernelGGL(k_empty_result, dim3(1), dim3(64), 0, s, res);
  return hipGetLastError();
}

typedef hipError_t (*flat_fn)(const Args&, int, hipStream_t);
typedef hipError_t (*dq_fn)(const Args&, int, int, hipStream_t);

// Kernel tables, filled by the instantiation units (one per input and output
// dtype): flat[format][FLAT_* mode], row[format][slot] with slots for 1, 2 or 4
// register-resident tiles per lane and the two-pass row.
struct KernelSet {
  flat_fn flat[kFormats][3];
  flat_fn row[kFormats][4];
};

}  // namespace lqd
