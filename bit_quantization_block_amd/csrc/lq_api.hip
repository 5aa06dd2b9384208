// lq_api.hip — the C ABI of liblq (declared in include/lq.h): argument checks,
// workspace and grid sizing, and kernel dispatch. Every check runs before the
// first launch, so a call that fails writes nothing.
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <numeric>
#include <mutex>

#include "lq.h"
#include "lq_fast.h"
#include "lq_kernels.h"

namespace lqd {
#define LQ_DECLARE(d, o) void kernels_##d##_##o(KernelSet& k);
LQ_DECLARE(0, 0) LQ_DECLARE(0, 1) LQ_DECLARE(0, 2)
LQ_DECLARE(1, 0) LQ_DECLARE(1, 1) LQ_DECLARE(1, 2)
LQ_DECLARE(2, 0) LQ_DECLARE(2, 1) LQ_DECLARE(2, 2)
#undef LQ_DECLARE
void fast_kernels_0(FastSet& k);
void fast_kernels_1(FastSet& k);

thread_local PlanRecorder* g_plan = nullptr;
}  // namespace lqd

using namespace lqd;

namespace {

struct Tables {
  KernelSet k[3][3];   // [input dtype][output dtype]
  FastSet fast[2];     // same input and output dtype: fp32, bf16
  LcSet lc;            // bf16, lane-contiguous layout
  fast_fn h16[kFormats];   // bf16, 4-bit E4M3 blocks of 16 under the 16-point rotation
  fast_fn h16_two[kFormats];   // the same under a two-level (fp32 tensor) scale
  flat_fn stat[3];
  dq_fn dq[kFormats];
  Tables() {
    kernels_0_0(k[0][0]); kernels_0_1(k[0][1]); kernels_0_2(k[0][2]);
    kernels_1_0(k[1][0]); kernels_1_1(k[1][1]); kernels_1_2(k[1][2]);
    kernels_2_0(k[2][0]); kernels_2_1(k[2][1]); kernels_2_2(k[2][2]);
    fast_kernels_0(fast[0]);
    fast_kernels_1(fast[1]);
    lc_kernels(lc);
    h16_kernels(h16, h16_two);
    stat[0] = &launch_stat<LQ_F32>;
    stat[1] = &launch_stat<LQ_BF16>;
    stat[2] = &launch_stat<LQ_F16>;
    dq[LQ_INT8] = &launch_dequant<LQ_INT8>;
    dq[LQ_INT4] = &launch_dequant<LQ_INT4>;
    dq[LQ_E4M3] = &launch_dequant<LQ_E4M3>;
    dq[LQ_E5M2] = &launch_dequant<LQ_E5M2>;
    dq[LQ_E2M1] = &launch_dequant<LQ_E2M1>;
    dq[LQ_E2M3] = &launch_dequant<LQ_E2M3>;
    dq[LQ_E3M2] = &launch_dequant<LQ_E3M2>;
  }
};
const Tables& tables() {
  static const Tables t;
  return t;
}

// Workgroups per compute unit for grid-stride launches; 256 CUs on MI355X.
#ifndef LQ_WG_PER_CU
#define LQ_WG_PER_CU 32
#endif
constexpr int kWgPerCu = LQ_WG_PER_CU;

// Process-wide cap set by lq_set_grid_limit (0: none).
std::atomic<int> g_grid_limit{0};

// Compute units of the current device, cached per device (calls from several
// host threads may fill it together; they store the same value); with no
// device (a launch plan asked for on a host without a GPU), MI355X's 256.
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

int capped(int64_t c) {
  const int lim = g_grid_limit.load(std::memory_order_relaxed);
  return (lim > 0 && lim < c) ? lim : (int)c;
}

// Grid cap of the grid-stride kernels: 32 workgroups per CU, at most kMaxWG.
int grid_cap() { return capped(std::min<int64_t>((int64_t)device_cus() * kWgPerCu, kMaxWG)); }

// Grid cap of the lane-contiguous kernels, which finish their QSNR in-kernel
// at any grid size: one 1024-element chunk per wave up to 128 workgroups of
// 4 waves per CU. Measured on C4's tensor: the NVFP4 / NVINT4 kernels under
// the 16-point rotation took 101.8-102.9 us in one pass over 32768
// workgroups against 107-108 us in four over 8192, and the bare traffic
// pattern 102.9 against 108.1 us.
constexpr int kWgPerCuInline = 128;
int grid_cap_inline() {
  return capped(std::min<int64_t>((int64_t)device_cus() * kWgPerCuInline, kMaxWGInline));
}

// Workgroups for `needed` units of work (one workgroup's share each) under
// `cap`: when the cap forces several passes, the fewest workgroups that take
// that many passes, so every workgroup runs the same number of them (capped
// at the limit instead, C3's lane-contiguous and tile-per-lane kernels left a
// quarter of their waves a second pass while the rest idled).
int balanced_grid(int64_t needed, int64_t cap) {
  if (needed <= cap) return (int)needed;
  const int64_t passes = (needed + cap - 1) / cap;
  return (int)((needed + passes - 1) / passes);
}

// Grid of a tile-per-lane kernel under a rotation with random signs: one pass
// over the tensor, or a stride (workgroups x nt tiles of 16 elements) that is
// a multiple of cols, so that every tile a lane takes sits at the same column
// and the kernel reads that lane's 16 sign bits once. The fewest workgroups,
// a multiple of m = cols / gcd(cols, 16 nt), that take as few passes as the
// largest such grid under the cap; 0 when m itself exceeds the cap.
int signed_rotation_grid(int64_t needed, int64_t cap, int nt, int64_t cols) {
  if (needed <= cap) return (int)needed;
  const int64_t m = cols / std::gcd(cols, (int64_t)nt * 16);
  if (m > cap) return 0;
  const int64_t largest = cap / m * m;
  const int64_t passes = (needed + largest - 1) / largest;
  const int64_t per_pass = (needed + passes - 1) / passes;
  return (int)((per_pass + m - 1) / m * m);
}

// (FP6 lane-contiguous grids take the same caps as the other formats: with
// the native conversion, c7's one-pass grid of 8192 workgroups took 31.9-32.0
// us per call against 36.4-36.6 us capped at 1024, and 34.5 / 37.2 / 38.7 us
// at 4096 / 2048 / 1536, one box. The bit-level encoder had measured the
// other way, 41-43 us at 1024 against 44-48 us at 8192.)

// Lane-contiguous kernels whose every workgroup first folds the statistic
// pass's partials (per-tensor and two-level scales) are capped lower: the
// fold is a dependent read and a barrier at each workgroup's start. Measured
// on c4t (C4's tensor, NVFP4 / NVINT4 two-level, statistic pass included):
// 153-157 us per call at 2048 workgroups, 158-165 at 8192, 178-209 at 32768.
constexpr int kFoldLcMaxWG = 2048;

bool is_int(int f) { return f == LQ_INT8 || f == LQ_INT4; }
bool is_four(int f) { return f == LQ_INT4 || f == LQ_E2M1; }
bool is_six(int f) { return f == LQ_E2M3 || f == LQ_E3M2; }
bool aligned(const void* p) { return ((uintptr_t)p & 15u) == 0u; }

int check_desc(const lq_desc* d) {
  if (!d) return LQ_ERR_NULL;
  if (d->format < LQ_INT8 || d->format > LQ_E3M2) return LQ_ERR_BAD_DESC;
  if (d->gran < LQ_PER_TENSOR || d->gran > LQ_PER_TILE) return LQ_ERR_BAD_DESC;
  if (d->scale_fmt < LQ_SCALE_F32 || d->scale_fmt > LQ_SCALE_E4M3) return LQ_ERR_BAD_DESC;
  if (d->symmetric != 0 && d->symmetric != 1) return LQ_ERR_BAD_DESC;
  if (d->rounding != LQ_RNE && d->rounding != LQ_RNA) return LQ_ERR_BAD_DESC;
  if (d->in_dtype < LQ_F32 || d->in_dtype > LQ_F16) return LQ_ERR_BAD_DESC;
  if (d->out_dtype < LQ_F32 || d->out_dtype > LQ_F16) return LQ_ERR_BAD_DESC;
  if (d->hadamard != 0 && d->hadamard != 16 && d->hadamard != 32 && d->hadamard != 64 && d->hadamard != 128 &&
      d->hadamard != 256 && d->hadamard != 512 && d->hadamard != 1024)
    return LQ_ERR_BAD_DESC;
  // a tile's rotation groups must lie inside it (each tile is one workgroup)
  if (d->gran == LQ_PER_TILE && d->hadamard > 16 && d->block % d->hadamard != 0) return LQ_ERR_UNSUPPORTED;
  if (d->scale_source != LQ_SCALE_DYNAMIC && d->scale_source != LQ_SCALE_GIVEN) return LQ_ERR_BAD_DESC;
  // a zero point is defined for the integer affine map only, with a scale that
  // is not a power of two / E4M3 block scale
  if (!d->symmetric && (!is_int(d->format) || (d->scale_fmt != LQ_SCALE_F32 && d->scale_fmt != LQ_SCALE_F16)))
    return LQ_ERR_BAD_DESC;
  // two-level scaling: an FP32 tensor scale above symmetric E4M3 block scales
  if (d->two_level != 0 && d->two_level != 1) return LQ_ERR_BAD_DESC;
  if (d->two_level && (d->gran != LQ_PER_BLOCK || d->scale_fmt != LQ_SCALE_E4M3 || !d->symmetric))
    return LQ_ERR_BAD_DESC;
  if (d->gran == LQ_PER_TILE && (d->tile_rows <= 0 || d->tile_rows > 65536)) return LQ_ERR_BAD_DESC;
  if (d->gran == LQ_PER_BLOCK || d->gran == LQ_PER_TILE) {
    if (d->block <= 0) return LQ_ERR_BAD_DESC;
    if (d->block != 16 && d->block != 32 && d->block != 64 && d->block != 128 && d->block != 256)
      return LQ_ERR_UNSUPPORTED;
  }
  return LQ_OK;
}

int check_shape(const lq_desc* d, int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return LQ_ERR_SHAPE;
  if (cols > 0 && rows > (INT64_C(1) << 58) / cols) return LQ_ERR_SHAPE;
  if ((d->gran == LQ_PER_BLOCK || d->gran == LQ_PER_TILE) && cols % d->block != 0) return LQ_ERR_SHAPE;
  if (is_four(d->format) && (cols & 1)) return LQ_ERR_SHAPE;
  if (is_six(d->format) && (cols & 3)) return LQ_ERR_SHAPE;
  if (d->hadamard && cols % d->hadamard != 0) return LQ_ERR_SHAPE;
  return LQ_OK;
}

int64_t n_scales(const lq_desc* d, int64_t rows, int64_t cols) {
  if (d->gran == LQ_PER_TENSOR) return 1;
  if (d->gran == LQ_PER_CHANNEL) return rows;
  if (d->gran == LQ_PER_TILE) return (rows + d->tile_rows - 1) / d->tile_rows * (cols / d->block);
  return rows * (cols / d->block);
}
size_t scale_size(int sf) { return sf == LQ_SCALE_F32 ? 4 : sf == LQ_SCALE_F16 ? 2 : 1; }

// Two-level: byte offset of the fp32 S in the scales buffer (after the E4M3
// block scales, at the next multiple of 16).
size_t tscale_offset(const lq_desc* d, int64_t rows, int64_t cols) {
  return ((size_t)n_scales(d, rows, cols) + 15) & ~(size_t)15;
}

int log2i(int v) {
  int s = 0;
  while ((1 << s) < v) s++;
  return s;
}

// 1/sqrt(n) rounded to binary32 for n = 2^l: 2^-(l/2), times RN(1/sqrt(2))
// (0x1.6a09e6p-1) for odd l; scaling by a power of two commutes with rounding.
float rotation_scale(int n) {
  if (n <= 0) return 1.0f;
  const int l = log2i(n);
  const float c = ldexpf(1.0f, -(l / 2));
  return (l & 1) ? c * 0x1.6a09e6p-1f : c;
}

// Tag for the partials of one call of the specialised per-block kernel: the
// collecting workgroup accepts a partial only when its tag matches, so stale
// words of earlier calls (or an uninitialised workspace) are never summed.
uint32_t next_epoch() {
  static std::atomic<uint32_t> counter{0};
  uint32_t e = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  if (e == 0) e = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  return e;
}

Args make_args(const lq_desc* d, const void* x, int64_t rows, int64_t cols, void* codes, void* scales,
               void* zeros, void* y, int unrotate, lq_result* res, void* ws) {
  Args a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.codes = (uint8_t*)codes;
  a.scales = scales;
  a.zeros = zeros;
  a.y = y;
  a.rows = rows;
  a.cols = cols;
  a.n = rows * cols;
  a.block_lanes = d->gran == LQ_PER_BLOCK ? d->block / 16 : 1;
  a.block_shift = log2i(a.block_lanes);
  if (d->gran == LQ_PER_TILE) {
    a.tile_rows = d->tile_rows;
    a.tile_cols = d->block;
    a.unit_shift = log2i(d->block / 16);
  }
  a.scale_fmt = d->scale_fmt;
  a.sym = d->symmetric;
  a.rnd = d->rounding;
  a.out_dt = d->out_dtype;
  a.had = d->hadamard;
  a.rot_c = rotation_scale(d->hadamard);
  a.signs = (const uint32_t*)d->signs;
  a.unrotate = unrotate ? 1 : 0;
  a.given = d->scale_source == LQ_SCALE_GIVEN;
  a.qsnr = res != nullptr;
  a.pow2 = d->scale_fmt == LQ_SCALE_UE8M0;
  a.maybe_ieee = d->scale_fmt == LQ_SCALE_F32 || d->scale_source == LQ_SCALE_GIVEN;
  a.ws = (Workspace*)ws;
  a.res = res;
  a.tscale = (d->two_level && scales) ? (float*)((char*)scales + tscale_offset(d, rows, cols)) : nullptr;
  return a;
}

// Arguments of the specialised kernels (k_fast, k_lc, k_row_lc); `ntiles`,
// `block_lanes` and `block_shift` are in the kernel's own units.
FastArgs fast_args(const Args& a, int64_t ntiles, int32_t block_lanes, int32_t block_shift) {
  FastArgs fa;
  fa.x = a.x;
  fa.codes = a.codes;
  fa.scales = a.scales;
  fa.zeros = a.zeros;
  fa.y = a.y;
  fa.ws = a.ws;
  fa.res = a.res;
  fa.epoch = next_epoch();
  fa.ntiles = ntiles;
  fa.block_lanes = block_lanes;
  fa.block_shift = block_shift;
  fa.unrotate = a.unrotate;
  fa.stat_parts = a.stat_parts;
  fa.tscale = a.tscale;
  fa.had = a.had;
  fa.rot_c = a.rot_c;
  fa.signs = a.signs;
  fa.cols = a.cols;
  fa.finish_inline = 0;
  fa.nwork = 0;
  return fa;
}

// One-row tiles are per-block scaling (the same scales in the same order):
// they take the per-block kernels.
lq_desc effective_desc(const lq_desc* d) {
  lq_desc e = *d;
  if (e.gran == LQ_PER_TILE && e.tile_rows == 1) e.gran = LQ_PER_BLOCK;
  return e;
}

// Shared body of quantize / fake-quant / hadamard-quant.
int run_quant(const lq_desc* desc, const void* x, int64_t rows, int64_t cols, void* codes, void* scales,
              void* zeros, void* y, int unrotate, lq_result* res, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  const lq_desc de = effective_desc(desc);
  const lq_desc* d = &de;
  rc = check_shape(d, rows, cols);
  if (rc) return rc;
  const int64_t n = rows * cols;
  const bool given = d->scale_source == LQ_SCALE_GIVEN;
  if (n > 0 && !x) return LQ_ERR_NULL;
  if (given && (!scales || (!d->symmetric && !zeros))) return LQ_ERR_NULL;
  for (const void* p : {x, (const void*)codes, (const void*)scales, (const void*)zeros, (const void*)y,
                        (const void*)res, (const void*)ws})
    if (p && !aligned(p)) return LQ_ERR_ALIGN;
  const bool needs_ws = res != nullptr || ((d->gran == LQ_PER_TENSOR || d->two_level) && !given);
  if (needs_ws && n > 0 && (!ws || ws_bytes < sizeof(Workspace))) return LQ_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (n == 0) {
    if (res && launch_empty_result(res, s) != hipSuccess) return LQ_ERR_HIP;
    return LQ_OK;
  }
  Args a = make_args(d, x, rows, cols, codes, scales, zeros, y, unrotate, res, ws);
  const Tables& T = tables();
  const KernelSet& K = T.k[d->in_dtype][d->out_dtype];
  const int cap = grid_cap();
  const int64_t ntiles = (n + 15) / 16;
  const int64_t wg_needed = (ntiles + kThreads - 1) / kThreads;
  const int nwg = balanced_grid(wg_needed, cap);
  hipError_t e;
  int parts = nwg;
  bool finished = false;   // the main kernel wrote *res itself
  // k_flat finishes the QSNR in-kernel (its grid is at most kMaxWG)
  const bool flat_inline = res != nullptr;
  if (d->gran == LQ_PER_TENSOR && !given && d->rounding == LQ_RNE && codes && scales && y && res &&
      d->symmetric && d->scale_fmt == LQ_SCALE_F32 && d->in_dtype == LQ_BF16 && d->out_dtype == LQ_BF16 &&
      !d->hadamard && n % 1024 == 0) {
    // lane-contiguous per-tensor kernel after the statistic pass
    const int nwg_stat = stat_grid(n, d->in_dtype);
    e = T.stat[d->in_dtype](a, nwg_stat, s);
    if (e != hipSuccess) return LQ_ERR_HIP;
    const int64_t nchunks = n / 1024;
    const int cap_wide = cap >= 4 ? cap / 4 : 1;
    const bool wide = T.lc.k[d->format][LQ_SCALE_F32][1][1] != nullptr &&
                      nchunks <= (int64_t)cap_wide * (fast_threads(true) / 64);
    const int waves = fast_threads(wide) / 64;
    const int cap_lc = wide ? cap_wide : std::min(cap, kFoldLcMaxWG);
    const int64_t wg_lc = (nchunks + waves - 1) / waves;
    const int nwg_lc = balanced_grid(wg_lc, cap_lc);
    if (nchunks <= (int64_t)kFastMaxIters * nwg_lc * waves) {
      a.stat_parts = nwg_stat;
      FastArgs fa = fast_args(a, nchunks, 1, 0);
      fa.finish_inline = 1;
      e = T.lc.k[d->format][LQ_SCALE_F32][1][wide ? 1 : 0](fa, nwg_lc, s);
      finished = true;
    } else {
      a.stat_parts = nwg_stat;
      if (flat_inline) {
        a.finish_inline = 1;
        a.epoch = next_epoch();
        finished = true;
      }
      e = K.flat[d->format][FLAT_TENSOR](a, nwg, s);
    }
  } else if (d->gran == LQ_PER_TENSOR) {
    if (!given) {
      // the statistic's partials are combined by every k_flat workgroup
      const int nwg_stat = stat_grid(n, d->in_dtype);
      e = T.stat[d->in_dtype](a, nwg_stat, s);
      if (e != hipSuccess) return LQ_ERR_HIP;
      a.stat_parts = nwg_stat;
    }
    if (flat_inline) {
      a.finish_inline = 1;
      a.epoch = next_epoch();
      finished = true;
    }
    e = K.flat[d->format][FLAT_TENSOR](a, nwg, s);
  } else if (d->gran == LQ_PER_BLOCK) {
    const bool two = d->two_level != 0;
    if (two && !given) {
      // the tensor scale's statistic; every workgroup of the kernel below
      // combines its partials
      const int nwg_stat = stat_grid(n, d->in_dtype);
      e = T.stat[d->in_dtype](a, nwg_stat, s);
      if (e != hipSuccess) return LQ_ERR_HIP;
      a.stat_parts = nwg_stat;
    }
    // the specialised kernel when the call matches it: data-driven scales,
    // half-to-even rounding, every output written, same input/output dtype
    fast_fn f = nullptr;
    const bool had = d->hadamard != 0;
    const bool common = !given && d->rounding == LQ_RNE && codes && scales && y && res && (d->symmetric || zeros) &&
                        d->in_dtype == d->out_dtype;
    const int cap_wide = cap >= 4 ? cap / 4 : 1;
    fast_fn const h16 = two ? T.h16_two[d->format] : T.h16[d->format];
    if (common && d->in_dtype == LQ_BF16 && d->hadamard == 16 && !d->signs && d->block == 16 &&
        d->scale_fmt == LQ_SCALE_E4M3 && d->symmetric && h16 && n % 1024 == 0 && (unrotate == 0 || unrotate == 1)) {
      // NVFP4 / NVINT4 blocks under the 16-point rotation: lane-contiguous
      // memory access through LDS, chunks of 1024 elements, 4 waves each
      // (two-level: every workgroup folds the statistic's partials, so the
      // grid is capped as for the lane-contiguous two-level kernels)
      const int64_t nchunks = n / 1024;
      const int cap_h = two ? std::min(grid_cap_inline(), kFoldLcMaxWG) : grid_cap_inline();
      const int nwg_h = balanced_grid((nchunks + 3) / 4, cap_h);
      if (nchunks <= (int64_t)kFastMaxIters * nwg_h * 4) {
        FastArgs fa = fast_args(a, nchunks, 1, 0);
        fa.finish_inline = 1;
        e = h16(fa, nwg_h, s);
        return e == hipSuccess ? LQ_OK : LQ_ERR_HIP;
      }
    }
    if (common && d->in_dtype == LQ_BF16 && !had && d->symmetric && n % 1024 == 0) {
      // lane-contiguous layout, in chunks of 1024 elements
      const int64_t nchunks = n / 1024;
      fast_fn const* tab = two ? T.lc.two[d->format] : T.lc.k[d->format][d->scale_fmt][0];
      const bool wide = tab[1] != nullptr && nchunks <= (int64_t)cap_wide * (fast_threads(true) / 64);
      const int waves = fast_threads(wide) / 64;
      const int cap_lc = wide ? cap_wide : two ? std::min(grid_cap_inline(), kFoldLcMaxWG) : grid_cap_inline();
      const int64_t wg_lc = (nchunks + waves - 1) / waves;
      const int nwg_lc = balanced_grid(wg_lc, cap_lc);
      fast_fn g = tab[wide ? 1 : 0];
      if (g && nchunks <= (int64_t)kFastMaxIters * nwg_lc * waves) {
        FastArgs fa = fast_args(a, nchunks, d->block / 8, log2i(d->block));
        fa.finish_inline = 1;
        e = g(fa, nwg_lc, s);
        return e == hipSuccess ? LQ_OK : LQ_ERR_HIP;
      }
    }
    // wide shape when its grid covers the tensor in one pass
    const bool wide =
        fast_can_be_wide(d->in_dtype, had, d->format) && ntiles <= (int64_t)cap_wide * fast_threads(true);
    const int nt = fast_threads(wide);
    const int cap_fast = wide ? cap_wide : cap;
    const int64_t wg_fast = (ntiles + nt - 1) / nt;
    int nwg_fast = balanced_grid(wg_fast, cap_fast);
    // random signs: each lane's tiles at one column (the kernel reads the
    // lane's sign bits once); without such a grid the call takes k_flat
    bool signs_fixed = true;
    if (had && d->signs && nwg_fast < wg_fast) {
      const int g = signed_rotation_grid(wg_fast, cap_fast, nt, cols);
      signs_fixed = g > 0;
      if (signs_fixed) nwg_fast = g;
    }
    // each lane records at most kFastMaxIters out-of-range tiles
    const bool fits = ntiles <= (int64_t)kFastMaxIters * nwg_fast * nt;
    if (common && d->in_dtype != LQ_F16 && (!had || unrotate == 0 || unrotate == 1) && fits && signs_fixed) {
      const FastSet& FS = T.fast[d->in_dtype];
      if (d->hadamard > kFastMaxRot)   // narrow only (wide is false with rotation)
        f = two ? FS.wrot_two[d->format] : d->symmetric ? FS.wrot[d->format][d->scale_fmt] : nullptr;
      else
        f = two ? FS.two[d->format][had ? 1 : 0][wide ? 1 : 0]
                : FS.k[d->format][d->scale_fmt][d->symmetric ? 0 : 1][had ? 1 : 0][wide ? 1 : 0];
    }
    if (f) {
      FastArgs fa = fast_args(a, ntiles, a.block_lanes, a.block_shift);
      fa.finish_inline = 1;
      e = f(fa, nwg_fast, s);
      finished = true;
    } else {
      if (flat_inline) {
        a.finish_inline = 1;
        a.epoch = next_epoch();
        finished = true;
      }
      e = K.flat[d->format][two ? FLAT_TWO : FLAT_BLOCK](a, nwg, s);
    }
  } else if (d->gran == LQ_PER_TILE) {
    // one workgroup per tile; tiles of up to 4 units of 16 per lane (128x128
    // and smaller) stay in registers between the statistic and quantizing
    const int64_t units = (int64_t)d->tile_rows * (d->block / 16);
    const int64_t per_lane = (units + kThreads - 1) / kThreads;
    const int slot = per_lane <= 1 ? 0 : per_lane <= 2 ? 1 : per_lane <= 4 ? 2 : 3;
    const int64_t ngroups = n_scales(d, rows, cols);
    parts = balanced_grid(ngroups, cap);
    const bool common = !given && d->rounding == LQ_RNE && codes && scales && y && res && d->symmetric &&
                        d->in_dtype == d->out_dtype && d->in_dtype != LQ_F16 && !d->hadamard;
    if (common && slot <= 2 && !is_six(d->format)) {
      // the tile kernel finishes the QSNR itself (its grid is at most kMaxWG)
      a.finish_inline = 1;
      a.epoch = next_epoch();
      finished = true;
      e = T.fast[d->in_dtype].tile[d->format][d->scale_fmt][slot](a, parts, s);
    } else {
      e = K.row[d->format][slot](a, parts, s);
    }
  } else {
    const bool common = !given && d->rounding == LQ_RNE && codes && scales && y && res && d->symmetric &&
                        d->in_dtype == LQ_BF16 && d->out_dtype == LQ_BF16 && !d->hadamard;
    if (common && cols % 1024 == 0 && cols <= 4096) {
      // one wave per row in the lane-contiguous layout; 4 rows per workgroup
      const int64_t wg = (rows + 3) / 4;
      const int64_t cap_row = cap < kInlineFinishMaxWG ? cap : kInlineFinishMaxWG;
      const int nwg_row = balanced_grid(wg, cap_row);
      const FastArgs fa = fast_args(a, rows, (int32_t)(cols / 1024), 0);
      e = T.lc.row[d->format][d->scale_fmt](fa, nwg_row, s);
      finished = true;
    } else {
      const int64_t tiles_per_row = (cols + 15) / 16;
      const int64_t per_lane = (tiles_per_row + kThreads - 1) / kThreads;
      const int slot = per_lane <= 1 ? 0 : per_lane <= 2 ? 1 : per_lane <= 4 ? 2 : 3;
      parts = balanced_grid(rows, cap);
      e = K.row[d->format][slot](a, parts, s);
    }
  }
  if (e != hipSuccess) return LQ_ERR_HIP;
  if (res && !finished && launch_finish((const Workspace*)ws, parts, res, s) != hipSuccess) return LQ_ERR_HIP;
  return LQ_OK;
}

// ---- the workspace of lq_fake_quant_qsnr_static: one array per device,
// in this library's code object, held until the process ends. In host code
// `scratch` names a host-side stand-in, not device memory: only the address
// hipGetSymbolAddress returns for the current device is passed to kernels.
constexpr size_t kScratchBytes = (sizeof(Workspace) + 255) & ~(size_t)255;
static_assert(kScratchBytes == LQ_STATIC_WORKSPACE_BYTES, "lq.h states the array's size");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // per device, set once under the mutex

// Device address of `scratch` on the current device (taken with that device
// current, once per device), or null on failure.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// Installs a launch-plan recorder on this thread for the lifetime of the object.
struct PlanScope {
  PlanRecorder rec;
  explicit PlanScope(char* buf, size_t bytes) {
    rec.buf = (buf && bytes) ? buf : nullptr;
    rec.cap = bytes;
    rec.len = 0;
    rec.count = 0;
    if (rec.buf) rec.buf[0] = '\0';
    g_plan = &rec;
  }
  ~PlanScope() { g_plan = nullptr; }
};

// Integer-vs-float pairs of the sweep table: (INT8, E4M3), (INT8, E5M2), (INT4, E2M1).
constexpr int kPairInt[3] = {LQ_INT8, LQ_INT8, LQ_INT4};
constexpr int kPairFp[3] = {LQ_E4M3, LQ_E5M2, LQ_E2M1};
enum : int { kIntWins = 0, kFpWins = 1, kTies = 2, kUndecided = 3 };

// Outcome of one contest. Equal QSNRs (both +inf included) tie; a NaN decides
// nothing; otherwise |difference| is compared with the tie band's edge, and a
// difference within margin_db of that edge is left undecided.
int contest_outcome(double qi, double qf, double tie_db, double margin_db) {
  if (qi != qi || qf != qf) return kUndecided;
  if (qi == qf) return kTies;   // tie_db > margin_db >= 0 (checked by the caller)
  const double diff = qi - qf;
  const double mag = diff < 0.0 ? -diff : diff;
  if (mag > tie_db + margin_db) return diff > 0.0 ? kIntWins : kFpWins;
  if (mag < tie_db - margin_db) return kTies;
  return kUndecided;
}

}  // namespace

extern "C" {

int lq_quantize(const lq_desc* desc, const void* x, int64_t rows, int64_t cols, void* codes, void* scales,
                void* zeros, void* ws, size_t ws_bytes, void* stream) {
  if (!codes && desc && rows * cols > 0) return LQ_ERR_NULL;
  return run_quant(desc, x, rows, cols, codes, scales, zeros, nullptr, 0, nullptr, ws, ws_bytes, stream);
}

int lq_fake_quant_qsnr(const lq_desc* desc, const void* x, int64_t rows, int64_t cols, void* codes,
                       void* scales, void* zeros, void* y, lq_result* res, void* ws, size_t ws_bytes,
                       void* stream) {
  if (desc && desc->hadamard != 0) return LQ_ERR_BAD_DESC;
  return run_quant(desc, x, rows, cols, codes, scales, zeros, y, 0, res, ws, ws_bytes, stream);
}

int lq_fake_quant_qsnr_static(const lq_desc* desc, const void* x, int64_t rows, int64_t cols, void* codes,
                              void* scales, void* zeros, void* y, lq_result* res, void* stream) {
  if (desc && desc->hadamard != 0) return LQ_ERR_BAD_DESC;
  int rc = check_desc(desc);
  if (rc) return rc;
  rc = check_shape(desc, rows, cols);
  if (rc) return rc;
  // every call needs at most sizeof(Workspace); the check keeps the bound explicit
  if (lq_workspace_bytes(desc, rows, cols) > kScratchBytes) return LQ_ERR_WORKSPACE;
  void* ws = scratch_for_current_device();
  if (!ws) return LQ_ERR_HIP;
  return run_quant(desc, x, rows, cols, codes, scales, zeros, y, 0, res, ws, kScratchBytes, stream);
}

int lq_hadamard_quant(const lq_desc* desc, const void* x, int64_t rows, int64_t cols, void* codes,
                      void* scales, void* zeros, void* y, int unrotate_y, lq_result* res, void* ws,
                      size_t ws_bytes, void* stream) {
  if (desc && desc->hadamard == 0) return LQ_ERR_BAD_DESC;
  return run_quant(desc, x, rows, cols, codes, scales, zeros, y, unrotate_y, res, ws, ws_bytes, stream);
}

int lq_dequantize(const lq_desc* desc, const void* codes, const void* scales, const void* zeros, int64_t rows,
                  int64_t cols, void* y, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  rc = check_shape(desc, rows, cols);
  if (rc) return rc;
  const int64_t n = rows * cols;
  if (n == 0) return LQ_OK;
  if (!codes || !scales || !y || (!desc->symmetric && !zeros)) return LQ_ERR_NULL;
  for (const void* p : {codes, scales, zeros, (const void*)y})
    if (p && !aligned(p)) return LQ_ERR_ALIGN;
  const lq_desc de = effective_desc(desc);
  const Args a = make_args(&de, nullptr, rows, cols, (void*)codes, (void*)scales, (void*)zeros, y, 1, nullptr,
                           nullptr);
  const int64_t ntiles = (n + 15) / 16;
  const int64_t wg_needed = (ntiles + kThreads - 1) / kThreads;
  const int cap = grid_cap();
  const int nwg = balanced_grid(wg_needed, cap);
  const int gran = de.gran;   // LQ_PER_TENSOR .. LQ_PER_TILE = 0 .. 3, as k_dequant numbers them
  const hipError_t e = tables().dq[desc->format](a, gran, nwg, (hipStream_t)stream);
  return e == hipSuccess ? LQ_OK : LQ_ERR_HIP;
}

size_t lq_workspace_bytes(const lq_desc* desc, int64_t rows, int64_t cols) {
  if (check_desc(desc) || check_shape(desc, rows, cols)) return 0;
  return sizeof(Workspace);
}

size_t lq_codes_bytes(const lq_desc* desc, int64_t rows, int64_t cols) {
  if (check_desc(desc) || check_shape(desc, rows, cols)) return 0;
  const int64_t n = rows * cols;
  return (size_t)(is_six(desc->format) ? n / 4 * 3 : is_four(desc->format) ? n / 2 : n);
}

size_t lq_scales_bytes(const lq_desc* desc, int64_t rows, int64_t cols) {
  if (check_desc(desc) || check_shape(desc, rows, cols)) return 0;
  if (desc->two_level) return tscale_offset(desc, rows, cols) + sizeof(float);
  return (size_t)n_scales(desc, rows, cols) * scale_size(desc->scale_fmt);
}

size_t lq_zeros_bytes(const lq_desc* desc, int64_t rows, int64_t cols) {
  if (check_desc(desc) || check_shape(desc, rows, cols)) return 0;
  if (desc->symmetric) return 0;
  return (size_t)n_scales(desc, rows, cols) * (desc->scale_fmt == LQ_SCALE_F16 ? 2 : 4);
}

int lq_set_grid_limit(int max_workgroups) {
  if (max_workgroups < 0) return LQ_ERR_SHAPE;
  g_grid_limit.store(max_workgroups, std::memory_order_relaxed);
  return LQ_OK;
}

int lq_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return LQ_ERR_NULL;
  if (!aligned(ws)) return LQ_ERR_ALIGN;
  const int64_t words = (int64_t)(ws_bytes / 4);
  if (words == 0) return LQ_OK;
  hipLaunchKernelGGL(k_fill_zero, dim3(64), dim3(256), 0, (hipStream_t)stream, (uint32_t*)ws, words);
  return hipGetLastError() == hipSuccess ? LQ_OK : LQ_ERR_HIP;
}

int lq_sweep_tally(const double* qsnr, int64_t n_tensors, double tie_db, double margin_db, int32_t* counts) {
  if (n_tensors < 0) return LQ_ERR_SHAPE;
  if (!counts || (n_tensors > 0 && !qsnr)) return LQ_ERR_NULL;
  if (!(margin_db >= 0.0) || !(tie_db > margin_db) || !(tie_db < __builtin_inf())) return LQ_ERR_BAD_DESC;
  memset(counts, 0, sizeof(int32_t) * 5 * 3 * 4);
  for (int64_t t = 0; t < n_tensors; t++) {
    const double* row = qsnr + t * 25;   // [format][granularity slot]
    for (int g = 0; g < 5; g++)
      for (int p = 0; p < 3; p++)
        counts[(g * 3 + p) * 4 + contest_outcome(row[kPairInt[p] * 5 + g], row[kPairFp[p] * 5 + g], tie_db,
                                                 margin_db)]++;
  }
  return LQ_OK;
}

int lq_call_kernels(const lq_desc* desc, int64_t rows, int64_t cols, uint32_t outputs, int unrotate_y, char* names,
                    size_t bytes) {
  if (!desc) return LQ_ERR_NULL;
  // any non-null, 16-byte aligned address stands for a buffer: nothing is
  // dereferenced or launched while the plan is recorded
  void* const buf = (void*)(uintptr_t)64;
  auto pick = [&](uint32_t bit) { return (outputs & bit) ? buf : nullptr; };
  const bool rot = desc->hadamard != 0;
  PlanScope scope(names, bytes);
  const int rc = run_quant(desc, buf, rows, cols, pick(LQ_OUT_CODES), pick(LQ_OUT_SCALES), pick(LQ_OUT_ZEROS),
                           pick(LQ_OUT_Y), rot ? unrotate_y : 0, (lq_result*)pick(LQ_OUT_QSNR), buf,
                           sizeof(Workspace), nullptr);
  return rc < 0 ? rc : scope.rec.count;
}

const char* lq_status_string(int status) {
  switch (status) {
    case LQ_OK: return "ok";
    case LQ_ERR_NULL: return "a required pointer is NULL";
    case LQ_ERR_BAD_DESC: return "invalid descriptor (unknown enum or undefined combination)";
    case LQ_ERR_SHAPE: return "invalid shape (negative size, cols % block, odd cols for 4-bit, cols % 16 with rotation)";
    case LQ_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case LQ_ERR_WORKSPACE: return "workspace missing or too small";
    case LQ_ERR_HIP: return "HIP launch failed";
    case LQ_ERR_UNSUPPORTED: return "block size not built (use 16, 32, 64, 128 or 256)";
    default: return "unknown status";
  }
}

}  // extern "C"
