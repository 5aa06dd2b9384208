/*
 * lq.h — C ABI of liblq: block-scaled quantize / dequantize ("fake-quant") with a
 * fused QSNR reduction, for AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources are web pages, cited by address and section):
 *   - Affine map, guijiagi.com/posts/quantization-int4-int8-fp8 "INT8量化":
 *       q = round(w / scale) + zero_point,   w = scale * (q - zero_point).
 *   - AbsMax quantizer, cyqw.cn/news/1000169 §2.1:
 *       s = max(abs(X)) / Qmax,   Xq = clip(round(X / s), Qmin, Qmax) * s,
 *     with the symmetric INT8 range [-127,127]; INT4 range [-8,7]
 *     (guijiagi.com "INT4量化").
 *   - Float element formats E4M3 (±448), E5M2 (±57344), E2M1 (±6) and FP6
 *     E2M3 (±7.5), E3M2 (±28), values (-1)^s * (1.m) * 2^(e-bias):
 *     walkerchi.com quantization playbook §4.1 table; cyqw.cn/news/1000169 §2.2.
 *   - Granularity: one scale per tensor, per channel (row) or per block of
 *     consecutive elements along the last dimension, cyqw.cn/news/1000169 §3.1;
 *     or per 2-D tile of tile_rows x block elements, walkerchi.com
 *     quantization playbook §4.4 (DeepSeek-V3: 1x128 activation tiles, 128x128
 *     weight tiles);
 *     MX blocks of 32 with a UE8M0 (power-of-two) scale (§2.1; playbook §4.3.1),
 *     NV-style blocks of 16 with an E4M3 scale (playbook §4.3.1).
 *   - Two-level (NVFP4-style) scaling, walkerchi.com quantization playbook
 *     §4.3.1 ("Tensor-level scale: FP32 scalar") and §4.3.2 (x = x_q * s_block *
 *     S_tensor; the tensor scale normalizes the whole tensor first).
 *   - Optional Walsh-Hadamard rotation of each aligned group of n = 16..1024
 *     columns before quantization, with QuaRot's random signs: x -> H_n D x /
 *     sqrt(n), D a ±1 diagonal (cyqw.cn/news/1000169 §4.2, §7.2; playbook §5.3:
 *     an orthogonal rotation undone by its transpose). Sylvester butterflies
 *     in binary32, then * 1/sqrt(n) rounded to binary32; the inverse takes the
 *     butterflies, the scale, then the signs.
 *   - QSNR = -10 log10(|X - Xq|^2 / |X|^2) per call (cyqw.cn/news/1000169 §4.1).
 *
 * Exact numerics (every code, scale, zero point and dequantized value is
 * bit-reproducible):
 *   scale   F32  : s = fl32(absmax / Qmax)
 *           F16  : s = fp16_rne(fl32(absmax / Qmax)), saturating at 65504
 *           E4M3 : s = e4m3_rne(fl32(absmax / Qmax)), saturating at 448
 *           UE8M0: s = 2^e, e the smallest integer with Qmax*2^e >= absmax,
 *                  clamped to [-127,127] (absmax = 0 gives e = -127)
 *           asymmetric (INT, F32/F16 only): lo = min(min x, 0), hi = max(max x, 0),
 *                  s = store(fl32(fl32(hi - lo) / (Qmax - Qmin))),
 *                  zp = clamp(Qmin - R(fl32(lo / s)), Qmin, Qmax); INT8 asymmetric
 *                  uses [-128,127]
 *           the STORED scale quantizes and dequantizes; a stored scale of 0 gives
 *           code 0 and a dequantized +0 for the whole group.
 *   two-level (two_level = 1; per-block, E4M3, symmetric): the pages give no
 *           rule for S; here S = fl32(max|x| / (448 * Qmax)) over the whole
 *           (rotated) tensor, 448 the largest E4M3 value, and an S of 0 becomes
 *           1. Every value is divided by S (fl32), the quotients are quantized
 *           with E4M3 block scales as above, and xhat = fl32(fl32(value * s) * S).
 *   element v = fl32(x / s) (correctly rounded);
 *           INT: q = clamp(R(v) [+ zp], Qmin, Qmax), R = round-half-even (LQ_RNE)
 *                or half-away-from-zero (LQ_RNA); xhat = fl32(q*s) or fl32(s*(q-zp))
 *           FP : nearest E4M3/E5M2/E2M1 value, ties to even, saturating at the
 *                format maximum, sign kept (a negative value rounding to zero gives
 *                the negative-zero code); xhat = fl32(value * s)
 *   output  y = xhat rounded to out_dtype (RNE; IEEE overflow), or xhat (F32).
 *   QSNR    err2 = sum (x - xhat)^2, sig2 = sum x^2 over fp32 x (after the
 *           rotation, if any) and fp32 xhat, accumulated in fp32 per 16 elements
 *           and in fp64 beyond; qsnr_db = -10 log10(err2 / sig2), +inf if err2 = 0.
 *
 * Layouts (all row-major, rows x cols):
 *   x, y       : elements of in_dtype / out_dtype
 *   codes      : 8-bit formats one byte per element (INT two's complement);
 *                4-bit formats two per byte, element 2j in bits [3:0] of byte j,
 *                element 2j+1 in bits [7:4]; INT4 nibbles two's complement,
 *                E2M1 nibble = s<<3 | e<<1 | m. rows*cols/2 bytes; cols must be even.
 *                FP6 (E2M3 s<<5 | e<<3 | m, E3M2 s<<5 | e<<2 | m): element e in
 *                bits 6e .. 6e+5 of the byte stream, low bits first; rows*cols*3/4
 *                bytes; cols must be a multiple of 4.
 *   scales     : PER_TENSOR 1, PER_CHANNEL rows, PER_BLOCK rows*(cols/block),
 *                PER_TILE ceil(rows/tile_rows)*(cols/block) (row-major over
 *                tiles; the last band of rows may be shorter than tile_rows)
 *                entries of 4 (F32), 2 (F16) or 1 (UE8M0 = e+127, E4M3) bytes;
 *                two-level: the fp32 S follows the block scales at the next
 *                multiple of 16 bytes
 *   zeros      : asymmetric only; same count as scales, fp32 (F32 scales) or
 *                fp16 (F16 scales), each an integer value
 *
 * Ownership and execution: the caller owns every buffer; all data pointers are
 * DEVICE pointers except where noted, and must be 16-byte aligned. Work is
 * enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 * call returns without waiting; results are valid once the stream has
 * completed. The library allocates nothing; the only state it keeps between
 * calls is a call counter (tags for workspace records) and the cap set by
 * lq_set_grid_limit.
 *
 * Workspace: calls that reduce (QSNR, or a per-tensor scale) need a device
 * workspace of at least lq_workspace_bytes() bytes for per-workgroup partial
 * results; it needs no initialisation (partial records a kernel sums within
 * itself carry the call's tag, and words of other calls are never summed).
 * Calls that overlap in time (different streams) must use different
 * workspaces.
 *
 * Errors: every argument check happens before anything is enqueued, and on
 * error nothing is written. Return values are LQ_OK or a negative LQ_ERR_*;
 * no C++ exception crosses this interface.
 */
#ifndef LQ_H
#define LQ_H

#include <stddef.h>
#include <stdint.h>

/* Every entry point below is exported from liblq.so; nothing else is (the
 * library is built with hidden visibility by default). */
#define LQ_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define LQ_OK 0
#define LQ_ERR_NULL (-1)        /* a required pointer is NULL */
#define LQ_ERR_BAD_DESC (-2)    /* unknown enum, or a combination the method does not define */
#define LQ_ERR_SHAPE (-3)       /* negative size, cols % block, odd cols for 4-bit, cols % 4 for FP6, cols % n with rotation */
#define LQ_ERR_ALIGN (-4)       /* a device pointer is not 16-byte aligned */
#define LQ_ERR_WORKSPACE (-5)   /* workspace missing or smaller than lq_workspace_bytes() */
#define LQ_ERR_HIP (-6)         /* a HIP launch failed */
#define LQ_ERR_UNSUPPORTED (-7) /* defined by the method but not built (block size) */

/* element formats */
typedef enum { LQ_INT8 = 0, LQ_INT4 = 1, LQ_E4M3 = 2, LQ_E5M2 = 3, LQ_E2M1 = 4, LQ_E2M3 = 5, LQ_E3M2 = 6 } lq_format;
/* granularity: one scale per tensor, per row, per `block` consecutive elements of a
 * row, or per 2-D tile of tile_rows rows x `block` columns */
typedef enum { LQ_PER_TENSOR = 0, LQ_PER_CHANNEL = 1, LQ_PER_BLOCK = 2, LQ_PER_TILE = 3 } lq_gran;
/* how a scale is stored */
typedef enum { LQ_SCALE_F32 = 0, LQ_SCALE_F16 = 1, LQ_SCALE_UE8M0 = 2, LQ_SCALE_E4M3 = 3 } lq_scale_fmt;
/* integer rounding */
typedef enum { LQ_RNE = 0, LQ_RNA = 1 } lq_round;
/* input / output float dtypes */
typedef enum { LQ_F32 = 0, LQ_BF16 = 1, LQ_F16 = 2 } lq_dtype;
/* where scales come from: computed from the data, or supplied by the caller (static calibration) */
typedef enum { LQ_SCALE_DYNAMIC = 0, LQ_SCALE_GIVEN = 1 } lq_scale_source;

typedef struct {
  int32_t format;       /* lq_format */
  int32_t gran;         /* lq_gran */
  int32_t block;        /* PER_BLOCK, PER_TILE: 16, 32, 64, 128 or 256 (columns); ignored otherwise */
  int32_t scale_fmt;    /* lq_scale_fmt */
  int32_t symmetric;    /* 1 = AbsMax; 0 = zero-point (INT formats with F32/F16 scales only) */
  int32_t rounding;     /* lq_round (integer formats) */
  int32_t in_dtype;     /* lq_dtype of x */
  int32_t out_dtype;    /* lq_dtype of y */
  int32_t hadamard;     /* 0, or n = 16, 32, 64, 128, 256, 512, 1024: rotate each aligned group of n
                           columns by H_n D / sqrt(n) first (D: `signs`) */
  int32_t scale_source; /* lq_scale_source */
  int32_t two_level;    /* 0, or 1 = an FP32 tensor scale above the block scales
                           (PER_BLOCK, LQ_SCALE_E4M3, symmetric only) */
  int32_t tile_rows;    /* PER_TILE: rows of a tile, 1 .. 65536; ignored otherwise */
  const void* signs;    /* with hadamard: DEVICE pointer to the random ±1 diagonal D, one bit
                           per column (bit j of the uint32 array set: column j negated),
                           at least ceil(cols/32) words; NULL = all +1. Read, not owned. */
} lq_desc;

/* Per-call result, written by the device into DEVICE memory. */
typedef struct {
  double err2;        /* sum (x - xhat)^2 */
  double sig2;        /* sum x^2 */
  double qsnr_db;     /* -10 log10(err2 / sig2); +inf when err2 == 0 */
  uint32_t nonfinite; /* count of NaN/Inf inputs (their outputs are unspecified) */
  uint32_t reserved;  /* 0; 1 when the sum could not be completed (a workgroup's
                         partial never arrived within the kernel's bounded wait):
                         err2, sig2 and qsnr_db are then NaN and nonfinite is
                         0xFFFFFFFF */
} lq_result;

/* Quantize x into codes (+ scales, zeros). With LQ_SCALE_GIVEN, scales (and
 * zeros when asymmetric; with two_level, S too) are INPUTS and are not written;
 * a given S must be positive and finite. With hadamard = n the rotated values
 * are quantized. scales/zeros may be NULL for DYNAMIC scales (not written).
 * ws: required for PER_TENSOR or two-level with DYNAMIC scales. */
LQ_API int lq_quantize(const lq_desc* desc, const void* x, int64_t rows, int64_t cols,
                void* codes, void* scales, void* zeros, void* ws, size_t ws_bytes,
                void* stream);

/* Dequantize codes with stored scales/zeros into y (out_dtype):
 * y = dec(code) * s, or s * (q - zp); two-level: (dec(code) * s) * S, S read
 * from the scales buffer. With hadamard = n the rotation is undone
 * (y = D H_n xhat / sqrt(n) per aligned n-group), giving y in the original domain.
 * desc->in_dtype and scale_source are ignored. */
LQ_API int lq_dequantize(const lq_desc* desc, const void* codes, const void* scales, const void* zeros,
                  int64_t rows, int64_t cols, void* y, void* stream);

/* Fake-quant plus QSNR in one pass over x: writes codes, scales, zeros, y
 * (each may be NULL to skip it) and *res (device pointer; may be NULL to skip
 * the reduction). desc->hadamard must be 0 (see lq_hadamard_quant). */
LQ_API int lq_fake_quant_qsnr(const lq_desc* desc, const void* x, int64_t rows, int64_t cols,
                       void* codes, void* scales, void* zeros, void* y, lq_result* res,
                       void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * lq_fake_quant_qsnr with the workspace taken from a device array inside the
 * library instead of the caller, LQ_STATIC_WORKSPACE_BYTES per device, held
 * from the first such call on a device until the process ends. It allocates
 * nothing and takes no workspace argument; arguments, outputs and errors are
 * those of lq_fake_quant_qsnr, plus LQ_ERR_WORKSPACE if a call would need
 * more than the array holds (none does: every call needs
 * lq_workspace_bytes() <= LQ_STATIC_WORKSPACE_BYTES) and LQ_ERR_HIP if the
 * array's device address cannot be obtained. Every call on one device shares
 * that device's array, which keeps the last call's contents; nothing in it
 * needs clearing (records carry the tag of the call that wrote them), but
 * calls that overlap in time on one device (other streams or host threads)
 * race on it: serialize them, or use lq_fake_quant_qsnr with separate
 * workspaces. */
#define LQ_STATIC_WORKSPACE_BYTES ((size_t)1483264)
LQ_API int lq_fake_quant_qsnr_static(const lq_desc* desc, const void* x, int64_t rows, int64_t cols,
                                     void* codes, void* scales, void* zeros, void* y, lq_result* res,
                                     void* stream);

/* As lq_fake_quant_qsnr with the rotation first (desc->hadamard = n of 16, 32,
 * 64, 128, 256, 512 or 1024; cols % n == 0; PER_TILE needs block % n == 0 when n > 16,
 * else LQ_ERR_UNSUPPORTED). Codes, scales and QSNR are in the rotated domain (the
 * rotation is orthonormal, so the QSNR equals the original-domain one up to
 * rounding); y is written in the rotated domain, or in the original domain when
 * unrotate_y != 0. */
LQ_API int lq_hadamard_quant(const lq_desc* desc, const void* x, int64_t rows, int64_t cols,
                      void* codes, void* scales, void* zeros, void* y, int unrotate_y,
                      lq_result* res, void* ws, size_t ws_bytes, void* stream);

/* Sizes in bytes of the buffers for a descriptor and shape (0 on a bad descriptor). */
LQ_API size_t lq_workspace_bytes(const lq_desc* desc, int64_t rows, int64_t cols);
LQ_API size_t lq_codes_bytes(const lq_desc* desc, int64_t rows, int64_t cols);
LQ_API size_t lq_scales_bytes(const lq_desc* desc, int64_t rows, int64_t cols);
LQ_API size_t lq_zeros_bytes(const lq_desc* desc, int64_t rows, int64_t cols);

/* Zero-fill a 16-byte aligned device buffer (for example a workspace) on
 * `stream` with a fill kernel (no memset node); ws_bytes is rounded down to 4. */
LQ_API int lq_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Caps the grid of every later launch in this process at max_workgroups
 * 256-thread workgroups (the per-block kernels with 1024-thread workgroups
 * take a quarter of that, at least one); 0 restores the default (32 per CU).
 * Results do not depend on it: a tuning and testing knob that trades
 * parallelism for more tiles per thread. Returns LQ_OK, or LQ_ERR_SHAPE for a
 * negative value. Not synchronised with launches already queued. */
LQ_API int lq_set_grid_limit(int max_workgroups);

/* Win counts for a sweep of tensors (host memory in and out; no device work),
 * the tensor-level analogue of the model win counts of cyqw.cn/news/1000169
 * §5.1. qsnr[t * 25 + f * 5 + g] holds tensor t's QSNR for format f (LQ_INT8,
 * LQ_INT4, LQ_E4M3, LQ_E5M2, LQ_E2M1) at granularity slot g (0 per-tensor,
 * 1 per-channel, 2/3/4 blocks of 16/32/64). For each slot g and each
 * integer-vs-float pair p (0: INT8 vs E4M3, 1: INT8 vs E5M2, 2: INT4 vs E2M1),
 * with d = QSNR_int - QSNR_fp (d = 0 for equal values, +inf and +inf included):
 *   |d| < tie_db - margin_db  -> a tie
 *   |d| > tie_db + margin_db  -> a win for the larger QSNR
 *   otherwise, or a NaN QSNR  -> undecided
 * and writes counts[(g * 3 + p) * 4 + {0,1,2,3}] = {INT wins, FP wins, ties,
 * undecided}. margin_db is the uncertainty of a difference: with QSNRs each
 * known to within t dB, 2t keeps every decided pair's outcome unchanged
 * however the two move. Returns LQ_OK, LQ_ERR_NULL, LQ_ERR_SHAPE
 * (n_tensors < 0) or LQ_ERR_BAD_DESC (unless 0 <= margin_db < tie_db < inf). */
LQ_API int lq_sweep_tally(const double* qsnr, int64_t n_tensors, double tie_db, double margin_db,
                          int32_t* counts);

/* Outputs a call writes, for lq_call_kernels. */
#define LQ_OUT_CODES 1u
#define LQ_OUT_SCALES 2u
#define LQ_OUT_ZEROS 4u
#define LQ_OUT_Y 8u
#define LQ_OUT_QSNR 16u

/* The kernels one call of lq_quantize / lq_fake_quant_qsnr / lq_hadamard_quant
 * with this descriptor, shape, set of non-NULL outputs (LQ_OUT_* bits) and
 * unrotate_y would launch on the current device (a host without a device
 * plans for MI355X's 256 compute units), from the library's own dispatch,
 * without launching anything or touching device memory. Writes one line per
 * kernel, in launch order, to `names` (host memory; NUL-terminated; lines
 * that do not fit in `bytes` are left out): the kernel's name as the HIP
 * runtime demangles it (the name profilers such as rocprofv3 report), a tab,
 * its number of workgroups, a tab, and its threads per workgroup. `names` may be NULL to count only. Returns
 * the number of kernels, or the negative LQ_ERR_* the call would return
 * (argument checks as in the call; pointer alignment aside). For tools that
 * match profiler records to calls. */
LQ_API int lq_call_kernels(const lq_desc* desc, int64_t rows, int64_t cols, uint32_t outputs, int unrotate_y,
                           char* names, size_t bytes);

/* Text for a status code (static storage). */
LQ_API const char* lq_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* LQ_H */
