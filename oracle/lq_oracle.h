/*
 * lq_oracle.h — plain, slow CPU model of block-scaled fake-quant + QSNR.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, includes or
 * calls this code; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load it. It shares no source with the HIP path: its enums,
 * format tables and rounding rules are written here from the definitions on
 * the source pages, independently.
 *
 * Sources (web pages; cited by address and section):
 *   guijiagi.com/posts/quantization-int4-int8-fp8  "INT8量化", "INT4量化" (affine
 *       map q = round(w/scale)+zero_point, dequant scale*(q-zero_point); INT4 range
 *       [-8,7]; group-wise INT4 example), "FP8量化" table (E4M3 ±448, E5M2 ±57344).
 *   cyqw.cn/news/1000169  §2.1 (AbsMax: s = max|X|/Qmax, Xq = clip(round(X/s),
 *       Qmin,Qmax)*s; MXINT8 blocks of 32 with a UE8M0 scale; symmetric [-127,127]),
 *       §2.2 (FP value (-1)^s*(1.m)*2^(e-bias)), §3.1 (per-tensor/per-channel/block),
 *       §4.1 (QSNR = -10 log10(|X-Xq|^2/|X|^2)), §4.2/§7.2 (Hadamard before NVINT4).
 *   walkerchi.com quantization playbook ("量化全景"), §4.4 (DeepSeek-V3: per-tile
 *       scaling, 1x128 tiles for activations and 128x128 for weights, E4M3),
 *       §4.1 FP-type table (bit
 *       layouts, ranges, smallest positive values), §4.3.1 (MXFP4: 32 values + E8M0
 *       scale; NVFP4: 16 values + E4M3 scale + an FP32 tensor-level scale), §4.3.2
 *       (two-level scaling: x = x_q * s_block * S_tensor; the tensor scale
 *       normalizes the whole tensor first), §5.3 (Hadamard: orthogonal ±1).
 *
 * Numerics: every decision that yields a code is taken in IEEE binary32 with
 * round-to-nearest-even (no FMA contraction, no flush-to-zero), because that is
 * the precision the pages' own example computes in (float tensors); format
 * rounding is done exactly in binary64 on each format's value grid; the QSNR sums
 * are binary64.
 */
#ifndef LQ_ORACLE_H
#define LQ_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element formats */
enum { OR_INT8 = 0, OR_INT4 = 1, OR_E4M3 = 2, OR_E5M2 = 3, OR_E2M1 = 4, OR_E2M3 = 5, OR_E3M2 = 6 };
/* number kinds usable with or_fp_* (element, scale and storage float formats) */
enum { ORK_E4M3 = 0, ORK_E5M2 = 1, ORK_E2M1 = 2, ORK_FP16 = 3, ORK_BF16 = 4, ORK_E2M3 = 5, ORK_E3M2 = 6 };
/* granularity: one scale per tensor, per row, per block of a row, or per
   2-D tile of tile_rows x block elements (DeepSeek-V3 style) */
enum { OR_TENSOR = 0, OR_CHANNEL = 1, OR_BLOCK = 2, OR_TILE = 3 };
/* scale storage */
enum { OR_S_F32 = 0, OR_S_F16 = 1, OR_S_UE8M0 = 2, OR_S_E4M3 = 3 };
/* integer rounding */
enum { OR_RNE = 0, OR_RNA = 1 };
/* input / output float dtypes */
enum { OR_F32 = 0, OR_BF16 = 1, OR_F16 = 2 };

typedef struct {
  int32_t fmt;          /* OR_INT8 .. OR_E3M2 */
  int32_t gran;         /* OR_TENSOR / OR_CHANNEL (one scale per row) / OR_BLOCK */
  int32_t block;        /* elements per block along the last dim (OR_BLOCK) */
  int32_t scale_fmt;    /* OR_S_* */
  int32_t symmetric;    /* 1 = AbsMax symmetric; 0 = min/max with zero-point (INT only) */
  int32_t rounding;     /* OR_RNE / OR_RNA (integer formats) */
  int32_t out_dtype;    /* OR_F32 / OR_BF16 / OR_F16 for the dequantized output */
  int32_t hadamard;     /* 0, or n = 16, 32, ..., 1024: rotate each aligned n-group by
                           H_n D / sqrt(n) first */
  int32_t unrotate_y;   /* with hadamard: write y in the original (un-rotated) domain */
  int32_t given_scales; /* 1 = read scales (and zeros) from the buffers instead of computing */
  int32_t two_level;    /* 1 = NVFP4-style FP32 tensor scale S above E4M3 block scales */
  int32_t tile_rows;    /* OR_TILE: rows of a tile (its columns: block) */
  const uint32_t* signs; /* with hadamard: the random ±1 diagonal D, bit j of the array
                            set = column j negated; NULL = all +1 */
} or_desc;

/* ---- number formats ---------------------------------------------------- */
/* Value of a code of kind k (may be +-inf or NaN for IEEE-style kinds). */
double   or_fp_decode(int kind, uint32_t code);
/* Nearest code to v (ties to even significand); saturate=1 clamps to +-max,
   saturate=0 overflows to the infinity code (IEEE kinds only). Sign kept. */
uint32_t or_fp_encode(int kind, double v, int saturate);
/* Largest finite value of a kind. */
double   or_fp_max(int kind);
/* Power-of-two scale exponent: smallest e with qmax*2^e >= absmax, in [-127,127]. */
int      or_ue8m0_exponent(double absmax, double qmax);
/* Integer rounding of a finite value: OR_RNE or OR_RNA. */
double   or_round_int(double v, int mode);
/* One 16-point Sylvester Walsh-Hadamard butterfly in binary32 followed by *0.25. */
void     or_hadamard16(float* v);
/* n-point rotation of v (n a power of two) whose first element is column col0:
   columns with their sign bit set negated, Sylvester butterflies in binary32,
   then * or_rotation_scale(n); or_unrotate: butterflies, scale, then signs. */
void     or_rotate(float* v, int n, const uint32_t* signs, int64_t col0);
void     or_unrotate(float* v, int n, const uint32_t* signs, int64_t col0);
/* 1/sqrt(n) rounded to binary32. */
float    or_rotation_scale(int n);

/* ---- the method -------------------------------------------------------- */
/* Statistics of the whole (rotated, if hadamard) tensor: out[0]=max|x|,
   out[1]=min(x), out[2]=max(x); returns the count of non-finite inputs. */
int64_t  or_tensor_stat(const or_desc* d, const float* x, int64_t rows, int64_t cols,
                        float out[3]);

/* Two-level tensor scale (playbook §4.3.1/§4.3.2; the pages give no rule for
 * it): S = amax / (448 * Qmax) in binary32, 448 the largest E4M3 value, so the
 * block holding the tensor's largest magnitude gets the largest block scale;
 * an S of zero (all-zero tensor, or an underflowing quotient) is replaced by 1. */
float    or_tensor_scale(const or_desc* d, float amax);

/* Fake-quantize rows [0, nrows) of a row block x (nrows x cols, fp32 values).
 * tstat: or_tensor_stat() of the WHOLE tensor (used for OR_TENSOR and two_level).
 * tscale: two_level only: the tensor scale S, read when given_scales, else
 *         written (may be NULL). With two_level each value is first divided by
 *         S, the quotients are block-quantized with E4M3 scales as usual, and
 *         xhat = (value * s_block) * S. Ignored otherwise.
 * Outputs (any may be NULL; all laid out for these nrows only):
 *   codes : 8-bit formats one byte per element; 4-bit formats two per byte,
 *           element 2j in bits [3:0] of byte j, 2j+1 in bits [7:4]; 6-bit (FP6)
 *           element e in bits 6e .. 6e+5 of the byte stream, low bits first
 *   scales: per-tensor 1, per-channel nrows, per-block nrows*cols/block entries,
 *           per-tile ceil(nrows/tile_rows)*(cols/block) entries in row-major
 *           tile order, each 4 (F32), 2 (F16) or 1 (UE8M0, E4M3) bytes. With
 *           OR_TILE the row block must start at a multiple of tile_rows (its
 *           tiles are whole, except the tensor's last band of rows)
 *   zeros : asymmetric only, same count as scales, 4 (F32) or 2 (F16) bytes
 *   xhat  : fp32 dequantized values (rotated domain when hadamard)
 *   y     : dequantized values in out_dtype (4 or 2 bytes), un-rotated if asked
 * err2/sig2 accumulate (+=) sum (x-xhat)^2 and sum x^2 in binary64.
 * Returns 0, or a negative value for an unsupported descriptor or a host FPU
 * mode (flush-to-zero / denormals-are-zero / non-nearest rounding) that would
 * change binary32 results. */
int or_fake_quant_rows(const or_desc* d, const float* x, int64_t nrows, int64_t cols,
                       const float tstat[3], float* tscale, uint8_t* codes, void* scales,
                       void* zeros, float* xhat, void* y, double* err2, double* sig2);

/* ---- sweep post-processing --------------------------------------------- */
/* INT-vs-FP win counts over a sweep of tensors: the tensor-level analogue of
 * the per-model win counts of cyqw.cn/news/1000169 §5.1 (the page gives no
 * tie rule; the reading here is stated with the function).
 * qsnr[t*25 + f*5 + g]: tensor t, format f in (INT8, INT4, E4M3, E5M2, E2M1),
 * granularity slot g in (per tensor, per channel, blocks of 16, 32, 64).
 * Pairs p: (INT8, E4M3), (INT8, E5M2), (INT4, E2M1). For each slot and pair,
 * with d = QSNR_int - QSNR_fp (equal values, infinities included, give d = 0):
 *   |d| < tie_db - margin_db        -> tie
 *   |d| > tie_db + margin_db        -> a win for the larger QSNR
 *   otherwise, or a NaN QSNR        -> undecided (the classification could
 *                                      change if either QSNR moved by
 *                                      margin_db / 2)
 * counts[(g*3 + p)*4 + k], k = 0 INT wins, 1 FP wins, 2 ties, 3 undecided.
 * Returns 0, or -1 for n_tensors < 0, a NULL pointer or not
 * (0 <= margin_db < tie_db). */
int or_sweep_tally(const double* qsnr, int64_t n_tensors, double tie_db, double margin_db, int32_t* counts);

/* Dequantize codes with stored scales/zeros (same layouts as above) into y;
 * tscale: the tensor scale S with two_level (ignored otherwise). */
int or_dequant_rows(const or_desc* d, const uint8_t* codes, const void* scales,
                    const void* zeros, float tscale, int64_t nrows, int64_t cols, void* y);

#ifdef __cplusplus
}
#endif
#endif
