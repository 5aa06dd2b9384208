/*
 * lq_oracle.c — plain, slow CPU model of block-scaled fake-quant + QSNR.
 *
 * TEST INFRASTRUCTURE ONLY (see lq_oracle.h): loaded by the test suite, the smoke
 * check and the benchmark's CPU-baseline leg, never by the product library.
 *
 * Every step below is written from its definition, one element at a time:
 *   - a float format is a set of values (its grid); encoding picks the nearest
 *     grid value, ties to the even significand, saturating at the largest finite
 *     value (or overflowing to infinity for the IEEE output dtypes);
 *   - a scale is max|x| / Qmax (AbsMax), stored in its own format, and the STORED
 *     scale is what quantizes and dequantizes;
 *   - the element is x / s in binary32, rounded into the element format;
 *   - dequantization is code value * s (or s * (q - zp)) in binary32;
 *   - QSNR sums are binary64.
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared.
 */
#include "lq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>

/* ------------------------------------------------------------------------ */
/* Float formats as value grids.                                             */
/*                                                                           */
/* walkerchi.com quantization playbook, §4.1 FP-type table: E2M1 = 1 sign, 2  */
/* exponent, 1 mantissa bits, range ±6, smallest positive 0.5; E4M3 = 1/4/3,  */
/* ±448, smallest ~0.00195 (=2^-9); E5M2 = 1/5/2, ±57344, smallest ~1.5e-5    */
/* (=2^-16); FP16 1/5/10 ±65504; BF16 1/8/7. cyqw.cn/news/1000169 §2.2 gives  */
/* the value of a field triple: (-1)^s * (1.m) * 2^(e-bias). The same table   */
/* gives FP6 E2M3 = 1/2/3 bits, ±7.5, and E3M2 = 1/3/2 bits, ±28 (MXFP6).     */
/* Those maxima and minima fix the biases (E4M3 7, E5M2 15, E2M1 1) and the   */
/* specials: E4M3 reaching 448 = 1.75*2^8 uses the all-ones exponent for       */
/* numbers, leaving only s.1111.111 as NaN (no infinity); E5M2's 57344 =       */
/* 1.75*2^15 leaves the all-ones exponent to inf/NaN as in IEEE; E2M1's 6 =    */
/* 1.5*2^2 uses every code for a number. 7.5 = 1.875*2^2 and 28 = 1.75*2^4    */
/* fix the FP6 biases (E2M3 1, E3M2 3) with every code a number as well; the  */
/* table's smallest-positive entries for FP6 fit neither (garbled), so the    */
/* maxima and bit layouts are what pin them.                                  */
/* ------------------------------------------------------------------------ */
typedef struct {
  int ebits, mbits, bias;
  int ieee_specials;   /* top exponent field reserved for inf/NaN */
  int nan_all_ones;    /* only the all-ones magnitude code is NaN (E4M3) */
} fpfmt;

static const fpfmt FMT[7] = {
  /* ORK_E4M3 */ {4, 3, 7, 0, 1},
  /* ORK_E5M2 */ {5, 2, 15, 1, 0},
  /* ORK_E2M1 */ {2, 1, 1, 0, 0},
  /* ORK_FP16 */ {5, 10, 15, 1, 0},
  /* ORK_BF16 */ {8, 7, 127, 1, 0},
  /* ORK_E2M3 */ {2, 3, 1, 0, 0},
  /* ORK_E3M2 */ {3, 2, 3, 0, 0},
};

static int valid_kind(int k) { return k >= 0 && k <= ORK_E3M2; }

double or_fp_decode(int kind, uint32_t code) {
  if (!valid_kind(kind)) return NAN;
  const fpfmt* f = &FMT[kind];
  const uint32_t emask = (1u << f->ebits) - 1u, mmask = (1u << f->mbits) - 1u;
  const uint32_t s = (code >> (f->ebits + f->mbits)) & 1u;
  const uint32_t e = (code >> f->mbits) & emask;
  const uint32_t m = code & mmask;
  double v;
  if (f->ieee_specials && e == emask) {
    v = (m == 0) ? INFINITY : NAN;
  } else if (f->nan_all_ones && e == emask && m == mmask) {
    v = NAN;
  } else if (e == 0) {
    /* subnormal: 0.m * 2^(1-bias) */
    v = ldexp((double)m, 1 - f->bias - f->mbits);
  } else {
    /* normal: 1.m * 2^(e-bias) */
    v = ldexp((double)((1u << f->mbits) | m), (int)e - f->bias - f->mbits);
  }
  return s ? -v : v;
}

double or_fp_max(int kind) {
  if (!valid_kind(kind)) return NAN;
  const fpfmt* f = &FMT[kind];
  int emax_field = (1 << f->ebits) - 1 - (f->ieee_specials ? 1 : 0);
  int mmax = (1 << f->mbits) - 1 - (f->nan_all_ones ? 1 : 0);
  return ldexp((double)((1 << f->mbits) | mmax), emax_field - f->bias - f->mbits);
}

/* Spacing of the grid around magnitude a (a >= 0): 2^(k-M) in binade
   [2^k, 2^(k+1)), and the first normal binade's spacing below it (gradual
   underflow). */
static double grid_ulp(const fpfmt* f, double a) {
  int kmin = 1 - f->bias;
  int k = kmin;
  if (a >= ldexp(1.0, kmin)) {
    int x;
    frexp(a, &x); /* a = frac * 2^x, frac in [0.5, 1) */
    k = x - 1;
  }
  return ldexp(1.0, k - f->mbits);
}

/* Round a finite magnitude a >= 0 to the nearest grid value, ties to the
   value with an even significand (even code). The result may lie above the
   largest finite value; the caller saturates or overflows. All operations are
   exact in binary64 for inputs that are binary32 values. */
static double grid_round(const fpfmt* f, double a) {
  double ulp = grid_ulp(f, a);
  double n = floor(a / ulp);
  double lo = n * ulp, hi = (n + 1.0) * ulp;
  double twice = 2.0 * a, mid2 = lo + hi;
  if (twice < mid2) return lo;
  if (twice > mid2) return hi;
  return (fmod(n, 2.0) == 0.0) ? lo : hi;
}

/* Field encoding of a non-negative grid value that is <= max. */
static uint32_t grid_code(const fpfmt* f, double v) {
  int kmin = 1 - f->bias;
  if (v < ldexp(1.0, kmin)) {
    return (uint32_t)(v / ldexp(1.0, kmin - f->mbits)); /* e field 0 */
  }
  int x;
  frexp(v, &x);
  int k = x - 1;
  uint32_t m = (uint32_t)(v / ldexp(1.0, k - f->mbits)) - (1u << f->mbits);
  uint32_t e = (uint32_t)(k + f->bias);
  return (e << f->mbits) | m;
}

uint32_t or_fp_encode(int kind, double v, int saturate) {
  if (!valid_kind(kind)) return 0;
  const fpfmt* f = &FMT[kind];
  const uint32_t sign = signbit(v) ? (1u << (f->ebits + f->mbits)) : 0u;
  const double maxv = or_fp_max(kind);
  if (isnan(v)) {
    /* NaN lies outside every grid: the kind's NaN code where it has one (all
       ones, or a quiet NaN for the IEEE kinds), else the largest magnitude */
    const uint32_t all = (1u << (f->ebits + f->mbits)) - 1u;
    if (f->nan_all_ones) return sign | all;
    if (f->ieee_specials) return sign | (((1u << f->ebits) - 1u) << f->mbits) | (1u << (f->mbits - 1));
    return sign | grid_code(f, maxv);
  }
  double a = fabs(v);
  double r;
  if (a >= maxv) {
    r = maxv;
    if (!saturate && f->ieee_specials && grid_round(f, a) > maxv) {
      return sign | (((1u << f->ebits) - 1u) << f->mbits); /* infinity */
    }
  } else {
    r = grid_round(f, a);
    if (r > maxv) {
      if (!saturate && f->ieee_specials)
        return sign | (((1u << f->ebits) - 1u) << f->mbits);
      r = maxv;
    }
  }
  return sign | grid_code(f, r);
}

/* ------------------------------------------------------------------------ */
/* Power-of-two (UE8M0) scale.                                               */
/* cyqw.cn/news/1000169 §2.1: each 32-element MXINT8 block shares one UE8M0   */
/* scale; walkerchi.com playbook §4.3.1: the MX block scale is E8M0, a power  */
/* of two with an integer exponent. AbsMax wants s >= max|x|/Qmax so nothing  */
/* clips; the power-of-two scale closest to that from above is 2^e with the   */
/* smallest integer e such that Qmax*2^e >= max|x|. E8M0 covers 2^-127..2^127 */
/* (code 255 is not a number), so e is clamped to that range; an all-zero     */
/* block takes the smallest scale.                                           */
/* ------------------------------------------------------------------------ */
int or_ue8m0_exponent(double absmax, double qmax) {
  if (!(absmax > 0.0)) return -127;
  int e;
  frexp(absmax / qmax, &e); /* estimate, then settle by exact comparisons */
  while (e > -200 && ldexp(qmax, e - 1) >= absmax) e--;
  while (ldexp(qmax, e) < absmax) e++;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

/* ------------------------------------------------------------------------ */
/* Integer rounding. guijiagi.com "INT4量化" example rounds with torch.round,  */
/* which rounds half to even; half-away-from-zero is offered as the other     */
/* mode.                                                                     */
/* ------------------------------------------------------------------------ */
double or_round_int(double v, int mode) {
  double f = floor(v);
  double d = v - f; /* exact: v is a binary32 value */
  if (d > 0.5) return f + 1.0;
  if (d < 0.5) return f;
  if (mode == OR_RNA) return (v > 0.0) ? f + 1.0 : f;
  return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* ------------------------------------------------------------------------ */
/* n-point Walsh-Hadamard rotation (walkerchi.com playbook §5.3: an orthogonal */
/* ±1 matrix, R^T R = I, QuaRot's randomized Hadamard; cyqw.cn/news/1000169    */
/* §4.2, §7.2: rotate before NVINT4). Sylvester ordering,                      */
/* H[i][j] = (-1)^popcount(i&j), applied as butterfly stages of                */
/* (a,b) -> (a+b, a-b) at strides 1, 2, 4, ..., n/2 in binary32, then          */
/* multiplied by 1/sqrt(n) rounded to binary32 (exact for n = 16, 64, 256) so  */
/* the map is orthonormal up to that rounding. QuaRot's random signs: a ±1     */
/* diagonal D per column, applied before the butterflies (x -> H D x / sqrt(n))*/
/* and after them on the way back (D H y / sqrt(n), H being symmetric).        */
/* ------------------------------------------------------------------------ */
float or_rotation_scale(int n) { return (float)(1.0 / sqrt((double)n)); }

static int sign_bit(const uint32_t* signs, int64_t col) {
  return signs ? (int)((signs[col >> 5] >> (col & 31)) & 1u) : 0;
}

static void butterflies(float* v, int n) {
  for (int h = 1; h < n; h <<= 1) {
    for (int i = 0; i < n; i++) {
      if ((i & h) == 0) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

void or_rotate(float* v, int n, const uint32_t* signs, int64_t col0) {
  for (int i = 0; i < n; i++)
    if (sign_bit(signs, col0 + i)) v[i] = -v[i];
  butterflies(v, n);
  const float c = or_rotation_scale(n);
  for (int i = 0; i < n; i++) v[i] = v[i] * c;
}

void or_unrotate(float* v, int n, const uint32_t* signs, int64_t col0) {
  butterflies(v, n);
  const float c = or_rotation_scale(n);
  for (int i = 0; i < n; i++) v[i] = v[i] * c;
  for (int i = 0; i < n; i++)
    if (sign_bit(signs, col0 + i)) v[i] = -v[i];
}

void or_hadamard16(float* v) { or_rotate(v, 16, NULL, 0); }

/* ------------------------------------------------------------------------ */
/* The quantizer.                                                            */
/* ------------------------------------------------------------------------ */
static int is_int_fmt(int fmt) { return fmt == OR_INT8 || fmt == OR_INT4; }
static int is_4bit(int fmt) { return fmt == OR_INT4 || fmt == OR_E2M1; }
static int is_6bit(int fmt) { return fmt == OR_E2M3 || fmt == OR_E3M2; }
static int elem_kind(int fmt) {
  return fmt == OR_E4M3   ? ORK_E4M3
         : fmt == OR_E5M2 ? ORK_E5M2
         : fmt == OR_E2M3 ? ORK_E2M3
         : fmt == OR_E3M2 ? ORK_E3M2
                          : ORK_E2M1;
}

/* Code range. Symmetric INT8 uses [-127,127] (cyqw.cn/news/1000169 §2.1);
   INT4 uses [-8,7] (guijiagi.com "INT4量化", clamp(-8, 7)); the asymmetric
   (zero-point) map uses the full two's-complement range [-128,127] of INT8
   (guijiagi.com "INT8量化"). Qmax of a float format is its largest finite
   value. */
static void int_range(const or_desc* d, double* qmin, double* qmax) {
  if (d->fmt == OR_INT8) {
    *qmax = 127.0;
    *qmin = d->symmetric ? -127.0 : -128.0;
  } else {
    *qmax = 7.0;
    *qmin = -8.0;
  }
}
static double elem_qmax(const or_desc* d) {
  if (d->fmt == OR_INT8) return 127.0;
  if (d->fmt == OR_INT4) return 7.0;
  return or_fp_max(elem_kind(d->fmt));
}

typedef struct {
  float s;        /* stored scale, as a binary32 value */
  float zp;       /* zero point (asymmetric), an integer */
  uint32_t sbits; /* stored bits of s */
  uint32_t zbits; /* stored bits of zp */
} scale_t;

static float f32_from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

/* Store a non-negative binary32 scale candidate t in the scale format.
   fp16 and E4M3 round to nearest-even and saturate at their maximum. */
static void store_scale(int scale_fmt, float t, scale_t* sc) {
  if (scale_fmt == OR_S_F16) {
    sc->sbits = or_fp_encode(ORK_FP16, (double)t, 1);
    sc->s = (float)or_fp_decode(ORK_FP16, sc->sbits);
  } else if (scale_fmt == OR_S_E4M3) {
    sc->sbits = or_fp_encode(ORK_E4M3, (double)t, 1);
    sc->s = (float)or_fp_decode(ORK_E4M3, sc->sbits);
  } else {
    sc->s = t;
    sc->sbits = bits_from_f32(t);
  }
}

/* Symmetric (AbsMax) scale of a group with maximum magnitude amax:
   s = max|x| / Qmax (cyqw.cn/news/1000169 §2.1), computed as a binary32
   quotient, then stored; UE8M0 takes the power of two described above. */
static scale_t scale_sym(const or_desc* d, float amax) {
  scale_t sc = {0.0f, 0.0f, 0u, 0u};
  double qmax = elem_qmax(d);
  if (d->scale_fmt == OR_S_UE8M0) {
    int e = or_ue8m0_exponent((double)amax, qmax);
    sc.sbits = (uint32_t)(e + 127);
    sc.s = (float)ldexp(1.0, e); /* exact, 2^-127 is a binary32 subnormal */
    return sc;
  }
  float t = amax / (float)qmax;
  store_scale(d->scale_fmt, t, &sc);
  return sc;
}

/* Asymmetric (zero-point) scale. The affine map of guijiagi.com "INT8量化"
   (q = round(w/scale) + zero_point; w = scale*(q - zero_point)) gives no rule
   for scale and zero point; the plainest one spreads [min(mn,0), max(mx,0)]
   over the code range: s = (mx-mn)/(Qmax-Qmin), zp = Qmin - round(mn/s),
   clamped into the code range, both stored in the scale format. Extending the
   range to include 0 keeps an exact zero representable. */
static scale_t scale_asym(const or_desc* d, float mn, float mx) {
  scale_t sc = {0.0f, 0.0f, 0u, 0u};
  double qmin, qmax;
  int_range(d, &qmin, &qmax);
  float lo = mn < 0.0f ? mn : 0.0f;
  float hi = mx > 0.0f ? mx : 0.0f;
  float t = (hi - lo) / (float)(qmax - qmin);
  store_scale(d->scale_fmt, t, &sc);
  if (sc.s == 0.0f) {
    sc.zp = 0.0f;
  } else {
    float m = lo / sc.s;
    double z = qmin - or_round_int((double)m, d->rounding);
    if (z < qmin) z = qmin;
    if (z > qmax) z = qmax;
    sc.zp = (float)z;
  }
  if (d->scale_fmt == OR_S_F16) sc.zbits = or_fp_encode(ORK_FP16, (double)sc.zp, 1);
  else sc.zbits = bits_from_f32(sc.zp + 0.0f);
  return sc;
}

/* Read a caller-supplied (calibrated) scale and zero point. */
static scale_t scale_given(const or_desc* d, const void* scales, const void* zeros, int64_t idx) {
  scale_t sc = {0.0f, 0.0f, 0u, 0u};
  switch (d->scale_fmt) {
    case OR_S_F32: sc.sbits = ((const uint32_t*)scales)[idx]; sc.s = f32_from_bits(sc.sbits); break;
    case OR_S_F16: sc.sbits = ((const uint16_t*)scales)[idx]; sc.s = (float)or_fp_decode(ORK_FP16, sc.sbits); break;
    case OR_S_UE8M0: sc.sbits = ((const uint8_t*)scales)[idx]; sc.s = (float)ldexp(1.0, (int)sc.sbits - 127); break;
    default: sc.sbits = ((const uint8_t*)scales)[idx]; sc.s = (float)or_fp_decode(ORK_E4M3, sc.sbits); break;
  }
  if (!d->symmetric) {
    if (d->scale_fmt == OR_S_F16) {
      sc.zbits = ((const uint16_t*)zeros)[idx];
      sc.zp = (float)or_fp_decode(ORK_FP16, sc.zbits);
    } else {
      sc.zbits = ((const uint32_t*)zeros)[idx];
      sc.zp = f32_from_bits(sc.zbits);
    }
  }
  return sc;
}

static void put_scale(const or_desc* d, void* scales, void* zeros, int64_t idx, const scale_t* sc) {
  if (scales) {
    switch (d->scale_fmt) {
      case OR_S_F32: ((uint32_t*)scales)[idx] = sc->sbits; break;
      case OR_S_F16: ((uint16_t*)scales)[idx] = (uint16_t)sc->sbits; break;
      default: ((uint8_t*)scales)[idx] = (uint8_t)sc->sbits; break;
    }
  }
  if (zeros && !d->symmetric) {
    if (d->scale_fmt == OR_S_F16) ((uint16_t*)zeros)[idx] = (uint16_t)sc->zbits;
    else ((uint32_t*)zeros)[idx] = sc->zbits;
  }
}

/* One element: v = x / s in binary32 with the stored s, then
   INT:  q = clamp(round(v), Qmin, Qmax)               (AbsMax, cyqw §2.1)
         q = clamp(round(v) + zp, Qmin, Qmax)          (affine, guijiagi "INT8量化")
         xhat = q * s  or  s * (q - zp)
   FP:   code = nearest E4M3/E5M2/E2M1 value (saturating), xhat = value * s.
   A zero stored scale (all-zero group, or a scale that underflows its format)
   gives code 0 and xhat = +0. */
static void quant_elem(const or_desc* d, float x, const scale_t* sc, uint32_t* code, float* xhat) {
  if (sc->s == 0.0f) {
    *code = 0u;
    *xhat = 0.0f;
    return;
  }
  float v = x / sc->s;
  if (is_int_fmt(d->fmt)) {
    double qmin, qmax;
    int_range(d, &qmin, &qmax);
    /* clip the rounded value (+ zero point) into the code range in binary64,
       then take the integer (so that a zero code dequantizes to +0) */
    double q = isnan(v) ? 0.0 : or_round_int((double)v, d->rounding);
    if (!d->symmetric) q += (double)sc->zp;
    /* NaN (from a NaN input, or the NaN zero point an infinite input leaves;
       both outside the contract) takes code 0 */
    if (isnan(q)) q = 0.0;
    if (q < qmin) q = qmin;
    if (q > qmax) q = qmax;
    int qi = (int)q;
    /* q - zp is exact: both are integers of at most 9 bits in the contract */
    if (d->symmetric) *xhat = (float)qi * sc->s;
    else *xhat = sc->s * (float)((double)qi - (double)sc->zp);
    *code = (uint32_t)qi & (d->fmt == OR_INT8 ? 0xFFu : 0xFu);
  } else {
    int k = elem_kind(d->fmt);
    *code = or_fp_encode(k, (double)v, 1);
    float val = (float)or_fp_decode(k, *code);
    *xhat = val * sc->s;
  }
}

/* 6-bit codes: element e occupies bits 6e .. 6e+5 of the byte stream, least
   significant bits first (it may straddle two bytes). */
static void put_code(const or_desc* d, uint8_t* codes, int64_t e, uint32_t code) {
  if (!codes) return;
  if (is_6bit(d->fmt)) {
    for (int k = 0; k < 6; k++) {
      const int64_t bit = 6 * e + k;
      uint8_t* b = &codes[bit >> 3];
      const uint8_t m = (uint8_t)(1u << (bit & 7));
      *b = (uint8_t)(((code >> k) & 1u) ? (*b | m) : (*b & (uint8_t)~m));
    }
  } else if (is_4bit(d->fmt)) {
    uint8_t* b = &codes[e >> 1];
    if ((e & 1) == 0) *b = (uint8_t)((*b & 0xF0u) | (code & 0xFu));
    else *b = (uint8_t)((*b & 0x0Fu) | ((code & 0xFu) << 4));
  } else {
    codes[e] = (uint8_t)code;
  }
}

static uint32_t get_code(const or_desc* d, const uint8_t* codes, int64_t e) {
  if (is_6bit(d->fmt)) {
    uint32_t c = 0;
    for (int k = 0; k < 6; k++) {
      const int64_t bit = 6 * e + k;
      c |= (uint32_t)((codes[bit >> 3] >> (bit & 7)) & 1u) << k;
    }
    return c;
  }
  if (is_4bit(d->fmt)) return (codes[e >> 1] >> ((e & 1) * 4)) & 0xFu;
  return codes[e];
}

static void put_y(const or_desc* d, void* y, int64_t e, float v) {
  if (!y) return;
  if (d->out_dtype == OR_F32) ((float*)y)[e] = v;
  else if (d->out_dtype == OR_BF16) ((uint16_t*)y)[e] = (uint16_t)or_fp_encode(ORK_BF16, (double)v, 0);
  else ((uint16_t*)y)[e] = (uint16_t)or_fp_encode(ORK_FP16, (double)v, 0);
}

/* binary32 results depend on the host FPU mode: insist on IEEE defaults. */
static int fpu_mode_ok(void) {
  unsigned csr = _mm_getcsr();
  const unsigned FTZ = 1u << 15, DAZ = 1u << 6, RC = 3u << 13;
  return (csr & (FTZ | DAZ | RC)) == 0u;
}

static int desc_check(const or_desc* d, int64_t cols) {
  if (d->fmt < OR_INT8 || d->fmt > OR_E3M2) return -1;
  if (d->gran < OR_TENSOR || d->gran > OR_TILE) return -1;
  if (d->scale_fmt < OR_S_F32 || d->scale_fmt > OR_S_E4M3) return -1;
  if (d->rounding != OR_RNE && d->rounding != OR_RNA) return -1;
  if (d->out_dtype < OR_F32 || d->out_dtype > OR_F16) return -1;
  if (d->hadamard != 0 && d->hadamard != 16 && d->hadamard != 32 && d->hadamard != 64 && d->hadamard != 128 &&
      d->hadamard != 256 && d->hadamard != 512 && d->hadamard != 1024)
    return -1;
  if (!d->symmetric && (!is_int_fmt(d->fmt) || (d->scale_fmt != OR_S_F32 && d->scale_fmt != OR_S_F16)))
    return -1;
  if ((d->gran == OR_BLOCK || d->gran == OR_TILE) && (d->block <= 0 || cols % d->block != 0)) return -2;
  if (d->gran == OR_TILE && d->tile_rows <= 0) return -2;
  if (is_4bit(d->fmt) && (cols % 2) != 0) return -2;
  if (is_6bit(d->fmt) && (cols % 4) != 0) return -2;   /* rows of whole bytes */
  if (d->hadamard && (cols % d->hadamard) != 0) return -2;
  if (d->two_level && (d->gran != OR_BLOCK || d->scale_fmt != OR_S_E4M3 || !d->symmetric)) return -1;
  if (!fpu_mode_ok()) return -3;
  return 0;
}

/* Copy one row and, with hadamard = n, rotate each aligned n-group. */
static int64_t load_row(const or_desc* d, const float* src, int64_t cols, float* dst) {
  int64_t bad = 0;
  for (int64_t j = 0; j < cols; j++) {
    dst[j] = src[j];
    if (!isfinite(src[j])) bad++;
  }
  if (d->hadamard)
    for (int64_t j = 0; j < cols; j += d->hadamard) or_rotate(dst + j, d->hadamard, d->signs, j);
  return bad;
}

int64_t or_tensor_stat(const or_desc* d, const float* x, int64_t rows, int64_t cols, float out[3]) {
  float amax = 0.0f, mn = INFINITY, mx = -INFINITY;
  int64_t bad = 0;
  float* row = (float*)malloc(sizeof(float) * (size_t)(cols > 0 ? cols : 1));
  for (int64_t r = 0; r < rows; r++) {
    bad += load_row(d, x + r * cols, cols, row);
    for (int64_t j = 0; j < cols; j++) {
      float a = fabsf(row[j]);
      if (a > amax) amax = a;
      if (row[j] < mn) mn = row[j];
      if (row[j] > mx) mx = row[j];
    }
  }
  free(row);
  out[0] = amax;
  out[1] = (rows > 0 && cols > 0) ? mn : 0.0f;
  out[2] = (rows > 0 && cols > 0) ? mx : 0.0f;
  return bad;
}

float or_tensor_scale(const or_desc* d, float amax) {
  const float denom = 448.0f * (float)elem_qmax(d); /* exact: at most 26 bits */
  const float S = amax / denom;
  return S == 0.0f ? 1.0f : S;
}

int or_fake_quant_rows(const or_desc* d, const float* x, int64_t nrows, int64_t cols,
                       const float tstat[3], float* tscale, uint8_t* codes, void* scales,
                       void* zeros, float* xhat, void* y, double* err2, double* sig2) {
  int rc = desc_check(d, cols);
  if (rc) return rc;
  float S = 1.0f;
  if (d->two_level) {
    if (d->given_scales) S = *tscale;
    else {
      S = or_tensor_scale(d, tstat[0]);
      if (tscale) *tscale = S;
    }
  }
  if (nrows <= 0 || cols <= 0) return 0;
  const int tile = d->gran == OR_TILE;
  const int64_t G = (d->gran == OR_BLOCK || tile) ? d->block : cols;
  const int64_t groups_per_row = cols / G;
  float* row = (float*)malloc(sizeof(float) * (size_t)cols);
  float* rq = (float*)malloc(sizeof(float) * (size_t)cols);
  float* nrm = (float*)malloc(sizeof(float) * (size_t)cols);
  /* 2-D tiles (playbook §4.4): one scale per tile_rows x block elements, from
     the statistic of the whole tile, so every band of tile_rows rows is read
     once for the statistics and once more to quantize */
  scale_t* tsc = NULL;
  if (tile) {
    const int64_t bands = (nrows + d->tile_rows - 1) / d->tile_rows;
    tsc = (scale_t*)malloc(sizeof(scale_t) * (size_t)(bands * groups_per_row));
    float* st = (float*)malloc(sizeof(float) * 3 * (size_t)groups_per_row);
    for (int64_t b = 0; b < bands; b++) {
      for (int64_t g = 0; g < groups_per_row; g++) {
        st[3 * g] = 0.0f;
        st[3 * g + 1] = INFINITY;
        st[3 * g + 2] = -INFINITY;
      }
      for (int64_t r = b * d->tile_rows; r < nrows && r < (b + 1) * d->tile_rows; r++) {
        load_row(d, x + r * cols, cols, row);
        for (int64_t j = 0; j < cols; j++) {
          float* t = st + 3 * (j / G);
          if (fabsf(row[j]) > t[0]) t[0] = fabsf(row[j]);
          if (row[j] < t[1]) t[1] = row[j];
          if (row[j] > t[2]) t[2] = row[j];
        }
      }
      for (int64_t g = 0; g < groups_per_row; g++) {
        const int64_t sidx = b * groups_per_row + g;
        if (d->given_scales) {
          tsc[sidx] = scale_given(d, scales, zeros, sidx);
        } else {
          tsc[sidx] = d->symmetric ? scale_sym(d, st[3 * g]) : scale_asym(d, st[3 * g + 1], st[3 * g + 2]);
          put_scale(d, scales, zeros, sidx, &tsc[sidx]);
        }
      }
    }
    free(st);
  }
  double e2 = 0.0, s2 = 0.0;
  for (int64_t r = 0; r < nrows; r++) {
    load_row(d, x + r * cols, cols, row);
    /* two-level: the whole tensor is normalized by S first, and the blocks
       quantize the quotients (playbook §4.3.2) */
    for (int64_t j = 0; j < cols; j++) nrm[j] = d->two_level ? row[j] / S : row[j];
    for (int64_t g = 0; g < groups_per_row; g++) {
      const float* v = nrm + g * G;
      const float* xo = row + g * G;
      int64_t sidx = (d->gran == OR_TENSOR) ? 0 : (d->gran == OR_CHANNEL) ? r : r * groups_per_row + g;
      scale_t sc;
      if (tile) {
        sc = tsc[(r / d->tile_rows) * groups_per_row + g];
      } else {
        float amax, mn, mx;
        if (d->gran == OR_TENSOR) {
          amax = tstat[0]; mn = tstat[1]; mx = tstat[2];
        } else {
          amax = 0.0f; mn = INFINITY; mx = -INFINITY;
          for (int64_t j = 0; j < G; j++) {
            float a = fabsf(v[j]);
            if (a > amax) amax = a;
            if (v[j] < mn) mn = v[j];
            if (v[j] > mx) mx = v[j];
          }
        }
        if (d->given_scales) sc = scale_given(d, scales, zeros, sidx);
        else sc = d->symmetric ? scale_sym(d, amax) : scale_asym(d, mn, mx);
        if (!d->given_scales) put_scale(d, scales, zeros, sidx, &sc);
      }
      for (int64_t j = 0; j < G; j++) {
        uint32_t code;
        float xh;
        quant_elem(d, v[j], &sc, &code, &xh);
        if (d->two_level) xh = xh * S; /* x = x_q * s_block * S_tensor, left to right */
        int64_t col = g * G + j;
        put_code(d, codes, r * cols + col, code);
        rq[col] = xh;
        double diff = (double)xo[j] - (double)xh;
        e2 += diff * diff;
        s2 += (double)xo[j] * (double)xo[j];
      }
    }
    if (xhat) memcpy(xhat + r * cols, rq, sizeof(float) * (size_t)cols);
    if (y) {
      if (d->hadamard && d->unrotate_y)
        for (int64_t j = 0; j < cols; j += d->hadamard) or_unrotate(rq + j, d->hadamard, d->signs, j);
      for (int64_t j = 0; j < cols; j++) put_y(d, y, r * cols + j, rq[j]);
    }
  }
  free(row);
  free(rq);
  free(nrm);
  free(tsc);
  if (err2) *err2 += e2;
  if (sig2) *sig2 += s2;
  return 0;
}

int or_dequant_rows(const or_desc* d, const uint8_t* codes, const void* scales,
                    const void* zeros, float tscale, int64_t nrows, int64_t cols, void* y) {
  int rc = desc_check(d, cols);
  if (rc) return rc;
  if (nrows <= 0 || cols <= 0) return 0;
  const int64_t G = (d->gran == OR_BLOCK || d->gran == OR_TILE) ? d->block : cols;
  const int64_t groups_per_row = cols / G;
  float* rq = (float*)malloc(sizeof(float) * (size_t)cols);
  for (int64_t r = 0; r < nrows; r++) {
    for (int64_t g = 0; g < groups_per_row; g++) {
      int64_t sidx = (d->gran == OR_TENSOR)    ? 0
                     : (d->gran == OR_CHANNEL) ? r
                     : (d->gran == OR_TILE)    ? (r / d->tile_rows) * groups_per_row + g
                                               : r * groups_per_row + g;
      scale_t sc = scale_given(d, scales, zeros, sidx);
      for (int64_t j = 0; j < G; j++) {
        int64_t col = g * G + j;
        uint32_t c = get_code(d, codes, r * cols + col);
        float xh;
        if (is_int_fmt(d->fmt)) {
          int q = (d->fmt == OR_INT8) ? (int)(int8_t)(uint8_t)c : ((c & 8u) ? (int)c - 16 : (int)c);
          if (sc.s == 0.0f) xh = 0.0f;
          else if (d->symmetric) xh = (float)q * sc.s;
          else xh = sc.s * (float)((double)q - (double)sc.zp);
        } else if (sc.s == 0.0f) {
          xh = 0.0f;
        } else {
          xh = (float)or_fp_decode(elem_kind(d->fmt), c) * sc.s;
        }
        if (d->two_level) xh = xh * tscale;
        rq[col] = xh;
      }
    }
    if (d->hadamard && d->unrotate_y)
      for (int64_t j = 0; j < cols; j += d->hadamard) or_unrotate(rq + j, d->hadamard, d->signs, j);
    for (int64_t j = 0; j < cols; j++) put_y(d, y, r * cols + j, rq[j]);
  }
  free(rq);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Win counts of a sweep (cyqw.cn/news/1000169 §5.1 reports how often the     */
/* integer format beats the float one; here each tensor and granularity is a  */
/* contest). A pair is decided only when its difference sits clear of the tie */
/* band's edge by more than margin_db; otherwise it is left undecided.        */
/* ------------------------------------------------------------------------ */
enum { OR_WIN_INT = 0, OR_WIN_FP = 1, OR_TIE = 2, OR_UNDECIDED = 3 };

static int contest(double q_int, double q_fp, double tie_db, double margin_db) {
  if (isnan(q_int) || isnan(q_fp)) return OR_UNDECIDED;
  const double d = (q_int == q_fp) ? 0.0 : q_int - q_fp; /* +inf vs +inf: equal */
  const double a = fabs(d);
  if (a < tie_db - margin_db) return OR_TIE;
  if (a > tie_db + margin_db) return d > 0.0 ? OR_WIN_INT : OR_WIN_FP;
  return OR_UNDECIDED;
}

int or_sweep_tally(const double* qsnr, int64_t n_tensors, double tie_db, double margin_db, int32_t* counts) {
  /* format slots of the table and the three integer-vs-float pairs */
  static const int int_slot[3] = {OR_INT8, OR_INT8, OR_INT4};
  static const int fp_slot[3] = {OR_E4M3, OR_E5M2, OR_E2M1};
  if (n_tensors < 0 || counts == NULL || (n_tensors > 0 && qsnr == NULL)) return -1;
  if (!(margin_db >= 0.0 && margin_db < tie_db)) return -1;
  for (int i = 0; i < 5 * 3 * 4; i++) counts[i] = 0;
  for (int64_t t = 0; t < n_tensors; t++) {
    for (int g = 0; g < 5; g++) {
      for (int p = 0; p < 3; p++) {
        const double qi = qsnr[t * 25 + int_slot[p] * 5 + g];
        const double qf = qsnr[t * 25 + fp_slot[p] * 5 + g];
        counts[(g * 3 + p) * 4 + contest(qi, qf, tie_db, margin_db)] += 1;
      }
    }
  }
  return 0;
}
