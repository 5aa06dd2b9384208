// lq_fast.hip — instantiates the specialised per-block kernels for one dtype
// (the same for input and output). Compiled once with -DLQ_FAST_DT=0 (fp32)
// and once with -DLQ_FAST_DT=1 (bf16).
#include "lq_fast.h"

#ifndef LQ_FAST_DT
#error "LQ_FAST_DT must be defined"
#endif
#define LQ_CAT2_(a, b) a##b
#define LQ_CAT2(a, b) LQ_CAT2_(a, b)

namespace lqd {

template <int F, int SF, bool SYM, bool HAD>
static void put(FastSet& k) {
  if constexpr (HAD && SYM) k.wrot[F][SF] = &launch_fast_wrot<LQ_FAST_DT, F, LQ_FAST_DT, SF, true>;
  k.k[F][SF][SYM ? 0 : 1][HAD ? 1 : 0][0] = &launch_fast<LQ_FAST_DT, F, LQ_FAST_DT, SF, SYM, HAD, false>;
  if constexpr (fast_can_be_wide(LQ_FAST_DT, HAD, F))
    k.k[F][SF][SYM ? 0 : 1][HAD ? 1 : 0][1] = &launch_fast<LQ_FAST_DT, F, LQ_FAST_DT, SF, SYM, HAD, true>;
}

// two-level: symmetric E4M3 block scales under the tensor scale (with
// rotation also the 512/1024-column kernel)
template <int F, bool HAD>
static void put_two(FastSet& k) {
  if constexpr (HAD) k.wrot_two[F] = &launch_fast_wrot<LQ_FAST_DT, F, LQ_FAST_DT, LQ_SCALE_E4M3, true, true>;
  k.two[F][HAD ? 1 : 0][0] = &launch_fast<LQ_FAST_DT, F, LQ_FAST_DT, LQ_SCALE_E4M3, true, HAD, false, true>;
  if constexpr (fast_can_be_wide(LQ_FAST_DT, HAD, F))
    k.two[F][HAD ? 1 : 0][1] = &launch_fast<LQ_FAST_DT, F, LQ_FAST_DT, LQ_SCALE_E4M3, true, HAD, true, true>;
}

template <int F, int SF>
static void put_tile(FastSet& k) {
  k.tile[F][SF][0] = &launch_tile<LQ_FAST_DT, F, SF, 1>;
  k.tile[F][SF][1] = &launch_tile<LQ_FAST_DT, F, SF, 2>;
  k.tile[F][SF][2] = &launch_tile<LQ_FAST_DT, F, SF, 4>;
}

template <int F>
static void for_fp6(FastSet& k) {
  put_two<F, false>(k);
  put_two<F, true>(k);
  put<F, LQ_SCALE_F32, true, false>(k);
  put<F, LQ_SCALE_F16, true, false>(k);
  put<F, LQ_SCALE_UE8M0, true, false>(k);
  put<F, LQ_SCALE_E4M3, true, false>(k);
}

template <int F>
static void put_all_scales(FastSet& k) {
  put_two<F, false>(k);
  put_two<F, true>(k);
  put_tile<F, LQ_SCALE_F32>(k);
  put_tile<F, LQ_SCALE_F16>(k);
  put_tile<F, LQ_SCALE_UE8M0>(k);
  put_tile<F, LQ_SCALE_E4M3>(k);
  put<F, LQ_SCALE_F32, true, false>(k);
  put<F, LQ_SCALE_F16, true, false>(k);
  put<F, LQ_SCALE_UE8M0, true, false>(k);
  put<F, LQ_SCALE_E4M3, true, false>(k);
}

void LQ_CAT2(fast_kernels_, LQ_FAST_DT)(FastSet& k) {
  for (auto& a : k.k)
    for (auto& b : a)
      for (auto& c : b)
        for (auto& d : c)
          for (auto& e : d) e = nullptr;
  for (auto& a : k.two)
    for (auto& b : a)
      for (auto& c : b) c = nullptr;
  for (auto& a : k.wrot)
    for (auto& b : a) b = nullptr;
  for (auto& a : k.wrot_two) a = nullptr;
  for (auto& a : k.tile)
    for (auto& b : a)
      for (auto& c : b) c = nullptr;
  put_all_scales<LQ_INT8>(k);
  put_all_scales<LQ_INT4>(k);
  put_all_scales<LQ_E4M3>(k);
  put_all_scales<LQ_E5M2>(k);
  put_all_scales<LQ_E2M1>(k);
  // FP6 (MXFP6): symmetric block scales of every format, no 2-D tile kernel
  for_fp6<LQ_E2M3>(k);
  for_fp6<LQ_E3M2>(k);
  // zero-point (integer formats, fp32/fp16 scales)
  put<LQ_INT8, LQ_SCALE_F32, false, false>(k);
  put<LQ_INT8, LQ_SCALE_F16, false, false>(k);
  put<LQ_INT4, LQ_SCALE_F32, false, false>(k);
  put<LQ_INT4, LQ_SCALE_F16, false, false>(k);
  // rotation: NV-style 4-bit blocks (E4M3 scales) and MX-style 8-bit blocks (UE8M0)
  put<LQ_INT4, LQ_SCALE_E4M3, true, true>(k);
  put<LQ_E2M1, LQ_SCALE_E4M3, true, true>(k);
  put<LQ_INT8, LQ_SCALE_UE8M0, true, true>(k);
  put<LQ_E4M3, LQ_SCALE_UE8M0, true, true>(k);
  put<LQ_E5M2, LQ_SCALE_UE8M0, true, true>(k);
}

}  // namespace lqd
