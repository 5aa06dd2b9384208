// lq_inst.hip — instantiates the flat and row kernels for one pair of input
// and output dtypes. Compiled once per pair with -DLQ_INST_DT=d -DLQ_INST_ODT=o
// (0 fp32, 1 bf16, 2 fp16).
#include "lq_kernels.h"

#if !defined(LQ_INST_DT) || !defined(LQ_INST_ODT)
#error "LQ_INST_DT and LQ_INST_ODT must be defined"
#endif
#define LQ_CAT3_(a, b, c) a##b##_##c
#define LQ_CAT3(a, b, c) LQ_CAT3_(a, b, c)

namespace lqd {

template <int F>
static void fill(KernelSet& k) {
  k.flat[F][FLAT_BLOCK] = &launch_flat<LQ_INST_DT, F, LQ_INST_ODT, FLAT_BLOCK>;
  k.flat[F][FLAT_TENSOR] = &launch_flat<LQ_INST_DT, F, LQ_INST_ODT, FLAT_TENSOR>;
  k.flat[F][FLAT_TWO] = &launch_flat<LQ_INST_DT, F, LQ_INST_ODT, FLAT_TWO>;
  k.row[F][0] = &launch_row<LQ_INST_DT, F, LQ_INST_ODT, 1>;
  k.row[F][1] = &launch_row<LQ_INST_DT, F, LQ_INST_ODT, 2>;
  k.row[F][2] = &launch_row<LQ_INST_DT, F, LQ_INST_ODT, 4>;
  k.row[F][3] = &launch_row<LQ_INST_DT, F, LQ_INST_ODT, 0>;
}

void LQ_CAT3(kernels_, LQ_INST_DT, LQ_INST_ODT)(KernelSet& k) {
  fill<LQ_INT8>(k);
  fill<LQ_INT4>(k);
  fill<LQ_E4M3>(k);
  fill<LQ_E5M2>(k);
  fill<LQ_E2M1>(k);
  fill<LQ_E2M3>(k);
  fill<LQ_E3M2>(k);
}

}  // namespace lqd
