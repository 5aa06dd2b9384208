// lq_inst.hip — instantiates the flat and row kernels for one input dtype.
// Compiled once per dtype with -DLQ_INST_DT=0 (fp32), 1 (bf16) or 2 (fp16).
#include "lq_kernels.h"

#ifndef LQ_INST_DT
#error "LQ_INST_DT must be defined"
#endif
#define LQ_CAT2(a, b) a##b
#define LQ_CAT(a, b) LQ_CAT2(a, b)

namespace lqd {

template <int F>
static void fill_flat(flat_fn out[2]) {
  out[0] = &launch_flat<LQ_INST_DT, F, false>;
  out[1] = &launch_flat<LQ_INST_DT, F, true>;
}
template <int F>
static void fill_row(flat_fn out[4]) {
  out[0] = &launch_row<LQ_INST_DT, F, 1>;
  out[1] = &launch_row<LQ_INST_DT, F, 2>;
  out[2] = &launch_row<LQ_INST_DT, F, 4>;
  out[3] = &launch_row<LQ_INST_DT, F, 0>;
}

void LQ_CAT(flat_table_, LQ_INST_DT)(flat_fn out[5][2]) {
  fill_flat<LQ_INT8>(out[LQ_INT8]);
  fill_flat<LQ_INT4>(out[LQ_INT4]);
  fill_flat<LQ_E4M3>(out[LQ_E4M3]);
  fill_flat<LQ_E5M2>(out[LQ_E5M2]);
  fill_flat<LQ_E2M1>(out[LQ_E2M1]);
}

void LQ_CAT(row_table_, LQ_INST_DT)(flat_fn out[5][4]) {
  fill_row<LQ_INT8>(out[LQ_INT8]);
  fill_row<LQ_INT4>(out[LQ_INT4]);
  fill_row<LQ_E4M3>(out[LQ_E4M3]);
  fill_row<LQ_E5M2>(out[LQ_E5M2]);
  fill_row<LQ_E2M1>(out[LQ_E2M1]);
}

}  // namespace lqd
