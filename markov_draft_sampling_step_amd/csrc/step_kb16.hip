// The step kernels of rank class KB = 16 (R = 512).
#include "step_kernel.h"

namespace markov_impl {
StepFn step_kernel_kb16(int rg, int mrb, bool exact) {
  return exact ? pick_plan<16, true>(rg, mrb) : pick_plan<16, false>(rg, mrb);
}
}  // namespace markov_impl
