// The step kernels of rank class KB = 2 (R = 64).
#include "step_kernel.h"

namespace markov_impl {
StepFn step_kernel_kb2(int rg, int mrb, bool exact) {
  return exact ? pick_plan<2, true>(rg, mrb) : pick_plan<2, false>(rg, mrb);
}
}  // namespace markov_impl
