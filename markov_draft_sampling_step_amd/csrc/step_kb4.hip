// The step kernels of rank class KB = 4 (R = 128).
#include "step_kernel.h"

namespace markov_impl {
StepFn step_kernel_kb4(int rg, int mrb, bool exact) {
  return exact ? pick_plan<4, true>(rg, mrb) : pick_plan<4, false>(rg, mrb);
}
}  // namespace markov_impl
