// The step kernels of rank class KB = 1 (R = 16 and 32).
#include "step_kernel.h"

namespace markov_impl {
StepFn step_kernel_kb1(int rg, int mrb, bool exact) {
  return exact ? pick_plan<1, true>(rg, mrb) : pick_plan<1, false>(rg, mrb);
}
}  // namespace markov_impl
