// The step kernels of rank class KB = 8 (R = 256).
#include "step_kernel.h"

namespace markov_impl {
StepFn step_kernel_kb8(int rg, int mrb, bool exact) {
  return exact ? pick_plan<8, true>(rg, mrb) : pick_plan<8, false>(rg, mrb);
}
}  // namespace markov_impl
