// One (rank class, variant) pair of step kernels: the build compiles this
// file once per pair listed in MARKOV_STEP_INSTANCES, with -DSTEP_KB and
// -DSTEP_VAR, so the pairs compile in parallel.
#include "step_kernel.h"

#if !defined(STEP_KB) || !defined(STEP_VAR)
#error "build with -DSTEP_KB=<rank class> -DSTEP_VAR=<variant>"
#endif

#define MARKOV_PICKER_NAME2(KB, VAR) step_kernel_kb##KB##_v##VAR
#define MARKOV_PICKER_NAME(KB, VAR) MARKOV_PICKER_NAME2(KB, VAR)

namespace markov_impl {
StepFn MARKOV_PICKER_NAME(STEP_KB, STEP_VAR)(int rg, int mrb) { return pick_plan<STEP_KB, STEP_VAR>(rg, mrb); }
}  // namespace markov_impl
