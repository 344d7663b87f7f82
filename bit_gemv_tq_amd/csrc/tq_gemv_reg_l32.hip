// tq_gemv_reg_l32.hip -- instantiations of the register-resident M = 1 GEMV
// (tq_gemv_reg.h) for 32-lane teams; split per team width so the library
// builds in parallel.
#include "tq_gemv_reg.h"

namespace tq {
TQ_DEFINE_LAUNCH_REG(32)
}  // namespace tq
