// tq_gemv_reg_l256_gemv.hip -- instantiations of the register-resident M = 1
// GEMV (tq_gemv_reg.h) for 256-lane teams, one weight stream (with the
// RMSNorm prologue forms); split per team width and stream count so the
// library builds in parallel.
#include "tq_gemv_reg.h"

namespace tq {
TQ_DEFINE_LAUNCH_REG_GEMV(256)
}  // namespace tq
