// Kernel launchers for the host-only sanitizer build of the planner: the
// driver calls only the pure-host entry points (validation, planning,
// workspace size, plan description), so none of these may run; each returns
// an error if one ever does.
#include "muon_internal.h"

namespace muon {

hipError_t launch_momentum(bool, const UnitDev*, const EwTask*, int, const K1Params&, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_gemm(int, bool, int, const UnitDev*, const GemmTask*, int, const GemmParams&, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_update(bool, const UnitDev*, const EwTask*, int, const K5Params&, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_precond_refresh(const PrecondBlockDev&, const void*, int64_t, int64_t, bool, float, uint32_t*,
                                  hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_precond_accumulate(const PrecondBlockDev&, const void*, int64_t, int64_t, bool, float, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_precond_refresh_accumulated(const PrecondBlockDev&, float, bool, uint32_t*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_precond_apply(const PrecondDev*, const ApplyTask*, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_identity(uint16_t*, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_adam_tick(AdamState*, float, float, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_adam_set(AdamState*, uint32_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_adamw(const AdamDev*, const AdamTask*, int, const AdamParams&, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace muon
