// Stand-ins for the kernel launchers of libwattn.so, for the sanitizer build of the host API
// (wattn_api.cpp) that tests/test_sanitized_abi.py makes.  That build has no device code: every
// call that passes the host checks reaches one of these and gets an error back, so only the
// host-side argument checks run, under AddressSanitizer and UndefinedBehaviorSanitizer.

#include <hip/hip_runtime_api.h>

#include "wattn_aux_plan.h"
#include "wattn_plan.h"

hipError_t wattn_launch_bf16(const WattnPlan&, int, bool, bool, const void*, const void*, const void*, void*,
                             const float*, const void*, const void*, float*, const void*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t wattn_launch_bwd(const WattnPlan&, bool, bool, const void*, const void*, const void*, const void*,
                            const void*, const float*, float*, float*, float*, float*, float*, const float*,
                            const void*, const void*, int, float*, float*, const void*, float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t wattn_launch_select(const float*, int, float, int*, int*, hipStream_t) { return hipErrorNoDevice; }
hipError_t wattn_launch_local(const LocalPlan&, bool, const void*, const void*, const void*, void*, const int*,
                              const int*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t wattn_launch_gated(const LocalPlan&, bool, const void*, const void*, const void*, void*, const float*,
                              float, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t wattn_launch_cla(const ClaPlan&, const void*, const float*, const float*, const float*, const float*,
                            void*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t wattn_launch_linear(const LinearPlan&, int, bool, bool, const void*, const void*, const float*,
                               const void*, void*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t wattn_launch_layernorm(const NormPlan&, bool, const void*, const float*, const float*, void*,
                                  hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t wattn_launch_stem(const StemPlan&, const void*, const void*, const float*, void*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t wattn_launch_token_mean(const void*, void*, int, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t wattn_launch_f32(const WattnF32Plan&, int, const void*, const void*, const void*, void*, const float*,
                            const void*, const void*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t wattn_noalloc_scratch(hipStream_t, void** out) {
  *out = nullptr;
  return hipErrorNoDevice;
}
