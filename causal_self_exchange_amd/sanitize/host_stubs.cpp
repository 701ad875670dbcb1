// Host-only stand-ins for the device-side functions the C API calls, for a
// build of relation_api.cpp with the host compiler's AddressSanitizer and
// UndefinedBehaviorSanitizer (the argument checks, workspace queries, status
// strings and kernel selection, none of which launches anything). Every
// launcher reports a launch failure; no MFMA kernel is reported available.
#include "rel_internal.h"

namespace rel {

hipError_t launch_fwd_scan(const FwdArgs&, const HeadParams&, bool, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t device_cu_count(int* n_cu) { *n_cu = 1; return hipSuccess; }
hipError_t launch_fwd_mfma_bf16(const FwdArgs&, const HeadParams&, hipStream_t, const RopeParams*) { return hipErrorLaunchFailure; }
bool fwd_mfma_rope_fusable(int, int) { return false; }
bool fwd_mfma_supported(int, int) { return false; }
hipError_t launch_bwd_prep(const BwdArgs&, const HeadParams&, bool, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_bwd_scan(const BwdArgs&, const HeadParams&, bool, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_bwd_mfma_bf16(const BwdArgs&, const HeadParams&, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_bwd_reduce(const BwdArgs&, hipStream_t) { return hipErrorLaunchFailure; }
bool bwd_mfma_supported(int, int) { return false; }
bool bwd_du_supported(int d_h, int T) {
  return (d_h == 32 || d_h == 48 || d_h == 64 || d_h == 80 || d_h == 128) && bwd_du_head_bytes(T) < 0x7fff0000LL;
}
hipError_t launch_prestep(const PrestepArgs&, const PrestepParams&, bool, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_linear(const LinArgs&, const HeadParams&, bool, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t launch_decode(const DecodeArgs&, const HeadParams&, bool, hipStream_t) { return hipErrorLaunchFailure; }
hipError_t decode_scratch(void**) { return hipErrorLaunchFailure; }
hipError_t launch_cache_append(void*, void*, int32_t*, const void*, const void*, int, int, int, int, bool,
                               hipStream_t) {
  return hipErrorLaunchFailure;
}

}  // namespace rel
