// Stand-ins for the kernel dispatchers of the HIP library, for a host-only
// build of the C ABI layer (la_api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer. Each returns success without launching, so the
// ABI's validation, planning and workspace carving run exactly as in the
// library while no device code is involved. Test infrastructure only.
#include "la_kernels.h"

namespace la {

hipError_t prefill_dispatch(const FwdArgs&, const ScanArgs&, int, int, int, int, bool, bool, hipStream_t,
                            hipEvent_t*) {
  return hipSuccess;
}
hipError_t scan_dispatch(const ScanArgs&, hipStream_t) { return hipSuccess; }
bool perf_fused_supported(int D, int DF, int dtype, bool causal, bool decay) {
  if (dtype != 1 || decay) return false;
  (void)causal;
  return (D == 32 && (DF == 64 || DF == 128)) || (D == 64 && (DF == 64 || DF == 128 || DF == 256)) ||
         (D == 128 && (DF == 64 || DF == 128));
}
hipError_t perf_fused_dispatch(const FwdArgs&, const ScanArgs&, int, int, bool, hipStream_t, hipEvent_t*) {
  return hipSuccess;
}
hipError_t backward_dispatch(const FwdArgs&, const ScanArgs&, const BwdArgs&, const ScanArgs&, int, int, int, bool,
                             hipStream_t) {
  return hipSuccess;
}
hipError_t gated_dispatch(const GatedArgs&, const ScanArgs&, int, int, int, hipStream_t) { return hipSuccess; }
hipError_t decode_dispatch(const DecodeArgs&, int, int, int, int, hipStream_t) { return hipSuccess; }
int poly_partials(int D) { return D == 32 ? 2 : 4; }
int poly_den_slots(int D) { return D == 32 ? 2 : 4; }
hipError_t poly_forward_dispatch(const PolyArgs&, int, int, bool, hipStream_t) { return hipSuccess; }
hipError_t poly_decode_dispatch(const DecodeArgs&, int, int, hipStream_t) { return hipSuccess; }
hipError_t poly_fmap_dispatch(const FmapArgs&, int, int, int, hipStream_t) { return hipSuccess; }
hipError_t fmap_dispatch(const FmapArgs&, int, int, int, int, int, hipStream_t) { return hipSuccess; }
hipError_t copy_state_dispatch(const float*, const float*, float*, float*, long long, long long, hipStream_t) {
  return hipSuccess;
}

}  // namespace la
