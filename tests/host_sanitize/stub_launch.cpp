// Launchers of the host-sanitizer build: they stand in for the HIP kernels, so
// that every path of the C ABI up to the launch can run under AddressSanitizer
// and UndefinedBehaviorSanitizer on a machine without a GPU. Each reports "no
// device", which the ABI maps to LIGER_E_HIP. Nothing is dereferenced.
#include "kernels.h"

namespace liger {

hipError_t launch_decode_step(const DecodeArgs&) { return hipErrorNoDevice; }
hipError_t launch_ring_fill(const RingFillArgs&) { return hipErrorNoDevice; }
hipError_t launch_ring_append(const RingFillArgs&) { return hipErrorNoDevice; }
hipError_t launch_prefill(const PrefillArgs&) { return hipErrorNoDevice; }
hipError_t launch_full_attn(const FullAttnArgs&) { return hipErrorNoDevice; }
hipError_t launch_carry_scan(float*, int64_t, int, int64_t, int, void*) { return hipErrorNoDevice; }
hipError_t launch_backward(const BackwardArgs&) { return hipErrorNoDevice; }

}  // namespace liger
