// Stand-ins for the kernel launchers, for the host AddressSanitizer build of
// the C ABI layer (csrc/fa_api.hip): every launcher reports failure without
// touching a GPU, so the checks of each entry point run instrumented and a
// call that passes them returns FA_ERR_HIP instead of launching.
#include "fa_params.h"

namespace fa {

hipError_t launch_fwd_bf16(const FwdParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fwd_f16(const FwdParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fwd_d128(const FwdParams&, hipStream_t, bool) { return hipErrorNotSupported; }
hipError_t launch_fwd_f32(const FwdParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_bf16(const BwdParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_f16(const BwdParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_decode_bf16(const DecodeParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fwd_fp8(const Fp8FwdParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_quantize_fp8(const QuantParams&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace fa
