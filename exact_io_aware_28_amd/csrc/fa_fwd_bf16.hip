// Forward entry points (bf16 and fp16): d = 64 and the biased d = 128
// kernels are instantiated here; the other d = 128 kernels in
// fa_fwd_bf16_d128.hip, which is built with the max-ILP instruction
// scheduler (1-2 % faster for them, slower for these).
#include "fa_fwd_kernel.h"

namespace fa {
namespace {

template <int D, bool CAUSAL, bool WINDOW, bool F16>
hipError_t launch3(const FwdParams& p, hipStream_t stream) {
  // a bias or dropout only reaches the bf16 entry points (dense batches for
  // a bias, no bias with dropout)
  if constexpr (D == 128) {
    if constexpr (!F16) {
      if (p.bias) return launch_w<128, 8, CAUSAL, WINDOW, false, false, true>(p, stream);
    }
    return launch_fwd_d128(p, stream, F16);  // fa_fwd_bf16_d128.hip
  } else {
    if constexpr (!F16) {
      if (p.bias) return launch_w<64, 4, CAUSAL, WINDOW, false, false, true>(p, stream);
      if (p.dropout) {
        if (p.cu_seqlens) return launch_w<64, 4, CAUSAL, WINDOW, true, false, false, true>(p, stream);
        return launch_w<64, 4, CAUSAL, WINDOW, false, false, false, true>(p, stream);
      }
    }
    if (p.cu_seqlens) return launch_w<64, 4, CAUSAL, WINDOW, true, F16>(p, stream);
    return launch_w<64, 4, CAUSAL, WINDOW, false, F16>(p, stream);
  }
}

template <int D, bool F16>
hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
  const bool win = p.window > 0;
  if (p.causal)
    return win ? launch3<D, true, true, F16>(p, stream) : launch3<D, true, false, F16>(p, stream);
  return win ? launch3<D, false, true, F16>(p, stream) : launch3<D, false, false, F16>(p, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  return p.d == 64 ? launch_d<64, false>(p, stream) : launch_d<128, false>(p, stream);
}

hipError_t launch_fwd_f16(const FwdParams& p, hipStream_t stream) {
  return p.d == 64 ? launch_d<64, true>(p, stream) : launch_d<128, true>(p, stream);
}

}  // namespace fa
