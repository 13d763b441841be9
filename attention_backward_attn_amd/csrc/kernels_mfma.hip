// bf16 matrix-core backward (placeholder until the MFMA kernels land).
#include "kernels.h"

namespace attn {

bool mfma_bwd_supported(const Params&) { return false; }

hipError_t launch_bwd_mfma(const Params&, const BwdArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace attn
