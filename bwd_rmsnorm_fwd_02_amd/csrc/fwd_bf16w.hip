// Forward kernels instantiated for a BF16 weight.
#include "fwd_kernels.h"

namespace rmsn {

int launch_fwd_bf16w(const FwdParams& p, const Route& rt, bool residual, hipStream_t s) {
    return launch_fwd_wt<uint16_t>(p, rt, residual, s);
}

}  // namespace rmsn
