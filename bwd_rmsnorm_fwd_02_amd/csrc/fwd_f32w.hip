// Forward kernels instantiated for a FP32 weight.
#include "fwd_kernels.h"

namespace rmsn {

int launch_fwd_f32w(const FwdParams& p, const Route& rt, bool residual, hipStream_t s) {
    return launch_fwd_wt<float>(p, rt, residual, s);
}

}  // namespace rmsn
