// LayerNorm kernels instantiated for a FP32 gamma/beta.
#include "ln_kernels.h"

namespace rmsn {

int launch_ln_fwd_f32w(const LnFwdParams& p, const Route& rt, hipStream_t s) {
    return launch_ln_fwd_wt<float>(p, rt, s);
}

int launch_ln_bwd_row_f32w(const LnBwdParams& p, const Route& rt, hipStream_t s) {
    return launch_ln_bwd_wt<float>(p, rt, s);
}

}  // namespace rmsn
