// Backward kernels instantiated for a FP32 weight.
#include "bwd_kernels.h"

namespace rmsn {

int launch_bwd_row_f32w(const BwdParams& p, const Route& rt, int form, hipStream_t s) {
    return launch_bwd_row_wt<float, false>(p, rt, form, s);
}

int launch_bwd_small_f32w(const BwdParams& p, const Route& rt, bool residual, hipStream_t s) {
    return launch_bwd_small_wt<float>(p, rt, residual, s);
}

}  // namespace rmsn
