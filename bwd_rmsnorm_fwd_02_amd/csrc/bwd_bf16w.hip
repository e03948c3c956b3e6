// Backward kernels instantiated for a BF16 weight.
#include "bwd_kernels.h"

namespace rmsn {

int launch_bwd_row_bf16w(const BwdParams& p, const Route& rt, int form, hipStream_t s) {
    return launch_bwd_row_wt<uint16_t, false>(p, rt, form, s);
}

int launch_bwd_small_bf16w(const BwdParams& p, const Route& rt, bool residual, hipStream_t s) {
    return launch_bwd_small_wt<uint16_t>(p, rt, residual, s);
}

}  // namespace rmsn
