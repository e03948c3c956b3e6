// LayerNorm kernels instantiated for a BF16 gamma/beta.
#include "ln_kernels.h"

namespace rmsn {

int launch_ln_fwd_bf16w(const LnFwdParams& p, const Route& rt, hipStream_t s) {
    return launch_ln_fwd_wt<uint16_t>(p, rt, s);
}

int launch_ln_bwd_row_bf16w(const LnBwdParams& p, const Route& rt, hipStream_t s) {
    return launch_ln_bwd_wt<uint16_t>(p, rt, s);
}

}  // namespace rmsn
