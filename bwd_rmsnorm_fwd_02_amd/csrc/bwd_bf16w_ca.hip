// Backward row kernels with the one-step slot combine, for a BF16 weight (a
// translation unit of their own, compiled in parallel with the others).
#include "bwd_kernels.h"

namespace rmsn {

int launch_bwd_row_bf16w_ca(const BwdParams& p, const Route& rt, int form, hipStream_t s) {
    return launch_bwd_row_wt<uint16_t, true>(p, rt, form, s);
}

}  // namespace rmsn
