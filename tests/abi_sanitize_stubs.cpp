// Kernel launchers replaced by stubs, for the host-sanitizer build of the C
// ABI layer (api.cpp, route.cpp): every launch reports RMSN_ERR_LAUNCH, so the
// driver exercises argument checking, aliasing spans and the route table
// with no GPU and no device code. Test infrastructure only.
#include "../bwd_rmsnorm_fwd_02_amd/csrc/rmsn_internal.h"

namespace rmsn {
int launch_fwd(const FwdParams&, const Route&, rmsn_dtype_t, bool, hipStream_t) { return RMSN_ERR_LAUNCH; }
int launch_bwd_row(const BwdParams&, const Route&, rmsn_dtype_t, int, hipStream_t) { return RMSN_ERR_LAUNCH; }
int launch_dw_reduce(const BwdParams&, const Route&, hipStream_t) { return RMSN_ERR_LAUNCH; }
int launch_col_reduce(const void*, const Route&, int32_t, float*, float*, int32_t, hipStream_t) {
    return RMSN_ERR_LAUNCH;
}
int launch_ln_fwd(const LnFwdParams&, const Route&, rmsn_dtype_t, hipStream_t) { return RMSN_ERR_LAUNCH; }
int launch_ln_bwd_row(const LnBwdParams&, const Route&, rmsn_dtype_t, hipStream_t) { return RMSN_ERR_LAUNCH; }
int launch_bwd_small(const BwdParams&, const Route&, rmsn_dtype_t, bool, hipStream_t) { return RMSN_ERR_LAUNCH; }
int launch_fill_zero(void*, size_t, hipStream_t) { return RMSN_ERR_LAUNCH; }
int launch_dw_reduce_batch(const DwJobs&, int64_t, hipStream_t) { return RMSN_ERR_LAUNCH; }
}  // namespace rmsn
