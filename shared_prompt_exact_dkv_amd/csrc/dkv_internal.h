// dkv_internal.h -- entry points shared between the library's translation units.
#pragma once

#include "../../include/dkv.h"

namespace dkv {

// dkv_bwd with the workspace `ws`; with `pageable`, the work lists are copied from
// pageable host memory (a copy HIP performs synchronously) instead of the pinned staging
// pool, so the call allocates nothing.
dkv_status bwd_call(const dkv_params *p, const void *q_resp, const void *k_p, const void *v_p,
                    const void *k_r, const void *v_r, const void *o_r, const float *lse_r,
                    const void *dout_r, void *dq_r, void *dk_r, void *dv_r, float *acc_dk_p,
                    float *acc_dv_p, int acc_flags, void *dk_p, void *dv_p, void *ws,
                    size_t ws_bytes, hipStream_t stream, bool pageable);

// Records `msg` as this host thread's dkv_last_error() and returns `st`.
dkv_status report(dkv_status st, const char *msg);

}  // namespace dkv
