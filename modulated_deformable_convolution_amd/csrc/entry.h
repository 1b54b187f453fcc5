// entry.h -- the forward pass behind the extern "C" entry points, for the
// entry points defined outside api.cpp.
#pragma once

#include "mdcn.h"

namespace mdcn {

// mdcn_forward's work (validation, planning, launches on `stream`) with the
// given workspace; the same contract and status codes.
mdcn_status forward_with_workspace(const mdcn_op *op, mdcn_dtype dtype, const int64_t dims[16],
                                   const void *x, const void *offset, const void *mask,
                                   const void *weight, const void *bias, int64_t bias_len,
                                   void *out, void *workspace, size_t workspace_bytes,
                                   void *stream);

}  // namespace mdcn
