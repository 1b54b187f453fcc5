// noalloc.hip -- mdcn_forward_noalloc: the forward pass with its workspace in
// a fixed device array of this library instead of a caller's buffer, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The array, `scratch`, is a file-scope __device__ variable: every GPU the
// library runs on holds its own copy (MDCN_NOALLOC_SCRATCH_BYTES) from the
// moment the library's code is loaded there until the process ends.  In host
// code its name is only a stand-in, not a device address: its address on a
// device comes from hipGetSymbolAddress, asked once per device (with that
// device current) and kept, and only that address reaches the kernels.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "entry.h"
#include "mdcn.h"

namespace {

constexpr size_t kScratchBytes = MDCN_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte blocks");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The device address of `scratch` on the current device (asked once per
// device, then cached).  MDCN_E_LAUNCH if the runtime cannot give it.
mdcn_status scratch_address(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return MDCN_E_DEVICE;
    static std::mutex mu;
    static std::map<int, void *> known;
    std::lock_guard<std::mutex> lock(mu);
    auto it = known.find(dev);
    if (it == known.end()) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return MDCN_E_LAUNCH;
        it = known.emplace(dev, ptr).first;
    }
    *out = it->second;
    return MDCN_OK;
}

}  // namespace

extern "C" mdcn_status mdcn_forward_noalloc(const mdcn_op *op, mdcn_dtype dtype,
                                            const int64_t dims[16], const void *x,
                                            const void *offset, const void *mask,
                                            const void *weight, const void *bias,
                                            int64_t bias_len, void *out, void *stream)
{
    try {
        if (!op || !dims)
            return MDCN_E_NULL;
        void *ws = nullptr;
        const mdcn_status st = scratch_address(&ws);
        if (st != MDCN_OK)
            return st;
        // The plan fits the chunk of images to the scratch it is given; a
        // problem whose smallest workspace exceeds the array is rejected
        // with MDCN_E_WORKSPACE before anything is enqueued.  Nothing here
        // allocates: the partial-sum flags and the status word the windowed
        // path uses are cleared by a kernel of the forward itself.
        return mdcn::forward_with_workspace(op, dtype, dims, x, offset, mask, weight, bias,
                                            bias_len, out, ws, kScratchBytes, stream);
    } catch (...) {
        return MDCN_E_INTERNAL;
    }
}
