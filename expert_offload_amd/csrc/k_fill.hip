// Cache fill: copy the planned experts from the pinned host pool into their
// device slots with a kernel that reads the pool over PCIe (zero-copy).
//
// zhichai.net article, section 2, Decode paragraph: q* of a step's misses are
// brought over PCIe into the device cache. The plan (fill list and slots) is
// read from device memory, so the copy is queued behind the plan kernel on the
// same stream with no round trip through the host; 64 workgroups already keep
// enough 16-byte reads in flight to saturate the link, leaving the other CUs
// free.
#include <hip/hip_ext.h>

#include "eo_internal.h"
#include "fill_dev.h"

namespace eo {

namespace {

__global__ __launch_bounds__(256) void k_fill(const DevPlan* __restrict__ plan,
                                              const uint8_t* __restrict__ pool,
                                              uint8_t* __restrict__ slots, uint64_t S,
                                              uint64_t S_pad) {
    if (plan->pad != 0) return;  // rejected lookup: nothing to fill
    const int q = plan->q_fill;
    for (int r = 0; r < q; ++r)
        copy_block(pool + (uint64_t)plan->fill_e[r] * S_pad,
                   slots + (uint64_t)plan->fill_slot[r] * S_pad, S, blockIdx.x, gridDim.x);
}

// One expert, the fill kernel's way (the B_P probe).
__global__ __launch_bounds__(256) void k_copy_expert(const uint8_t* __restrict__ src,
                                                     uint8_t* __restrict__ dst, uint64_t S) {
    copy_block(src, dst, S, blockIdx.x, gridDim.x);
}

}  // namespace

hipError_t launch_fill(const DevPlan* plan, const uint8_t* pool_layer_dev, uint8_t* slots,
                       uint64_t S, uint64_t S_pad, hipStream_t s, hipEvent_t ev_start,
                       hipEvent_t ev_stop) {
    hipExtLaunchKernelGGL(k_fill, dim3(kFillBlocks), dim3(256), 0, s, ev_start, ev_stop, 0, plan,
                          pool_layer_dev, slots, S, S_pad);
    return hipGetLastError();
}

hipError_t launch_copy_expert(const uint8_t* src_dev, uint8_t* dst, uint64_t S, hipStream_t s) {
    k_copy_expert<<<kFillBlocks, 256, 0, s>>>(src_dev, dst, S);
    return hipGetLastError();
}

}  // namespace eo
