// launch.hpp -- host launchers of the gfx950 kernels (one per kernel family).
#pragma once

#include <hip/hip_runtime_api.h>

#include "plan.hpp"

namespace atom {

// Per-device SNAC workspace: the staging ring, the per-slot flags, the task
// ticket and the error word. Owned by the library, allocated on first use.
struct Workspace {
    char* ring = nullptr;
    int64_t ring_bytes = 0;
    unsigned long long* counts = nullptr;  // kMaxSlots slot counts, kFlagStride apart
    unsigned long long* tags = nullptr;    // tagged ring of small calls, kTagBytes
    unsigned int* ticket = nullptr;
    unsigned int* error = nullptr;         // last timed-out call's sequence number
    unsigned int* done = nullptr;
    int wall_khz = 0;                      // rate of the device's constant clock
    uint32_t seq = 0;                      // sequence number of the last staged call
};

constexpr int kMaxDevices = 64;

// The fixed workspace of atom_collective_noalloc on the current device: the
// library's static device array, its address looked up once per device. The
// first call on a device enqueues a kernel on `stream` that clears the flags.
// Returns ATOM_OK, ATOM_ERR_UNSUPPORTED (device index out of range) or
// ATOM_ERR_HIP (*hip_err set).
atom_status static_workspace(hipStream_t stream, Workspace** out, hipError_t* hip_err);
// This device's fixed-workspace error word, or NULL before its first use.
unsigned int* static_error_word(int dev);

hipError_t launch_reduce(const Plan& p, hipStream_t stream);
hipError_t launch_copy(const Plan& p, hipStream_t stream);
// seq: the call's sequence number (nonzero), recorded in the error word if
// one of its waits times out.
hipError_t launch_snac(const Plan& p, const Workspace& ws, uint32_t seq, hipStream_t stream);
// Zeroes the workspace's tagged ring on `stream` (a kernel, so it may be
// captured): done when the sequence numbers wrap, so that no pair left by a
// call whose consumer gave up carries a number a later call takes.
hipError_t launch_clear_tags(const Workspace& ws, hipStream_t stream);
hipError_t launch_moe_route(const MoeRoutePlan& p, hipStream_t stream);
hipError_t launch_moe_move(const MoeMovePlan& p, bool combine, hipStream_t stream);

}  // namespace atom
