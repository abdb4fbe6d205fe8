// Internal interface between the host entry points (kda_api.cpp) and the
// kernel launchers (*.hip).  Arguments reaching a launcher have passed the
// host-side validation in kda_api.cpp.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "../../include/kda.h"

namespace kda {

// Timing events of the next call on this thread (kda_set_call_events): the
// call's first kernel records `start` as it begins and every kernel records
// `stop` as it ends, so the last one leaves the call's end.  The events are
// stamped by the dispatches themselves (hipExtLaunchKernel), so the interval
// holds no launch gap before the first kernel or after the last.
struct CallEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
CallEvents& call_events();

// Every kernel launch of the library goes through here.
template <typename... P, typename... A>
inline void klaunch(void (*kernel)(P...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, A&&... args) {
    CallEvents& ev = call_events();
    if (ev.start == nullptr && ev.stop == nullptr) {
        kernel<<<grid, block, shmem, s>>>(static_cast<A&&>(args)...);
        return;
    }
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, ev.start, ev.stop, 0, static_cast<A&&>(args)...);
    ev.start = nullptr;
}

hipError_t launch_decode(const kda_decode_args& a, hipStream_t stream);
hipError_t launch_decode_conv(const kda_decode_conv_args& a, hipStream_t stream);
hipError_t launch_verify(const kda_verify_args& a, hipStream_t stream);
// Outputs-only verify (no snapshots) on fp32 matrix tiles.
hipError_t launch_verify_outputs(const kda_verify_args& a, hipStream_t stream);
hipError_t launch_commit(const kda_commit_args& a, hipStream_t stream);
hipError_t launch_conv_update(const kda_conv_update_args& a, hipStream_t stream);
// Replay-mode verify launch writing the pool, then the conv-state roll.
hipError_t launch_commit_replay(const kda_verify_args& a, const int32_t* accepted, hipStream_t stream);

// Prefill: upper bound on the number of chunks the call can produce
// (B * ceil(T / C) fixed, floor(T / C) + num_seqs packed).
int64_t prefill_max_chunks(const kda_prefill_args& a);
size_t prefill_workspace_bytes(const kda_prefill_args& a);
bool prefill_mfma_eligible(const kda_prefill_args& a);    // the matrix-core path takes the call
hipError_t launch_prefill(const kda_prefill_args& a, void* workspace, hipStream_t stream);

// Device address of the built-in scratch (KDA_NOALLOC_SCRATCH_BYTES) on the
// current device, looked up on the first request per device.
hipError_t noalloc_scratch(void** ptr);

}  // namespace kda
