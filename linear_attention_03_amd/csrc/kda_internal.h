// Internal interface between the host entry points (kda_api.cpp) and the
// kernel launchers (*.hip).  Arguments reaching a launcher have passed the
// host-side validation in kda_api.cpp.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/kda.h"

namespace kda {

hipError_t launch_decode(const kda_decode_args& a, hipStream_t stream);
hipError_t launch_verify(const kda_verify_args& a, hipStream_t stream);
hipError_t launch_commit(const kda_commit_args& a, hipStream_t stream);
hipError_t launch_conv_update(const kda_conv_update_args& a, hipStream_t stream);
// Replay-mode verify launch writing the pool, then the conv-state roll.
hipError_t launch_commit_replay(const kda_verify_args& a, const int32_t* accepted, hipStream_t stream);

// Prefill: upper bound on the number of chunks the call can produce
// (B * ceil(T / C) fixed, floor(T / C) + num_seqs packed).
int64_t prefill_max_chunks(const kda_prefill_args& a);
size_t prefill_workspace_bytes(const kda_prefill_args& a);
hipError_t launch_prefill(const kda_prefill_args& a, void* workspace, hipStream_t stream);

}  // namespace kda
