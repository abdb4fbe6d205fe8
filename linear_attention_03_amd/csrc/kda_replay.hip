// Commit by replay: the verify kernel in replay mode (the accepted path's
// state written to the pool slot), then the conv-state roll by the commit
// kernel with no snapshot to copy.  The kernel is in kda_verify_kernel.h.

#include "kda_verify_kernel.h"

namespace kda {

hipError_t launch_commit_replay(const kda_verify_args& a, const int32_t* accepted, hipStream_t s) {
    VerifyParams p = make_verify_params(a);
    p.snaps = nullptr;
    p.o = nullptr;
    p.accepted = accepted;
    p.pool_w = const_cast<float*>(a.state_pool);   // this entry point owns the pool for writing
    hipError_t e = launch_mode<kModeReplay>(a, p, s);
    if (e != hipSuccess) return e;
    kda_commit_args c{};
    c.struct_size = sizeof(c);
    c.dtype = a.dtype;
    c.B = a.B; c.N = a.N; c.HV = a.HV; c.K = a.K; c.V = a.V;
    c.conv_dim = 2 * a.H * a.K + a.HV * a.V;
    c.conv_width = a.conv_width;
    c.accepted = accepted; c.parents = a.parents;
    c.state_pool = p.pool_w; c.num_slots = a.num_slots; c.state_indices = a.state_indices;
    c.conv_state = const_cast<void*>(a.conv_state);
    c.num_conv_slots = a.num_conv_slots; c.conv_state_indices = a.conv_state_indices;
    c.mixed_qkv = a.mixed_qkv; c.mixed_stride = a.mixed_stride;
    return launch_commit(c, s);
}

}  // namespace kda
