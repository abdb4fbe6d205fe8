// Target verify launches (snapshot and outputs-only modes).  The kernel and
// its launch helpers are in kda_verify_kernel.h.

#include "kda_verify_kernel.h"

namespace kda {

hipError_t launch_verify(const kda_verify_args& a, hipStream_t s) {
    const VerifyParams p = make_verify_params(a);
    return a.snapshots ? launch_mode<kModeSnap>(a, p, s) : launch_mode<kModeOut>(a, p, s);
}

}  // namespace kda
