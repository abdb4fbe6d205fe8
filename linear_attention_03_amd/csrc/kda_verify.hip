// Target verify launches: with snapshots, the row-recurrence kernel of
// kda_verify_kernel.h; outputs only, the matrix-tile kernel of
// kda_verify_tile.hip.

#include "kda_verify_kernel.h"

namespace kda {

hipError_t launch_verify(const kda_verify_args& a, hipStream_t s) {
    const VerifyParams p = make_verify_params(a);
    return a.snapshots ? launch_mode<kModeSnap>(a, p, s) : launch_verify_outputs(a, s);
}

}  // namespace kda
