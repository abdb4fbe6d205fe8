// Commit after target verify (A10): for every request with an accepted
// node, bit-copy that node's snapshot into the request's pool slot, and
// roll the request's conv state to the last W-1 inputs of (conv state,
// tokens on the path root .. accepted node).  Blocks [0, copy_blocks) of
// grid row r copy 32 KiB each of request r's state; the remaining blocks
// roll 256 conv channels each.  Every destination element has one owner.
// Commit of a partially accepted prefix between verify rounds follows the
// review thread of "[KDA] Support Helion MTP verification and harden
// prefill, decode".

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

struct CommitParams {
    const int32_t* accepted;
    const int32_t* parents;
    const float* snaps;
    const int32_t* sidx;
    float* pool;
    const int32_t* idx;
    void* cs;
    const int32_t* cidx;
    const void* mixed;
    int64_t ms;
    int64_t state_elems;   // HV * V * K
    int64_t conv_dim;
    int W, N;
    int num_slots, num_snap_slots, num_conv_slots;
    int copy_blocks;
};

constexpr int kCopyFloat4PerBlock = 2048;   // 32 KiB

template <typename TIn>
__global__ __launch_bounds__(256) void commit_kernel(const CommitParams p) {
    const int r = blockIdx.y;
    const int acc = p.accepted[r];
    const int slot = p.idx[r];
    if (acc < 0 || acc >= p.N || slot < 0 || slot >= p.num_slots) return;
    const int tid = threadIdx.x;

    if ((int)blockIdx.x < p.copy_blocks) {
        const int sslot = p.sidx ? p.sidx[r] : r;
        if (sslot < 0 || sslot >= p.num_snap_slots) return;
        const float4* src = reinterpret_cast<const float4*>(p.snaps + ((int64_t)sslot * p.N + acc) * p.state_elems);
        float4* dst = reinterpret_cast<float4*>(p.pool + (int64_t)slot * p.state_elems);
        const int64_t n4 = p.state_elems / 4;
        const int64_t e0 = (int64_t)blockIdx.x * kCopyFloat4PerBlock + tid;
        // all eight loads before any store (source and destination never
        // overlap, which the compiler cannot know)
        constexpr int kPer = kCopyFloat4PerBlock / 256;
        float4 v[kPer];
        if ((int64_t)(blockIdx.x + 1) * kCopyFloat4PerBlock <= n4) {
            // a whole block, branch-free: a store under a branch makes the
            // compiler wait for every earlier store before it
#pragma unroll
            for (int u = 0; u < kPer; ++u) v[u] = src[e0 + (int64_t)u * 256];
#pragma unroll
            for (int u = 0; u < kPer; ++u) dst[e0 + (int64_t)u * 256] = v[u];
            return;
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int64_t e = e0 + (int64_t)u * 256;
            v[u] = e < n4 ? src[e] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int64_t e = e0 + (int64_t)u * 256;
            if (e < n4) dst[e] = v[u];
        }
        return;
    }
    if (p.cs == nullptr) return;
    const int64_t c = (int64_t)(blockIdx.x - p.copy_blocks) * 256 + tid;
    if (c >= p.conv_dim) return;

    // path root .. acc, as row indices within the request's draft
    int path[16];
    int depth = 0;
    // parents[r, i] < i makes the walk end; a parent outside [-1, i) is
    // treated as a root, so the walk stays inside the draft
    for (int i = acc; i >= 0 && depth < 16;) {
        path[depth++] = i;
        const int par = p.parents ? p.parents[r * p.N + i] : i - 1;
        i = (par >= -1 && par < i) ? par : -1;
    }
    const int cslot = p.cidx ? p.cidx[r] : slot;
    if (cslot < 0 || cslot >= p.num_conv_slots) return;
    TIn* cs = static_cast<TIn*>(p.cs) + ((int64_t)cslot * p.conv_dim + c) * (p.W - 1);
    const TIn* mixed_r = static_cast<const TIn*>(p.mixed) + (int64_t)r * p.N * p.ms + c;

    // sequence = cs[0 .. W-2], x[path[depth-1]], ..., x[path[0]]; keep its last W-1
    TIn old[3];
    for (int j = 0; j < p.W - 1; ++j) old[j] = cs[j];
    const int total = (p.W - 1) + depth;
    for (int j = 0; j < p.W - 1; ++j) {
        const int pos = total - (p.W - 1) + j;        // index in the sequence
        TIn val;
        if (pos < p.W - 1) val = old[pos];
        else val = mixed_r[(int64_t)path[depth - 1 - (pos - (p.W - 1))] * p.ms];
        cs[j] = val;
    }
}

template <typename TIn>
hipError_t launch_t(const kda_commit_args& a, CommitParams& p, hipStream_t s) {
    const int64_t n4 = p.state_elems / 4;
    // no snapshots: conv roll only (commit by replay has written the pool)
    p.copy_blocks = p.snaps ? static_cast<int>((n4 + kCopyFloat4PerBlock - 1) / kCopyFloat4PerBlock) : 0;
    const int conv_blocks = a.conv_state ? static_cast<int>((a.conv_dim + 255) / 256) : 0;
    const dim3 grid(static_cast<unsigned>(p.copy_blocks + conv_blocks), static_cast<unsigned>(a.B));
    klaunch(commit_kernel<TIn>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_commit(const kda_commit_args& a, hipStream_t s) {
    CommitParams p;
    p.accepted = a.accepted; p.parents = a.parents;
    p.snaps = a.snapshots; p.sidx = a.snapshot_indices;
    p.pool = a.state_pool; p.idx = a.state_indices;
    p.cs = a.conv_state; p.cidx = a.conv_state_indices;
    p.mixed = a.mixed_qkv; p.ms = a.mixed_stride;
    p.state_elems = a.HV * a.V * a.K;
    p.conv_dim = a.conv_dim;
    p.W = static_cast<int>(a.conv_width); p.N = static_cast<int>(a.N);
    p.num_slots = static_cast<int>(a.num_slots);
    p.num_snap_slots = static_cast<int>(a.num_snapshot_slots);
    p.num_conv_slots = a.conv_state ? static_cast<int>(a.num_conv_slots) : 0;
    return a.dtype == KDA_BF16 ? launch_t<bf16>(a, p, s) : launch_t<float>(a, p, s);
}

}  // namespace kda
