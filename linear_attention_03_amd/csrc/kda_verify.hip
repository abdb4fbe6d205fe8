// Speculative target verify (A8 + A9): depthwise causal conv1d fused with
// the KDA recurrence over chain or tree drafts, one state snapshot per node.
//
// One block owns 32 state rows of one (request, head).  Prologue, in LDS:
//   * the conv of the q and k channels of the head and of the block's v
//     channels for every draft node: node i's window is the node itself,
//     then its ancestors, then the request's conv state (newest first);
//     SiLU; then the L2 norms and q.k of every node;
//   * exp(g) and beta of every node.
// Main loop: each state row (K/4 lanes, float4 per lane) is read once from
// the pool, every node's row state is kept in registers, node i starts from
// its parent's registers (pool row for a root), and every node's row goes
// to its snapshot with a streaming store.  The pool is never written.
// Fused conv1d + recurrence in one launch as in "[KDA] Default GLM-5-Next
// spec verify to the CuTe DSL KDA kernel" (Summary); chain / tree drafts
// with per-candidate snapshots as in "[KDA] Support Helion MTP verification
// and harden prefill, decode" (Modifications).

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

struct VerifyParams {
    const void* mixed;
    int64_t ms;
    const void* cw;
    const void* cb;
    const void* cs;
    const int32_t* cidx;
    const int32_t* parents;
    void* o;
    int64_t os0, os1;
    const void* a;
    int64_t as0;
    const void* b;
    int64_t bs0;
    const float* A_log;
    const float* dt_bias;
    float lb;
    float scale;
    int has_alog, beta_is_raw, l2norm, act;
    int W, N, H, HV;
    int num_slots, num_snap_slots, num_conv_slots;
    const float* pool;
    const int32_t* idx;
    float* snaps;
    const int32_t* sidx;
};

constexpr int kRowsPerBlock = 32;
constexpr int kWaves = 4;

// Conv output of channel c for draft node i of request r.
template <typename TIn>
__device__ __forceinline__ float conv_node(const VerifyParams& p, const TIn* mixed_r, const TIn* cs_c,
                                           const int* s_par, int c, int i) {
    const TIn* w = static_cast<const TIn*>(p.cw) + (int64_t)c * p.W;
    float acc = p.cb ? ld(static_cast<const TIn*>(p.cb), c) : 0.0f;
    acc = fmaf(ld(w, p.W - 1), ld(mixed_r, (int64_t)i * p.ms + c), acc);
    int par = s_par[i];
    int csi = p.W - 2;
    for (int jj = p.W - 2; jj >= 0; --jj) {
        float val;
        if (par >= 0) {
            val = ld(mixed_r, (int64_t)par * p.ms + c);
            par = s_par[par];
        } else {
            val = ld(cs_c, csi);
            --csi;
        }
        acc = fmaf(ld(w, jj), val, acc);
    }
    if (p.act == KDA_ACT_SILU) acc = acc * sigmoidf(acc);
    return acc;
}

template <typename TIn, int K, int V, int NMAX>
__global__ __launch_bounds__(256) void verify_kernel(const VerifyParams p) {
    constexpr int LPR = K / 4;
    constexpr int RPI = 64 / LPR;
    constexpr int RPW = kRowsPerBlock / kWaves;
    constexpr int IT = RPW / RPI;
    constexpr int NRB = V / kRowsPerBlock;
    static_assert(IT >= 1 && RPW % RPI == 0, "row tiling");

    __shared__ float s_q[NMAX][K];
    __shared__ float s_k[NMAX][K];
    __shared__ float s_eg[NMAX][K];
    __shared__ float s_v[NMAX][kRowsPerBlock];
    __shared__ float s_o[NMAX][kRowsPerBlock];
    __shared__ float s_beta[NMAX], s_qk[NMAX], s_rq[NMAX], s_rk[NMAX];
    __shared__ int s_par[NMAX];

    const int blk = blockIdx.x;
    const int rb = blk % NRB;
    const int bh = blk / NRB;
    const int h = bh % p.HV;
    const int r = bh / p.HV;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int N = p.N;
    const int64_t conv_dim = 2 * (int64_t)p.H * K + (int64_t)p.HV * V;

    TIn* o = static_cast<TIn*>(p.o);
    const int slot = p.idx[r];
    const int sslot = p.sidx ? p.sidx[r] : r;
    const int cslot = p.cidx ? p.cidx[r] : slot;
    if (slot < 0 || slot >= p.num_slots || sslot < 0 || sslot >= p.num_snap_slots || cslot < 0 ||
        cslot >= p.num_conv_slots) {                 // padded request (or an index out of range)
        for (int t = tid; t < N * kRowsPerBlock; t += 256) {
            const int i = t / kRowsPerBlock, rr = t % kRowsPerBlock;
            o[((int64_t)r * N + i) * p.os0 + h * p.os1 + rb * kRowsPerBlock + rr] = from_f32<TIn>(0.0f);
        }
        return;
    }

    if (tid < N) {
        // a parent outside [-1, i) is treated as a root, so no walk leaves the draft
        const int par = p.parents ? p.parents[r * N + tid] : tid - 1;
        s_par[tid] = (par >= -1 && par < tid) ? par : -1;
    }
    lds_barrier();

    const TIn* mixed_r = static_cast<const TIn*>(p.mixed) + (int64_t)r * N * p.ms;
    const TIn* cs_base = static_cast<const TIn*>(p.cs) + (int64_t)cslot * conv_dim * (p.W - 1);

    // conv of the head's q and k channels, all nodes
    for (int t = tid; t < 2 * K; t += 256) {
        const int c = t < K ? h * K + t : p.H * K + h * K + (t - K);
        const TIn* cs_c = cs_base + (int64_t)c * (p.W - 1);
        for (int i = 0; i < N; ++i) {
            const float y = conv_node(p, mixed_r, cs_c, s_par, c, i);
            if (t < K) s_q[i][t] = y; else s_k[i][t - K] = y;
        }
    }
    // conv of this block's v channels
    for (int t = tid; t < N * kRowsPerBlock; t += 256) {
        const int i = t / kRowsPerBlock, rr = t % kRowsPerBlock;
        const int c = 2 * p.H * K + h * V + rb * kRowsPerBlock + rr;
        s_v[i][rr] = conv_node(p, mixed_r, cs_base + (int64_t)c * (p.W - 1), s_par, c, i);
    }
    // gate and beta
    const bool has_alog = p.has_alog;
    const float expA = has_alog ? __expf(p.A_log[h]) : 0.0f;
    for (int t = tid; t < N * K; t += 256) {
        const int i = t / K, kk = t % K;
        const float raw = ld(static_cast<const TIn*>(p.a), ((int64_t)r * N + i) * p.as0 + h * K + kk);
        const float dt = p.dt_bias ? p.dt_bias[h * K + kk] : 0.0f;
        s_eg[i][kk] = gate_decay(raw, has_alog, expA, dt, p.lb);
    }
    if (tid < N) {
        float bt = ld(static_cast<const TIn*>(p.b), ((int64_t)r * N + tid) * p.bs0 + h);
        s_beta[tid] = p.beta_is_raw ? sigmoidf(bt) : bt;
    }
    lds_barrier();

    // L2 norms and q.k per node
    for (int i = wave; i < N; i += kWaves) {
        float sq = 0.f, sk = 0.f, sqk = 0.f;
        for (int kk = lane; kk < K; kk += 64) {
            const float qv = s_q[i][kk], kv = s_k[i][kk];
            sq += qv * qv; sk += kv * kv; sqk += qv * kv;
        }
        sq = group_sum<64>(sq); sk = group_sum<64>(sk); sqk = group_sum<64>(sqk);
        if (lane == 0) {
            const float rq = p.l2norm ? rsqrtf(sq + kL2Eps) : 1.0f;
            const float rk = p.l2norm ? rsqrtf(sk + kL2Eps) : 1.0f;
            s_rq[i] = rq; s_rk[i] = rk; s_qk[i] = sqk * rq * rk;
        }
    }
    lds_barrier();

    const int j = lane % LPR;
    const int rs = lane / LPR;
    const int rloc0 = wave * RPW + rs;
    const float* S = p.pool + ((int64_t)slot * p.HV + h) * (int64_t)V * K;
    float* snap0 = p.snaps + ((int64_t)sslot * N * p.HV + h) * (int64_t)V * K;
    const int64_t node_stride = (int64_t)p.HV * V * K;

    float4 x0[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it)
        x0[it] = ld4(S, (int64_t)(rb * kRowsPerBlock + rloc0 + it * RPI) * K + 4 * j);

#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int rloc = rloc0 + it * RPI;
        const int row = rb * kRowsPerBlock + rloc;
        float4 xs[NMAX];
#pragma unroll
        for (int i = 0; i < NMAX; ++i) {
            if (i < N) {
            const int pi = s_par[i];
            float4 xp = x0[it];
#pragma unroll
            for (int jn = 0; jn < NMAX - 1; ++jn)
                if (jn < i && pi == jn) xp = xs[jn];
            const float rk = s_rk[i], rq = s_rq[i];
            const float4 kv = f4scale(*reinterpret_cast<const float4*>(&s_k[i][4 * j]), rk);
            const float4 qv = f4scale(*reinterpret_cast<const float4*>(&s_q[i][4 * j]), rq);
            const float4 eg = *reinterpret_cast<const float4*>(&s_eg[i][4 * j]);
            const float4 xd = f4mul(eg, xp);
            float kx = fdot4(kv, xd), qx = fdot4(qv, xd);
#pragma unroll
            for (int m = LPR / 2; m >= 1; m >>= 1) {
                kx += __shfl_xor(kx, m, 64);
                qx += __shfl_xor(qx, m, 64);
            }
            const float d = s_beta[i] * (s_v[i][rloc] - kx);
            xs[i] = f4fma(kv, d, xd);
            st4_nt(snap0 + i * node_stride + (int64_t)row * K + 4 * j, xs[i]);
            if (j == 0) s_o[i][rloc] = p.scale * (qx + d * s_qk[i]);
            }
        }
    }
    lds_barrier();
    for (int t = tid; t < N * kRowsPerBlock; t += 256) {
        const int i = t / kRowsPerBlock, rr = t % kRowsPerBlock;
        o[((int64_t)r * N + i) * p.os0 + h * p.os1 + rb * kRowsPerBlock + rr] = from_f32<TIn>(s_o[i][rr]);
    }
}

template <typename TIn, int K, int V, int NMAX>
hipError_t launch_kvn(const kda_verify_args& a, const VerifyParams& p, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(a.B * a.HV * (V / kRowsPerBlock)));
    hipLaunchKernelGGL((verify_kernel<TIn, K, V, NMAX>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

template <typename TIn, int K, int V>
hipError_t launch_kv(const kda_verify_args& a, const VerifyParams& p, hipStream_t s) {
    return a.N <= 8 ? launch_kvn<TIn, K, V, 8>(a, p, s) : launch_kvn<TIn, K, V, 16>(a, p, s);
}

template <typename TIn, int K>
hipError_t launch_k(const kda_verify_args& a, const VerifyParams& p, hipStream_t s) {
    switch (a.V) {
        case 32: return launch_kv<TIn, K, 32>(a, p, s);
        case 64: return launch_kv<TIn, K, 64>(a, p, s);
        default: return launch_kv<TIn, K, 128>(a, p, s);
    }
}

template <typename TIn>
hipError_t launch_t(const kda_verify_args& a, const VerifyParams& p, hipStream_t s) {
    switch (a.K) {
        case 32: return launch_k<TIn, 32>(a, p, s);
        case 64: return launch_k<TIn, 64>(a, p, s);
        default: return launch_k<TIn, 128>(a, p, s);
    }
}

}  // namespace

hipError_t launch_verify(const kda_verify_args& a, hipStream_t s) {
    VerifyParams p;
    p.mixed = a.mixed_qkv; p.ms = a.mixed_stride;
    p.cw = a.conv_weight; p.cb = a.conv_bias; p.cs = a.conv_state; p.cidx = a.conv_state_indices;
    p.parents = a.parents;
    p.o = a.o; p.os0 = a.o_stride[0]; p.os1 = a.o_stride[1];
    p.a = a.a; p.as0 = a.a_stride; p.b = a.b; p.bs0 = a.b_stride;
    p.A_log = a.A_log; p.dt_bias = a.dt_bias; p.lb = a.lower_bound; p.scale = a.scale;
    p.has_alog = a.A_log != nullptr; p.beta_is_raw = a.beta_is_raw; p.l2norm = a.use_qk_l2norm;
    p.act = a.conv_activation;
    p.W = static_cast<int>(a.conv_width); p.N = static_cast<int>(a.N);
    p.H = static_cast<int>(a.H); p.HV = static_cast<int>(a.HV);
    p.num_slots = static_cast<int>(a.num_slots);
    p.num_snap_slots = static_cast<int>(a.num_snapshot_slots);
    p.num_conv_slots = static_cast<int>(a.num_conv_slots);
    p.pool = a.state_pool; p.idx = a.state_indices;
    p.snaps = a.snapshots; p.sidx = a.snapshot_indices;
    return a.dtype == KDA_BF16 ? launch_t<bf16>(a, p, s) : launch_t<float>(a, p, s);
}

}  // namespace kda
