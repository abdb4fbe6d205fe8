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
// to its snapshot with a streaming store (skipped when no snapshot buffer
// is given).  The pool is never written.
//
// Replay mode (commit without snapshots): the same prologue, then each
// state row walks only the nodes on the path root .. accepted node and the
// result is stored back to the request's pool slot.  Every node runs the
// same instruction sequence as in the verify launch, so the committed state
// equals the accepted node's snapshot bit for bit.  The conv-state roll is
// a second launch (commit kernel, conv part only), since the q and k
// channels of a head are read by every row block of that head.
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
    int gate, beta_is_raw, l2norm, act;
    int W, N, H, HV;
    int group;                 // HV / H: value heads per q/k head
    int num_slots, num_snap_slots, num_conv_slots;
    const float* pool;
    const int32_t* idx;
    float* snaps;
    const int32_t* sidx;
    const int32_t* accepted;   // replay mode
    float* pool_w;             // replay mode: the pool, written in place
};

constexpr int kRowsPerBlock = 32;
constexpr int kWaves = 4;
constexpr int kMaxWidth = 4;

// CHAIN: parents == NULL (node i extends node i - 1), so the recurrence
// needs only the previous node's row; otherwise every node's row is kept.
// REPLAY: commit by replaying the accepted path (see the file comment).
template <typename TIn, int K, int V, int NMAX, bool CHAIN, bool REPLAY>
__global__ __launch_bounds__(256) void verify_kernel(const VerifyParams p) {
    // A state row is held by LPR lanes, NV float4 per lane (element offsets
    // 4j and, for NV = 2, K/2 + 4j): 8 elements per lane for K >= 64, so a
    // row's dot products need log2(LPR) lane-exchange steps per 8 elements.
    constexpr int NV = K >= 64 ? 2 : 1;
    constexpr int LPR = K / (4 * NV);
    constexpr int RPI = 64 / LPR;                    // rows per wave instruction
    constexpr int RPW = kRowsPerBlock / kWaves;
    constexpr int IT = RPW / RPI;
    constexpr int NRB = V / kRowsPerBlock;
    constexpr int CH = 2 * K + kRowsPerBlock;        // conv channels of one block
    constexpr int NCS = (CH + 255) / 256;
    constexpr int NG = (NMAX * K + 255) / 256;       // gate elements per thread
    constexpr int HALF = K / NV;
    static_assert(IT >= 1 && RPW % RPI == 0, "row tiling");

    __shared__ float s_q[NMAX][K];
    __shared__ float s_k[NMAX][K];
    __shared__ float s_eg[NMAX][K];
    __shared__ float s_v[NMAX][kRowsPerBlock];
    __shared__ float s_o[NMAX][kRowsPerBlock];
    __shared__ float s_beta[NMAX], s_rq[NMAX], s_rk[NMAX], s_qk[NMAX];
    __shared__ TIn s_in[NMAX + kMaxWidth - 1][CH];   // per channel: node inputs, then conv state by age
    __shared__ int s_par[kWaves][NMAX];               // one copy per wave

    const int blk = blockIdx.x;
    const int rb = blk % NRB;
    const int bh = blk / NRB;
    const int h = bh % p.HV;
    const int r = bh / p.HV;
    const int hq = h / p.group;                      // q/k head of this value head
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int N = p.N;
    const int W = p.W;
    const int64_t conv_dim = 2 * (int64_t)p.H * K + (int64_t)p.HV * V;

    TIn* o = static_cast<TIn*>(p.o);
    const int slot = p.idx[r];
    const int sslot = p.sidx ? p.sidx[r] : r;
    const int cslot = p.cidx ? p.cidx[r] : slot;
    const bool bad_snap = p.snaps != nullptr && (sslot < 0 || sslot >= p.num_snap_slots);
    if (REPLAY) {
        const int acc = p.accepted[r];
        // nothing accepted, or a padded request: the slot stays as it is
        if (acc < 0 || acc >= N || slot < 0 || slot >= p.num_slots || cslot < 0 || cslot >= p.num_conv_slots)
            return;
    } else if (slot < 0 || slot >= p.num_slots || bad_snap || cslot < 0 ||
               cslot >= p.num_conv_slots) {          // padded request (or an index out of range)
        for (int t = tid; t < N * kRowsPerBlock; t += 256) {
            const int i = t / kRowsPerBlock, rr = t % kRowsPerBlock;
            o[((int64_t)r * N + i) * p.os0 + h * p.os1 + rb * kRowsPerBlock + rr] = from_f32<TIn>(0.0f);
        }
        return;
    }

    // ---- every global load of the block is issued here, before any use ----
    const int j = lane % LPR;
    const int rs = lane / LPR;
    const int rloc0 = wave * RPW + rs;
    const float* S = p.pool + ((int64_t)slot * p.HV + h) * (int64_t)V * K;
    float4 x0[IT][NV];
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int u = 0; u < NV; ++u)
            x0[it][u] = ld4(S, (int64_t)(rb * kRowsPerBlock + rloc0 + it * RPI) * K + u * HALF + 4 * j);

    // parents; a parent outside [-1, i) is treated as a root, so no walk
    // leaves the draft.  Kept per lane (for the per-wave LDS copy) and as
    // block-uniform values (for the recurrence).
    int par[NMAX];
#pragma unroll
    for (int i = 0; i < NMAX; ++i) {
        int pi = CHAIN ? i - 1 : p.parents[(int64_t)r * N + min(i, N - 1)];
        par[i] = (i < N && pi >= -1 && pi < i) ? pi : -1;
    }
    const int lpar_raw = CHAIN ? lane - 1 : p.parents[(int64_t)r * N + min(lane, N - 1)];

    // conv inputs: this thread's channels at every node, the conv state and
    // the weights, both by age (age 0 = the node itself; conv-state age 1 is
    // its newest entry)
    const TIn* mixed_r = static_cast<const TIn*>(p.mixed) + (int64_t)r * N * p.ms;
    const TIn* cs_base = static_cast<const TIn*>(p.cs) + (int64_t)cslot * conv_dim * (W - 1);
    const TIn* cw = static_cast<const TIn*>(p.cw);
    TIn raw[NCS][NMAX], cs_age[NCS][kMaxWidth - 1];
    float w_age[NCS][kMaxWidth], bias[NCS];
#pragma unroll
    for (int sl = 0; sl < NCS; ++sl) {
        const int cc = min(tid + 256 * sl, CH - 1);
        const int64_t c = cc < K ? (int64_t)hq * K + cc
                        : cc < 2 * K ? (int64_t)p.H * K + hq * K + (cc - K)
                        : 2 * (int64_t)p.H * K + h * V + rb * kRowsPerBlock + (cc - 2 * K);
#pragma unroll
        for (int i = 0; i < NMAX; ++i) raw[sl][i] = mixed_r[(int64_t)min(i, N - 1) * p.ms + c];
#pragma unroll
        for (int m = 0; m < kMaxWidth - 1; ++m) cs_age[sl][m] = cs_base[c * (W - 1) + max(W - 2 - m, 0)];
#pragma unroll
        for (int m = 0; m < kMaxWidth; ++m) w_age[sl][m] = ld(cw, c * W + max(W - 1 - m, 0));
        bias[sl] = p.cb ? ld(static_cast<const TIn*>(p.cb), c) : 0.0f;
    }

    // gate and beta inputs
    float graw[NG], gdt[NG];
#pragma unroll
    for (int u = 0; u < NG; ++u) {
        const int t = tid + 256 * u;
        const int i = min(t / K, N - 1), kk = t % K;
        graw[u] = ld(static_cast<const TIn*>(p.a), ((int64_t)r * N + i) * p.as0 + h * K + kk);
        gdt[u] = p.dt_bias ? p.dt_bias[h * K + kk] : 0.0f;
    }
    const float braw = ld(static_cast<const TIn*>(p.b), ((int64_t)r * N + min(tid, N - 1)) * p.bs0 + h);
    const int gmode = p.gate;
    const float expA = gmode != kGateRaw ? __expf(p.A_log[h]) : 0.0f;

    // ---- conv + SiLU per channel and node, walking the ancestor path ----
    if (lane < N) s_par[wave][lane] = (lpar_raw >= -1 && lpar_raw < lane) ? lpar_raw : -1;
#pragma unroll
    for (int sl = 0; sl < NCS; ++sl) {
        const int cc = tid + 256 * sl;
        if (cc < CH) {
#pragma unroll
            for (int i = 0; i < NMAX; ++i) s_in[i][cc] = raw[sl][i];
#pragma unroll
            for (int m = 0; m < kMaxWidth - 1; ++m) s_in[NMAX + m][cc] = cs_age[sl][m];
        }
    }
    // (each thread reads back only its own columns, and its wave's parent
    // copy: LDS operations of one wave complete in order, no barrier needed)
#pragma unroll
    for (int sl = 0; sl < NCS; ++sl) {
        const int cc = tid + 256 * sl;
        if (cc < CH) {
#pragma unroll
            for (int i = 0; i < NMAX; ++i) {
                if (i < N) {
                    float acc = fmaf(w_age[sl][0], to_f32(raw[sl][i]), bias[sl]);
                    int a = par[i], row_cs = NMAX;
#pragma unroll
                    for (int m = 1; m < kMaxWidth; ++m) {
                        if (m < W) {
                            int src;
                            if (a >= 0) {
                                src = a;
                                a = CHAIN ? a - 1 : s_par[wave][a];
                            } else {
                                src = row_cs++;
                            }
                            acc = fmaf(w_age[sl][m], to_f32(s_in[src][cc]), acc);
                        }
                    }
                    if (p.act == KDA_ACT_SILU) acc = acc * sigmoidf(acc);
                    if (cc < K) s_q[i][cc] = acc;
                    else if (cc < 2 * K) s_k[i][cc - K] = acc;
                    else s_v[i][cc - 2 * K] = acc;
                }
            }
        }
    }
#pragma unroll
    for (int u = 0; u < NG; ++u) {
        const int t = tid + 256 * u;
        if (t < N * K) s_eg[t / K][t % K] = gate_decay(graw[u], gmode, expA, gdt[u], p.lb);
    }
    if (tid < N) s_beta[tid] = p.beta_is_raw ? sigmoidf(braw) : braw;
    lds_barrier();

    // ---- per-node L2 norms and q.k: wave w takes nodes w, w + 4, ... ----
    for (int i = wave; i < N; i += kWaves) {
        float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
        for (int kk = lane; kk < K; kk += 64) {
            const float qv = s_q[i][kk], kv = s_k[i][kk];
            sq = fmaf(qv, qv, sq);
            sk = fmaf(kv, kv, sk);
            sqk = fmaf(qv, kv, sqk);
        }
        if (K >= 64) {
            sq = wave_sum(sq); sk = wave_sum(sk); sqk = wave_sum(sqk);
        } else {
            sq = lane_sum<32>(sq); sk = lane_sum<32>(sk); sqk = lane_sum<32>(sqk);
        }
        if (lane == 0) {
            const float rq = p.l2norm ? rsqrtf(sq + kL2Eps) : 1.0f;
            const float rk = p.l2norm ? rsqrtf(sk + kL2Eps) : 1.0f;
            s_rq[i] = rq; s_rk[i] = rk; s_qk[i] = sqk * rq * rk;
        }
    }
    lds_barrier();

    if (REPLAY) {
        // The path root .. accepted node as a bit mask over node indices.
        // Every parent has a smaller index than its child, so walking the
        // indices downwards meets each ancestor in turn, and taking the
        // set bits upwards visits the path root first.
        unsigned path = 0;
        int a = p.accepted[r];
#pragma unroll
        for (int i = NMAX - 1; i >= 0; --i)
            if (i == a) { path |= 1u << i; a = par[i]; }
        float* dst = p.pool_w + ((int64_t)slot * p.HV + h) * (int64_t)V * K;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int rloc = rloc0 + it * RPI;
            const int row = rb * kRowsPerBlock + rloc;
            float4 x[NV];
#pragma unroll
            for (int u = 0; u < NV; ++u) x[u] = x0[it][u];
#pragma unroll
            for (int i = 0; i < NMAX; ++i) {
                if (i < N && ((path >> i) & 1u)) {
                    const float rk = s_rk[i];
                    float4 kv[NV], xd[NV];
                    float kx = 0.f;
#pragma unroll
                    for (int u = 0; u < NV; ++u) {
                        kv[u] = *reinterpret_cast<const float4*>(&s_k[i][u * HALF + 4 * j]);
                        const float4 eg = *reinterpret_cast<const float4*>(&s_eg[i][u * HALF + 4 * j]);
                        xd[u] = f4mul(eg, x[u]);
                        kx += fdot4(kv[u], xd[u]);
                    }
                    kx = lane_sum<LPR>(kx) * rk;
                    const float d = s_beta[i] * (s_v[i][rloc] - kx);
                    const float dk = d * rk;
#pragma unroll
                    for (int u = 0; u < NV; ++u) x[u] = f4fma(kv[u], dk, xd[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < NV; ++u) st4(dst + (int64_t)row * K + u * HALF + 4 * j, x[u]);
        }
        return;
    }

    // ---- recurrence over the draft nodes, one row group at a time ----
    // The norms enter as scalars: k.x_d = rk (k_raw . x_d), and the update
    // x = x_d + d rk k_raw.
    const bool snap = p.snaps != nullptr;
    float* snap0 = snap ? p.snaps + ((int64_t)sslot * N * p.HV + h) * (int64_t)V * K : nullptr;
    const int64_t node_stride = (int64_t)p.HV * V * K;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int rloc = rloc0 + it * RPI;
        const int row = rb * kRowsPerBlock + rloc;
        float* snap_row = snap0 + (int64_t)row * K + 4 * j;
        float4 xs[CHAIN ? 1 : NMAX][NV];
#pragma unroll
        for (int i = 0; i < NMAX; ++i) {
            if (i < N) {
                float4 xp[NV];
#pragma unroll
                for (int u = 0; u < NV; ++u) {
                    if (CHAIN) {
                        xp[u] = i == 0 ? x0[it][u] : xs[0][u];
                    } else {
                        const int pi = par[i];
                        xp[u] = x0[it][u];
#pragma unroll
                        for (int jn = 0; jn < NMAX - 1; ++jn)
                            if (jn < i && pi == jn) xp[u] = xs[jn][u];
                    }
                }
                const float rk = s_rk[i], rq = s_rq[i];
                float4 kv[NV], xd[NV];
                float kx = 0.f, qx = 0.f;
#pragma unroll
                for (int u = 0; u < NV; ++u) {
                    kv[u] = *reinterpret_cast<const float4*>(&s_k[i][u * HALF + 4 * j]);
                    const float4 qv = *reinterpret_cast<const float4*>(&s_q[i][u * HALF + 4 * j]);
                    const float4 eg = *reinterpret_cast<const float4*>(&s_eg[i][u * HALF + 4 * j]);
                    xd[u] = f4mul(eg, xp[u]);
                    kx += fdot4(kv[u], xd[u]);
                    qx += fdot4(qv, xd[u]);
                }
                kx = lane_sum<LPR>(kx) * rk;
                qx = lane_sum<LPR>(qx) * rq;
                const float d = s_beta[i] * (s_v[i][rloc] - kx);
                const float dk = d * rk;
#pragma unroll
                for (int u = 0; u < NV; ++u) {
                    const float4 xn = f4fma(kv[u], dk, xd[u]);
                    xs[CHAIN ? 0 : i][u] = xn;
                    if (snap) st4_nt(snap_row + i * node_stride + u * HALF, xn);
                }
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
    const bool replay = p.accepted != nullptr;
    if (p.parents) {
        if (replay) hipLaunchKernelGGL((verify_kernel<TIn, K, V, NMAX, false, true>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((verify_kernel<TIn, K, V, NMAX, false, false>), grid, dim3(256), 0, s, p);
    } else {
        if (replay) hipLaunchKernelGGL((verify_kernel<TIn, K, V, NMAX, true, true>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((verify_kernel<TIn, K, V, NMAX, true, false>), grid, dim3(256), 0, s, p);
    }
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

VerifyParams make_params(const kda_verify_args& a) {
    VerifyParams p;
    p.mixed = a.mixed_qkv; p.ms = a.mixed_stride;
    p.cw = a.conv_weight; p.cb = a.conv_bias; p.cs = a.conv_state; p.cidx = a.conv_state_indices;
    p.parents = a.parents;
    p.o = a.o; p.os0 = a.o_stride[0]; p.os1 = a.o_stride[1];
    p.a = a.a; p.as0 = a.a_stride; p.b = a.b; p.bs0 = a.b_stride;
    p.A_log = a.A_log; p.dt_bias = a.dt_bias; p.lb = a.lower_bound; p.scale = a.scale;
    p.gate = gate_mode(a.A_log, a.has_lower_bound); p.beta_is_raw = a.beta_is_raw; p.l2norm = a.use_qk_l2norm;
    p.group = static_cast<int>(a.HV / a.H);
    p.act = a.conv_activation;
    p.W = static_cast<int>(a.conv_width); p.N = static_cast<int>(a.N);
    p.H = static_cast<int>(a.H); p.HV = static_cast<int>(a.HV);
    p.num_slots = static_cast<int>(a.num_slots);
    p.num_snap_slots = static_cast<int>(a.num_snapshot_slots);
    p.num_conv_slots = static_cast<int>(a.num_conv_slots);
    p.pool = a.state_pool; p.idx = a.state_indices;
    p.snaps = a.snapshots; p.sidx = a.snapshot_indices;
    p.accepted = nullptr; p.pool_w = nullptr;
    return p;
}

}  // namespace

hipError_t launch_verify(const kda_verify_args& a, hipStream_t s) {
    const VerifyParams p = make_params(a);
    return a.dtype == KDA_BF16 ? launch_t<bf16>(a, p, s) : launch_t<float>(a, p, s);
}

hipError_t launch_commit_replay(const kda_verify_args& a, const int32_t* accepted, hipStream_t s) {
    VerifyParams p = make_params(a);
    p.snaps = nullptr;
    p.o = nullptr;
    p.accepted = accepted;
    p.pool_w = const_cast<float*>(a.state_pool);   // this entry point owns the pool for writing
    hipError_t e = a.dtype == KDA_BF16 ? launch_t<bf16>(a, p, s) : launch_t<float>(a, p, s);
    if (e != hipSuccess) return e;
    // conv-state roll: the commit kernel with no snapshot to copy
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
