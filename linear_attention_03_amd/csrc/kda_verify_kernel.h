// Speculative target verify kernel with snapshots (A8 + A9) and its replay
// mode, shared by the verify launcher (kda_verify.hip) and the replayed
// commit (kda_replay.hip): depthwise causal conv1d fused with the KDA
// recurrence over chain or tree drafts.  (Verify without snapshots is the
// matrix-tile kernel of kda_verify_tile.hip; it shares VerifyParams.)
//
// One block owns RB state rows of one (request, head).  Prologue, in LDS:
//   * the conv of the q and k channels of the head and of the block's v
//     channels for every draft node: node i's window is the node itself,
//     then its ancestors, then the request's conv state (newest first);
//     SiLU; then the L2 norms and q.k of every node;
//   * exp(g) and beta of every node.
// Main loop: each state row (K/4 lanes, float4 per lane) is read once from
// the pool and carried through the nodes in registers; node i starts from
// its parent's state (the pool row for a root).  Every node's row goes to
// its snapshot with a streaming store; the pool is never written.
//
// Replay mode (commit without snapshots): the same prologue, then each
// state row walks only the nodes on the path root .. accepted node and the
// result is stored back to the request's pool slot.  Every node runs the
// same arithmetic as in the verify launch, so the committed state equals
// the accepted node's snapshot bit for bit.  The conv-state roll is a
// second launch (commit kernel, conv part only), since the q and k
// channels of a head are read by every row block of that head.
// Fused conv1d + recurrence in one launch as in "[KDA] Default GLM-5-Next
// spec verify to the CuTe DSL KDA kernel" (Summary); chain / tree drafts
// with per-candidate snapshots as in "[KDA] Support Helion MTP verification
// and harden prefill, decode" (Modifications).
#pragma once

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

constexpr int kWaves = 4;
constexpr int kMaxWidth = 4;

// What a launch writes: snapshots and outputs, or (replay)
// the state after the accepted node, in place in the pool.
enum VerifyMode { kModeSnap = 0, kModeReplay = 2 };

// The row-state arithmetic of one node, shared by every loop structure so
// that a replayed node rounds exactly like the verified one.  Every product
// and sum is written out (explicit fma, fixed order): left to contraction,
// the compiler fuses a dot product's terms in an order that differs between
// instantiations.
__device__ __forceinline__ float dot4_fixed(float4 a, float4 b) {
    return fmaf(a.w, b.w, fmaf(a.z, b.z, fmaf(a.y, b.y, a.x * b.x)));
}

// x_d = e^g x, then this lane's partial k.x_d and q.x_d (summed over the
// row's lanes by the caller).
template <int NV>
__device__ __forceinline__ void node_decay_dots(const float4 (&eg)[NV], const float4 (&kv)[NV],
                                                const float4 (&qv)[NV], float4 (&x)[NV], float& kx,
                                                float& qx, bool want_q) {
#pragma unroll
    for (int u = 0; u < NV; ++u) x[u] = f4mul(eg[u], x[u]);
    kx = dot4_fixed(kv[0], x[0]);
    qx = want_q ? dot4_fixed(qv[0], x[0]) : 0.f;
#pragma unroll
    for (int u = 1; u < NV; ++u) {
        kx = kx + dot4_fixed(kv[u], x[u]);
        if (want_q) qx = qx + dot4_fixed(qv[u], x[u]);
    }
}

// d = beta (v - rk ksum), from the row sum ksum of k_raw . x_d
__device__ __forceinline__ float node_delta(float ksum, float rk, float v, float beta) {
    return beta * fmaf(-rk, ksum, v);
}

// CHAIN: parents == NULL (node i extends node i - 1), so the recurrence
// needs only the previous node's row; otherwise every node's row is kept.
// RB: state rows per block (V / RB blocks per request and head).
template <typename TIn, int K, int V, int NMAX, bool CHAIN, int MODE, int RB>
__global__ __launch_bounds__(256) void verify_kernel(const VerifyParams p) {
    constexpr bool REPLAY = MODE == kModeReplay;
    constexpr bool SNAP = MODE == kModeSnap;
    // A state row is held by LPR lanes, NV float4 per lane (element offsets
    // 4j and, for NV = 2, K/2 + 4j): 8 elements per lane for K >= 64, so a
    // row's dot products need log2(LPR) lane-exchange steps per 8 elements.
    constexpr int NV = K >= 64 ? 2 : 1;
    constexpr int LPR = K / (4 * NV);
    constexpr int RPI = 64 / LPR;                    // rows per wave instruction
    constexpr int RPW = RB / kWaves;
    constexpr int IT = RPW / RPI;
    constexpr int NRB = V / RB;
    constexpr int CH = 2 * K + RB;        // conv channels of one block
    constexpr int NCS = (CH + 255) / 256;
    constexpr int NG = (NMAX * K + 255) / 256;       // gate elements per thread
    constexpr int HALF = K / NV;
    static_assert(IT >= 1 && RPW % RPI == 0, "row tiling");

    __shared__ float s_q[NMAX][K];
    __shared__ float s_k[NMAX][K];
    __shared__ float s_eg[NMAX][K];
    __shared__ float s_v[NMAX][RB];
    __shared__ float s_o[NMAX][RB];
    __shared__ float s_beta[NMAX], s_rq[NMAX], s_rk[NMAX], s_qk[NMAX];
    // trees only (a chain's conv windows come from registers):
    __shared__ TIn s_in[CHAIN ? 1 : NMAX + kMaxWidth - 1][CHAIN ? 1 : CH];   // node inputs, then conv state by age
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
    const bool bad_snap = SNAP && p.snaps != nullptr && (sslot < 0 || sslot >= p.num_snap_slots);
    if (REPLAY) {
        const int acc = p.accepted[r];
        // nothing accepted, or a padded request: the slot stays as it is
        if (acc < 0 || acc >= N || slot < 0 || slot >= p.num_slots || cslot < 0 || cslot >= p.num_conv_slots)
            return;
    } else if (slot < 0 || slot >= p.num_slots || bad_snap || cslot < 0 ||
               cslot >= p.num_conv_slots) {          // padded request (or an index out of range)
        for (int t = tid; t < N * RB; t += 256) {
            const int i = t / RB, rr = t % RB;
            o[((int64_t)r * N + i) * p.os0 + h * p.os1 + rb * RB + rr] = from_f32<TIn>(0.0f);
        }
        return;
    }

    // ---- every global load of the block is issued here, before any use:
    // the prologue's inputs first, then the state rows, which the prologue
    // does not need, so that they are still in flight while it runs ----
    const int j = lane % LPR;
    const int rs = lane / LPR;
    const int rloc0 = wave * RPW + rs;

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
    // optional inputs are read branch-free from a valid address (a branch
    // around a load makes the compiler wait for every load in flight)
    const bool has_bias = p.cb != nullptr;
    const TIn* cb = has_bias ? static_cast<const TIn*>(p.cb) : cw;
    TIn raw[NCS][NMAX], cs_age[NCS][kMaxWidth - 1], bias_raw[NCS];
    float w_age[NCS][kMaxWidth];
#pragma unroll
    for (int sl = 0; sl < NCS; ++sl) {
        const int cc = min(tid + 256 * sl, CH - 1);
        const int64_t c = cc < K ? (int64_t)hq * K + cc
                        : cc < 2 * K ? (int64_t)p.H * K + hq * K + (cc - K)
                        : 2 * (int64_t)p.H * K + h * V + rb * RB + (cc - 2 * K);
#pragma unroll
        for (int i = 0; i < NMAX; ++i) raw[sl][i] = mixed_r[(int64_t)min(i, N - 1) * p.ms + c];
#pragma unroll
        for (int m = 0; m < kMaxWidth - 1; ++m) cs_age[sl][m] = cs_base[c * (W - 1) + max(W - 2 - m, 0)];
#pragma unroll
        for (int m = 0; m < kMaxWidth; ++m) w_age[sl][m] = ld(cw, c * W + max(W - 1 - m, 0));
        bias_raw[sl] = cb[has_bias ? c : 0];
    }

    // gate and beta inputs
    float graw[NG], gdt[NG];
#pragma unroll
    for (int u = 0; u < NG; ++u) {
        const int t = tid + 256 * u;
        const int i = min(t / K, N - 1), kk = t % K;
        graw[u] = ld(static_cast<const TIn*>(p.a), ((int64_t)r * N + i) * p.as0 + h * K + kk);
        const float dt_raw = (p.dt_bias ? p.dt_bias : p.pool)[p.dt_bias ? h * K + kk : 0];
        gdt[u] = p.dt_bias ? dt_raw : 0.0f;
    }
    const float braw = ld(static_cast<const TIn*>(p.b), ((int64_t)r * N + min(tid, N - 1)) * p.bs0 + h);
    const int gmode = p.gate;
    const float alog = (p.A_log ? p.A_log : p.pool)[p.A_log ? h : 0];
    const float expA = gmode != kGateRaw ? __expf(alog) : 0.0f;

    const float* S = p.pool + ((int64_t)slot * p.HV + h) * (int64_t)V * K;
    float4 x0[IT][NV];
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int u = 0; u < NV; ++u)
            x0[it][u] = ld4(S, (int64_t)(rb * RB + rloc0 + it * RPI) * K + u * HALF + 4 * j);

    // ---- conv + SiLU per channel and node ----
    if constexpr (CHAIN) {
        // A chain's window is static: tap m of node i reads node i - m, or
        // conv-state age m - i once the draft is exhausted.  Everything is
        // already in registers, so there is no walk and no branch; nodes
        // past N are computed from the clamped rows and never used.  Taps
        // at or beyond W leave the sum unchanged (a select, so an unused
        // state entry cannot leak in).
#pragma unroll
        for (int sl = 0; sl < NCS; ++sl) {
            const int cc = tid + 256 * sl;
            if (cc < CH) {
#pragma unroll
                for (int i = 0; i < NMAX; ++i) {
                    float acc = fmaf(w_age[sl][0], to_f32(raw[sl][i]), has_bias ? to_f32(bias_raw[sl]) : 0.0f);
#pragma unroll
                    for (int m = 1; m < kMaxWidth; ++m) {
                        const float x = i - m >= 0 ? to_f32(raw[sl][i - m >= 0 ? i - m : 0])
                                                   : to_f32(cs_age[sl][m - i - 1 >= 0 ? m - i - 1 : 0]);
                        const float t = fmaf(w_age[sl][m], x, acc);
                        acc = m < W ? t : acc;
                    }
                    if (p.act == KDA_ACT_SILU) acc = acc * sigmoidf(acc);
                    if (cc < K) s_q[i][cc] = acc;
                    else if (cc < 2 * K) s_k[i][cc - K] = acc;
                    else s_v[i][cc - 2 * K] = acc;
                }
            }
        }
    }
    // trees: each thread walks its channel's ancestor path in LDS
    if constexpr (!CHAIN) {
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
                    float acc = fmaf(w_age[sl][0], to_f32(raw[sl][i]), has_bias ? to_f32(bias_raw[sl]) : 0.0f);
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
    }   // !CHAIN
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

    // One (request, head, RB rows) per block.  Chains and the replay walk
    // one state per row: nodes outer, the lane's row groups inner, so each
    // node's k, q and e^g are read from LDS once and the row groups give
    // independent work between the row reductions.  Trees keep every
    // node's state: row groups outer, nodes inner.
    const bool snap = SNAP && p.snaps != nullptr;
    float* snap0 = snap ? p.snaps + ((int64_t)sslot * N * p.HV + h) * (int64_t)V * K : nullptr;
    const int64_t node_stride = (int64_t)p.HV * V * K;
    if constexpr (CHAIN || REPLAY) {
        unsigned path = 0;
        if constexpr (REPLAY) {
            // The path root .. accepted node as a bit mask over node
            // indices.  Every parent has a smaller index than its child, so
            // walking the indices downwards meets each ancestor in turn, and
            // taking the set bits upwards visits the path root first.
            int a = p.accepted[r];
#pragma unroll
            for (int i = NMAX - 1; i >= 0; --i)
                if (i == a) { path |= 1u << i; a = par[i]; }
        }
        float4 x[IT][NV];
#pragma unroll
        for (int it = 0; it < IT; ++it)
#pragma unroll
            for (int u = 0; u < NV; ++u) x[it][u] = x0[it][u];
#pragma unroll
        for (int i = 0; i < NMAX; ++i) {
            const bool on = REPLAY ? (i < N && ((path >> i) & 1u)) : i < N;
            if (on) {
                float4 kv[NV], qv[NV], eg[NV];
#pragma unroll
                for (int u = 0; u < NV; ++u) {
                    kv[u] = *reinterpret_cast<const float4*>(&s_k[i][u * HALF + 4 * j]);
                    eg[u] = *reinterpret_cast<const float4*>(&s_eg[i][u * HALF + 4 * j]);
                    qv[u] = REPLAY ? make_float4(0.f, 0.f, 0.f, 0.f)
                                   : *reinterpret_cast<const float4*>(&s_q[i][u * HALF + 4 * j]);
                }
                const float rk = s_rk[i], rq = s_rq[i], bt = s_beta[i], qk = s_qk[i];
                float kx[IT], qx[IT];
#pragma unroll
                for (int it = 0; it < IT; ++it) node_decay_dots<NV>(eg, kv, qv, x[it], kx[it], qx[it], !REPLAY);
#pragma unroll
                for (int it = 0; it < IT; ++it) {
                    kx[it] = lane_sum<LPR>(kx[it]);
                    if (!REPLAY) qx[it] = lane_sum<LPR>(qx[it]) * rq;
                }
                float ov[IT];
#pragma unroll
                for (int it = 0; it < IT; ++it) {
                    const int rloc = rloc0 + it * RPI;
                    const float d = node_delta(kx[it], rk, s_v[i][rloc], bt);
                    const float dk = d * rk;
#pragma unroll
                    for (int u = 0; u < NV; ++u) x[it][u] = f4fma(kv[u], dk, x[it][u]);
                    if (SNAP) {
                        float* dst = snap0 + i * node_stride + (int64_t)(rb * RB + rloc) * K + 4 * j;
#pragma unroll
                        for (int u = 0; u < NV; ++u) st4_nt(dst + u * HALF, x[it][u]);
                    }
                    ov[it] = p.scale * fmaf(d, qk, qx[it]);
                }
                if (!REPLAY && j == 0) {
#pragma unroll
                    for (int it = 0; it < IT; ++it) s_o[i][rloc0 + it * RPI] = ov[it];
                }
            }
        }
        if constexpr (REPLAY) {
            float* dst = p.pool_w + ((int64_t)slot * p.HV + h) * (int64_t)V * K;
#pragma unroll
            for (int it = 0; it < IT; ++it)
#pragma unroll
                for (int u = 0; u < NV; ++u)
                    st4(dst + (int64_t)(rb * RB + rloc0 + it * RPI) * K + u * HALF + 4 * j, x[it][u]);
            return;
        }
    } else {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int rloc = rloc0 + it * RPI;
            const int row = rb * RB + rloc;
            float* snap_row = snap ? snap0 + (int64_t)row * K + 4 * j : nullptr;
            float4 xs[NMAX][NV];
#pragma unroll
            for (int i = 0; i < NMAX; ++i) {
                if (i < N) {
                    float4 xp[NV];
                    const int pi = par[i];
#pragma unroll
                    for (int u = 0; u < NV; ++u) {
                        xp[u] = x0[it][u];
#pragma unroll
                        for (int jn = 0; jn < NMAX - 1; ++jn)
                            if (jn < i && pi == jn) xp[u] = xs[jn][u];
                    }
                    float4 kv[NV], qv[NV], eg[NV];
#pragma unroll
                    for (int u = 0; u < NV; ++u) {
                        kv[u] = *reinterpret_cast<const float4*>(&s_k[i][u * HALF + 4 * j]);
                        qv[u] = *reinterpret_cast<const float4*>(&s_q[i][u * HALF + 4 * j]);
                        eg[u] = *reinterpret_cast<const float4*>(&s_eg[i][u * HALF + 4 * j]);
                    }
                    const float rk = s_rk[i], rq = s_rq[i];
                    float kx, qx;
                    node_decay_dots<NV>(eg, kv, qv, xp, kx, qx, true);
                    kx = lane_sum<LPR>(kx);
                    qx = lane_sum<LPR>(qx) * rq;
                    const float d = node_delta(kx, rk, s_v[i][rloc], s_beta[i]);
                    const float dk = d * rk;
#pragma unroll
                    for (int u = 0; u < NV; ++u) {
                        xs[i][u] = f4fma(kv[u], dk, xp[u]);
                        if (SNAP) st4_nt(snap_row + i * node_stride + u * HALF, xs[i][u]);
                    }
                    if (j == 0) s_o[i][rloc] = p.scale * fmaf(d, s_qk[i], qx);
                }
            }
        }
    }
    lds_barrier();
    for (int t = tid; t < N * RB; t += 256) {
        const int i = t / RB, rr = t % RB;
        o[((int64_t)r * N + i) * p.os0 + h * p.os1 + rb * RB + rr] = from_f32<TIn>(s_o[i][rr]);
    }
}


// State rows per block (at most V), measured on the 48 x 6 workload: with
// snapshots the launch is bound by its streaming stores and more, smaller
// blocks start them sooner (32 rows); the replay carries one state per row
// and gains from more row groups per lane between the row reductions (128
// rows).
template <bool CHAIN, int MODE, int V>
constexpr int rows_per_block() {
    constexpr int want = MODE == kModeReplay ? 128 : 32;
    return V < want ? V : want;
}

template <typename TIn, int K, int V, int NMAX, int MODE>
hipError_t launch_kvn(const kda_verify_args& a, const VerifyParams& p, hipStream_t s) {
    if (p.parents) {
        constexpr int RB = rows_per_block<false, MODE, V>();
        const dim3 grid(static_cast<unsigned>(a.B * a.HV * (V / RB)));
        klaunch(verify_kernel<TIn, K, V, NMAX, false, MODE, RB>, grid, dim3(256), 0, s, p);
    } else {
        constexpr int RB = rows_per_block<true, MODE, V>();
        const dim3 grid(static_cast<unsigned>(a.B * a.HV * (V / RB)));
        klaunch(verify_kernel<TIn, K, V, NMAX, true, MODE, RB>, grid, dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

template <typename TIn, int K, int V, int MODE>
hipError_t launch_kv(const kda_verify_args& a, const VerifyParams& p, hipStream_t s) {
    return a.N <= 8 ? launch_kvn<TIn, K, V, 8, MODE>(a, p, s) : launch_kvn<TIn, K, V, 16, MODE>(a, p, s);
}

template <typename TIn, int K, int MODE>
hipError_t launch_k(const kda_verify_args& a, const VerifyParams& p, hipStream_t s) {
    switch (a.V) {
        case 32: return launch_kv<TIn, K, 32, MODE>(a, p, s);
        case 64: return launch_kv<TIn, K, 64, MODE>(a, p, s);
        default: return launch_kv<TIn, K, 128, MODE>(a, p, s);
    }
}

template <int MODE>
hipError_t launch_mode(const kda_verify_args& a, const VerifyParams& p, hipStream_t s) {
    auto by_k = [&](auto tin) -> hipError_t {
        using TIn = decltype(tin);
        switch (a.K) {
            case 32: return launch_k<TIn, 32, MODE>(a, p, s);
            case 64: return launch_k<TIn, 64, MODE>(a, p, s);
            default: return launch_k<TIn, 128, MODE>(a, p, s);
        }
    };
    return a.dtype == KDA_BF16 ? by_k(bf16{}) : by_k(float{});
}

inline VerifyParams make_verify_params(const kda_verify_args& a) {
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
}  // namespace kda
