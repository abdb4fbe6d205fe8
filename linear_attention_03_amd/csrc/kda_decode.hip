// Packed one-token decode (A7): per request r and head h, every row v of
// the stored state x = pool[slot, h, v, :] (= column v of S) becomes
//
//   x_d = exp(g) * x                      (Diag(exp g) S)
//   d   = beta * (v_v - k.x_d)            (delta-rule error)
//   x'  = x_d + d * k                     (rank-1 correction)
//   o_v = scale * q.x' = scale * (q.x_d + d * (q.k))
//
// The two dot products use x_d only, so one pass over the row suffices.
// Layout: K/4 lanes hold one row as float4 (a 512-byte row of K = 128 is
// one coalesced half-wave access); a block of 4 waves owns 64 rows of one
// (request, head); every state byte is read once and written once.
// Follows the bounded-gate packed decode of "[KDA] Support Helion MTP
// verification and harden prefill, decode" (Modifications) with the input
// checks of the 35197 report (validate_packed_decode_inputs).

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    const void* a;
    const void* b;
    int64_t qs0, qs1, ks0, ks1, vs0, vs1, os0, os1, as0, bs0;
    const float* A_log;
    const float* dt_bias;
    float lb;
    float scale;
    int gate, beta_is_raw, l2norm;
    int HV;
    int group;                 // HV / H: value heads per q/k head
    int num_slots;
    float* pool;
    const int32_t* idx;
};

constexpr int kWaves = 4;

// State rows per block: 64 of a 128-row head, two blocks per (request,
// head).  In a step whose state comes from HBM this measured 19.7 us for 48
// requests against 20.9 us with whole-head blocks (32-row blocks: 19.7 us).
constexpr int decode_rows_per_block(int V) { return V >= 64 ? 64 : V; }

// A state row is held by LPR lanes, NV float4 per lane at element offsets
// 4j and (NV = 2) K/2 + 4j, with j = lane % LPR: 8 elements per lane for
// K >= 64, so each row's dot products take log2(LPR) exchange steps.
template <typename TIn, int K, int V>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeParams p) {
    constexpr int NV = K >= 64 ? 2 : 1;
    constexpr int LPR = K / (4 * NV);        // lanes per state row
    constexpr int RPI = 64 / LPR;            // rows per wave instruction
    // RB rows of one head per block, the state rows of all four waves'
    // loads in flight at once
    constexpr int RB = decode_rows_per_block(V);
    constexpr int RPW = RB / kWaves;
    constexpr int IT = RPW / RPI;            // row groups per lane
    constexpr int HALF = K / NV;
    static_assert(IT >= 1 && RPW % RPI == 0, "row tiling");
    constexpr int NRB = V / RB;

    const int blk = blockIdx.x;
    const int rb = blk % NRB;
    const int bh = blk / NRB;
    const int h = bh % p.HV;
    const int r = bh / p.HV;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane % LPR;
    const int rs = lane / LPR;
    const int row0 = rb * RB + wave * RPW + rs;

    TIn* o = static_cast<TIn*>(p.o) + r * p.os0 + h * p.os1;
    const int slot = p.idx[r];
    if (slot < 0 || slot >= p.num_slots) {    // padded request (or index out of range)
        if (j == 0) {
#pragma unroll
            for (int it = 0; it < IT; ++it) o[row0 + it * RPI] = from_f32<TIn>(0.0f);
        }
        return;
    }
    float* S = p.pool + (static_cast<int64_t>(slot) * p.HV + h) * (int64_t)V * K;

    // every load first: this lane's q, k, gate channels, v and beta, then
    // the state rows, which the norms and the gate map do not need.  The
    // optional inputs are read branch-free from a valid address (a branch
    // around a load makes the compiler wait for every load in flight).
    const int hq = h / p.group;                // q/k head of this value head
    const TIn* qp = static_cast<const TIn*>(p.q) + r * p.qs0 + hq * p.qs1;
    const TIn* kp = static_cast<const TIn*>(p.k) + r * p.ks0 + hq * p.ks1;
    const TIn* ap = static_cast<const TIn*>(p.a) + r * p.as0 + h * K;
    const TIn* vp = static_cast<const TIn*>(p.v) + r * p.vs0 + h * p.vs1;
    float qv[NV][4], kv[NV][4], av[NV][4], dv[NV][4];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        const float4 q4 = ld4(qp, u * HALF + 4 * j), k4 = ld4(kp, u * HALF + 4 * j), a4 = ld4(ap, u * HALF + 4 * j);
        qv[u][0] = q4.x; qv[u][1] = q4.y; qv[u][2] = q4.z; qv[u][3] = q4.w;
        kv[u][0] = k4.x; kv[u][1] = k4.y; kv[u][2] = k4.z; kv[u][3] = k4.w;
        av[u][0] = a4.x; av[u][1] = a4.y; av[u][2] = a4.z; av[u][3] = a4.w;
        const float4 d4 = ld4(p.dt_bias ? p.dt_bias : p.pool, p.dt_bias ? (int64_t)h * K + u * HALF + 4 * j : 0);
        const bool has_dt = p.dt_bias != nullptr;
        dv[u][0] = has_dt ? d4.x : 0.f; dv[u][1] = has_dt ? d4.y : 0.f;
        dv[u][2] = has_dt ? d4.z : 0.f; dv[u][3] = has_dt ? d4.w : 0.f;
    }
    float vv[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) vv[it] = ld(vp, row0 + it * RPI);
    float beta = ld(static_cast<const TIn*>(p.b) + r * p.bs0, h);
    const int gmode = p.gate;
    const float alog = (p.A_log ? p.A_log : p.pool)[p.A_log ? h : 0];
    const float expA = gmode != kGateRaw ? __expf(alog) : 0.0f;
    float4 x[IT][NV];
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int u = 0; u < NV; ++u) x[it][u] = ld4(S, (int64_t)(row0 + it * RPI) * K + u * HALF + 4 * j);

    // norms, q.k and the gate; the norms enter as scalars: k.x_d = rk (k . x_d)
    // and x = x_d + (d rk) k
    float sq = 0.f, sk = 0.f, sqk = 0.f;
    float4 kk[NV], eg[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sq = fmaf(qv[u][e], qv[u][e], sq);
            sk = fmaf(kv[u][e], kv[u][e], sk);
            sqk = fmaf(qv[u][e], kv[u][e], sqk);
        }
        kk[u] = make_float4(kv[u][0], kv[u][1], kv[u][2], kv[u][3]);
        eg[u] = make_float4(gate_decay(av[u][0], gmode, expA, dv[u][0], p.lb),
                            gate_decay(av[u][1], gmode, expA, dv[u][1], p.lb),
                            gate_decay(av[u][2], gmode, expA, dv[u][2], p.lb),
                            gate_decay(av[u][3], gmode, expA, dv[u][3], p.lb));
    }
    sq = lane_sum<LPR>(sq);
    sk = lane_sum<LPR>(sk);
    sqk = lane_sum<LPR>(sqk);
    const float rq = p.l2norm ? rsqrtf(sq + kL2Eps) : 1.0f;
    const float rk = p.l2norm ? rsqrtf(sk + kL2Eps) : 1.0f;
    const float qk = sqk * rq * rk;
    if (p.beta_is_raw) beta = sigmoidf(beta);

#pragma unroll
    for (int it = 0; it < IT; ++it) {
        float4 xd[NV];
        float kx = 0.f, qx = 0.f;
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            xd[u] = f4mul(eg[u], x[it][u]);
            kx += fdot4(kk[u], xd[u]);
            qx += fdot4(make_float4(qv[u][0], qv[u][1], qv[u][2], qv[u][3]), xd[u]);
        }
        kx = lane_sum<LPR>(kx) * rk;
        qx = lane_sum<LPR>(qx) * rq;
        const float d = beta * (vv[it] - kx);
        const float dk = d * rk;
        const int row = row0 + it * RPI;
#pragma unroll
        for (int u = 0; u < NV; ++u) st4(S + (int64_t)row * K + u * HALF + 4 * j, f4fma(kk[u], dk, xd[u]));
        if (j == 0) o[row] = from_f32<TIn>(p.scale * (qx + d * qk));
    }
}

template <typename TIn, int K, int V>
hipError_t launch_kv(const kda_decode_args& a, const DecodeParams& p, hipStream_t s) {
    // V / RB blocks per (request, head)
    const dim3 grid(static_cast<unsigned>(a.B * a.HV * (V / decode_rows_per_block(V))));
    klaunch(decode_kernel<TIn, K, V>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

template <typename TIn, int K>
hipError_t launch_k(const kda_decode_args& a, const DecodeParams& p, hipStream_t s) {
    switch (a.V) {
        case 32: return launch_kv<TIn, K, 32>(a, p, s);
        case 64: return launch_kv<TIn, K, 64>(a, p, s);
        default: return launch_kv<TIn, K, 128>(a, p, s);
    }
}

template <typename TIn>
hipError_t launch_t(const kda_decode_args& a, const DecodeParams& p, hipStream_t s) {
    switch (a.K) {
        case 32: return launch_k<TIn, 32>(a, p, s);
        case 64: return launch_k<TIn, 64>(a, p, s);
        default: return launch_k<TIn, 128>(a, p, s);
    }
}

}  // namespace

hipError_t launch_decode(const kda_decode_args& a, hipStream_t s) {
    DecodeParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o; p.a = a.a; p.b = a.b;
    p.qs0 = a.q_stride[0]; p.qs1 = a.q_stride[1];
    p.ks0 = a.k_stride[0]; p.ks1 = a.k_stride[1];
    p.vs0 = a.v_stride[0]; p.vs1 = a.v_stride[1];
    p.os0 = a.o_stride[0]; p.os1 = a.o_stride[1];
    p.as0 = a.a_stride; p.bs0 = a.b_stride;
    p.A_log = a.A_log; p.dt_bias = a.dt_bias; p.lb = a.lower_bound; p.scale = a.scale;
    p.gate = gate_mode(a.A_log, a.has_lower_bound); p.beta_is_raw = a.beta_is_raw; p.l2norm = a.use_qk_l2norm;
    p.HV = static_cast<int>(a.HV);
    p.group = static_cast<int>(a.HV / a.H);
    p.num_slots = static_cast<int>(a.num_slots);
    p.pool = a.state_pool; p.idx = a.state_indices;
    return a.dtype == KDA_BF16 ? launch_t<bf16>(a, p, s) : launch_t<float>(a, p, s);
}

}  // namespace kda
