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
// one coalesced half-wave access); a block of 4 waves owns 32 rows of one
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
    int has_alog, beta_is_raw, l2norm;
    int HV;
    int num_slots;
    float* pool;
    const int32_t* idx;
};

constexpr int kRowsPerBlock = 32;
constexpr int kWaves = 4;

template <typename TIn, int K, int V>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeParams p) {
    constexpr int LPR = K / 4;               // lanes per state row
    constexpr int RPI = 64 / LPR;            // rows per wave instruction
    constexpr int RPW = kRowsPerBlock / kWaves;
    constexpr int IT = RPW / RPI;            // row groups per lane
    static_assert(IT >= 1 && RPW % RPI == 0, "row tiling");
    constexpr int NRB = V / kRowsPerBlock;

    const int blk = blockIdx.x;
    const int rb = blk % NRB;
    const int bh = blk / NRB;
    const int h = bh % p.HV;
    const int r = bh / p.HV;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane % LPR;
    const int rs = lane / LPR;
    const int row0 = rb * kRowsPerBlock + wave * RPW + rs;

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

    float4 x[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) x[it] = ld4(S, (int64_t)(row0 + it * RPI) * K + 4 * j);

    const TIn* qp = static_cast<const TIn*>(p.q) + r * p.qs0 + h * p.qs1 + 4 * j;
    const TIn* kp = static_cast<const TIn*>(p.k) + r * p.ks0 + h * p.ks1 + 4 * j;
    const TIn* ap = static_cast<const TIn*>(p.a) + r * p.as0 + h * K + 4 * j;
    const TIn* vp = static_cast<const TIn*>(p.v) + r * p.vs0 + h * p.vs1;
    float4 qv = make_float4(ld(qp, 0), ld(qp, 1), ld(qp, 2), ld(qp, 3));
    float4 kv = make_float4(ld(kp, 0), ld(kp, 1), ld(kp, 2), ld(kp, 3));
    float vv[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) vv[it] = ld(vp, row0 + it * RPI);

    if (p.l2norm) {
        const float sq = lane_sum<LPR>(fdot4(qv, qv)), sk = lane_sum<LPR>(fdot4(kv, kv));
        qv = f4scale(qv, rsqrtf(sq + kL2Eps));
        kv = f4scale(kv, rsqrtf(sk + kL2Eps));
    }
    const float qk = lane_sum<LPR>(fdot4(qv, kv));

    const bool has_alog = p.has_alog;
    const float expA = has_alog ? __expf(p.A_log[h]) : 0.0f;
    float4 dt = make_float4(0.f, 0.f, 0.f, 0.f);
    if (p.dt_bias) dt = ld4(p.dt_bias, (int64_t)h * K + 4 * j);
    float4 eg;
    eg.x = gate_decay(ld(ap, 0), has_alog, expA, dt.x, p.lb);
    eg.y = gate_decay(ld(ap, 1), has_alog, expA, dt.y, p.lb);
    eg.z = gate_decay(ld(ap, 2), has_alog, expA, dt.z, p.lb);
    eg.w = gate_decay(ld(ap, 3), has_alog, expA, dt.w, p.lb);
    float beta = ld(static_cast<const TIn*>(p.b) + r * p.bs0, h);
    if (p.beta_is_raw) beta = sigmoidf(beta);

#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const float4 xd = f4mul(eg, x[it]);
        const float kx = lane_sum<LPR>(fdot4(kv, xd)), qx = lane_sum<LPR>(fdot4(qv, xd));
        const float d = beta * (vv[it] - kx);
        const int row = row0 + it * RPI;
        st4(S + (int64_t)row * K + 4 * j, f4fma(kv, d, xd));
        if (j == 0) o[row] = from_f32<TIn>(p.scale * (qx + d * qk));
    }
}

template <typename TIn, int K, int V>
hipError_t launch_kv(const kda_decode_args& a, const DecodeParams& p, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(a.B * a.HV * (V / kRowsPerBlock)));
    hipLaunchKernelGGL((decode_kernel<TIn, K, V>), grid, dim3(256), 0, s, p);
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
    p.has_alog = a.A_log != nullptr; p.beta_is_raw = a.beta_is_raw; p.l2norm = a.use_qk_l2norm;
    p.HV = static_cast<int>(a.HV);
    p.num_slots = static_cast<int>(a.num_slots);
    p.pool = a.state_pool; p.idx = a.state_indices;
    return a.dtype == KDA_BF16 ? launch_t<bf16>(a, p, s) : launch_t<float>(a, p, s);
}

}  // namespace kda
