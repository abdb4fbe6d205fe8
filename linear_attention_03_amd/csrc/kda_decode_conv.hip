// Packed one-token decode with the depthwise causal conv update fused in:
// one launch does what kda_conv_update followed by kda_decode on the conv's
// q || k || v output does ("[KDA] Default GLM-5-Next spec verify to the
// CuTe DSL KDA kernel", Summary: the conv1d update and the recurrence in
// one launch).
//
// Per request r and q/k head hq one block of 8 waves (4 where V is small)
// convolves the token's
// q and k channels of hq and the v channels of every value head reading hq
// (the conv outputs stay in fp32, as in the verify kernel's fused conv;
// the two-launch path stores them in the input dtype first), runs the
// decode update of every state row of those value heads, and rolls the
// conv state of all those channels in place.  Each conv-state entry is read and
// written by this one block only: each group of 4 q / k channels is
// convolved by one thread (inputs, weights and state in 8-byte loads),
// which also rolls it, and shared with every wave through LDS; each v
// channel is convolved by the wave that owns its row, handed to the row's
// lanes by shuffles and rolled once every copy has been used.
//
// The per-row arithmetic is the decode kernel's, in the same order.

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

struct DecodeConvParams {
    const void* x;              // mixed_qkv, pre-conv [B, conv_dim]
    int64_t xs;
    const void* w;              // [conv_dim, W]
    const void* bias;           // [conv_dim] or null
    void* cs;                   // [num_conv_slots, conv_dim, W-1]
    const int32_t* cidx;        // [B] or null (state index)
    int64_t conv_dim;
    int num_conv_slots, act;
    void* o;
    const void* a;
    const void* b;
    int64_t os0, os1, as0, bs0;
    const float* A_log;
    const float* dt_bias;
    float lb, scale;
    int gate, beta_is_raw, l2norm;
    int H, HV, group, num_slots;
    float* pool;
    const int32_t* idx;
};

// Conv of one channel: window = conv state (oldest first) then the new
// input, newest tap first as in the conv update and verify kernels, then
// the activation.
template <typename T, int W>
__device__ __forceinline__ float conv_channel(const DecodeConvParams& p, const T* xrow, const T* st, int64_t c,
                                              bool valid) {
    // (loads branch-free: st and the bias address are valid whatever `valid`
    // and p.bias are, and a branch around a load makes the compiler wait for
    // every load in flight)
    const T* wc = static_cast<const T*>(p.w) + c * W;
    const T* bp = p.bias ? static_cast<const T*>(p.bias) : static_cast<const T*>(p.w);
    const float braw = ld(bp, p.bias ? c : 0);
    const float b = p.bias ? braw : 0.0f;
    float acc = fmaf(to_f32(wc[W - 1]), to_f32(xrow[c]), b);
#pragma unroll
    for (int t = W - 2; t >= 0; --t) acc = fmaf(to_f32(wc[t]), to_f32(st[c * (W - 1) + t]), acc);
    if (p.act == KDA_ACT_SILU) acc = acc * sigmoidf(acc);
    return valid ? acc : 0.0f;
}

// n consecutive elements of type T from p (8-byte aligned, n * sizeof(T) a
// multiple of 8) in 8-byte loads.
template <typename T, int N>
struct Span {
    T e[N];
};
template <typename T, int N>
__device__ __forceinline__ Span<T, N> load_span(const T* p) {
    static_assert((N * sizeof(T)) % 8 == 0, "8-byte units");
    Span<T, N> s;
    uint2 u[N * sizeof(T) / 8];
#pragma unroll
    for (int i = 0; i < (int)(N * sizeof(T) / 8); ++i) u[i] = reinterpret_cast<const uint2*>(p)[i];
    __builtin_memcpy(s.e, u, sizeof(s.e));
    return s;
}

// Conv of the 4 consecutive channels c .. c+3 (c a multiple of 4): the
// input, the weights and the state of the group are contiguous, so they
// come in 8-byte loads; same arithmetic as conv_channel.
template <typename T, int W>
__device__ __forceinline__ void conv_group4(const DecodeConvParams& p, const T* xrow, const T* st, int64_t c,
                                            bool valid, float out[4]) {
    const Span<T, 4> x = load_span<T, 4>(xrow + c);
    const Span<T, 4 * W> w = load_span<T, 4 * W>(static_cast<const T*>(p.w) + c * W);
    const Span<T, 4 * (W - 1)> s = load_span<T, 4 * (W - 1)>(st + c * (W - 1));
    const T* bp = p.bias ? static_cast<const T*>(p.bias) : static_cast<const T*>(p.w);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float braw = ld(bp, p.bias ? c + e : 0);
        const float b = p.bias ? braw : 0.0f;
        float acc = fmaf(to_f32(w.e[e * W + W - 1]), to_f32(x.e[e]), b);
#pragma unroll
        for (int t = W - 2; t >= 0; --t) acc = fmaf(to_f32(w.e[e * W + t]), to_f32(s.e[e * (W - 1) + t]), acc);
        if (p.act == KDA_ACT_SILU) acc = acc * sigmoidf(acc);
        out[e] = valid ? acc : 0.0f;
    }
}

// Roll of one channel: the state keeps the window's last W-1 entries.
template <typename T, int W>
__device__ __forceinline__ void roll_channel(const T* xrow, T* st, int64_t c) {
    T keep[W - 1];
#pragma unroll
    for (int t = 0; t < W - 2; ++t) keep[t] = st[c * (W - 1) + t + 1];
    keep[W - 2] = xrow[c];
#pragma unroll
    for (int t = 0; t < W - 1; ++t) st[c * (W - 1) + t] = keep[t];
}

// Roll of the 4 consecutive channels c .. c+3 (c a multiple of 4): their
// states are one contiguous span, read and written in 8-byte units.
template <typename T, int W>
__device__ __forceinline__ void roll_group4(const T* xrow, T* st, int64_t c) {
    constexpr int NS = 4 * (W - 1);
    const Span<T, 4> x = load_span<T, 4>(xrow + c);
    const Span<T, NS> s = load_span<T, NS>(st + c * (W - 1));
    Span<T, NS> n;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int t = 0; t < W - 2; ++t) n.e[e * (W - 1) + t] = s.e[e * (W - 1) + t + 1];
        n.e[e * (W - 1) + W - 2] = x.e[e];
    }
    uint2 u[NS * sizeof(T) / 8];
    __builtin_memcpy(u, n.e, sizeof(u));
#pragma unroll
    for (int i = 0; i < (int)(NS * sizeof(T) / 8); ++i) reinterpret_cast<uint2*>(st + c * (W - 1))[i] = u[i];
}

template <int K, int V>
struct DecodeConvShape {
    static constexpr int NV = K >= 64 ? 2 : 1;
    static constexpr int LPR = K / (4 * NV);            // lanes per state row
    static constexpr int RPI = 64 / LPR;                // rows per wave instruction
    static constexpr int WAVES = V / RPI >= 4 * 8 ? 8 : 4;   // 4 row groups per lane where V allows
    static constexpr int RPW = V / WAVES;               // rows of a head per wave
    static constexpr int IT = RPW / RPI;                // row groups per lane
    static constexpr int HALF = K / NV;
};

// kGrouped: HV > H (several value heads per q/k head, walked in a loop);
// without it the body is straight-line code, which keeps the register count
// near that of the plain decode.
template <typename TIn, int K, int V, int W, bool kGrouped>
__device__ __forceinline__ void decode_conv_body(const DecodeConvParams& p) {
    using Sh = DecodeConvShape<K, V>;
    constexpr int NV = Sh::NV, LPR = Sh::LPR, RPI = Sh::RPI, RPW = Sh::RPW, IT = Sh::IT, HALF = Sh::HALF;
    static_assert(IT >= 1 && RPW % RPI == 0 && RPW <= 64, "row tiling");

    const int hq = blockIdx.x % p.H;
    const int r = blockIdx.x / p.H;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane % LPR;
    const int rs = lane / LPR;
    const int row0 = wave * RPW + rs;
    const int h0 = hq * p.group;             // first value head reading hq

    const int slot = p.idx[r];
    if (slot < 0 || slot >= p.num_slots) {   // padded request: zero output, nothing else touched
        for (int hh = 0; hh < p.group; ++hh) {
            TIn* o = static_cast<TIn*>(p.o) + r * p.os0 + (h0 + hh) * p.os1;
            if (j == 0) {
#pragma unroll
                for (int it = 0; it < IT; ++it) o[row0 + it * RPI] = from_f32<TIn>(0.0f);
            }
        }
        return;
    }
    const int cslot = p.cidx ? p.cidx[r] : slot;
    const bool cvalid = cslot >= 0 && cslot < p.num_conv_slots;
    const TIn* xrow = static_cast<const TIn*>(p.x) + (int64_t)r * p.xs;
    TIn* st = static_cast<TIn*>(p.cs) + (int64_t)(cvalid ? cslot : 0) * p.conv_dim * (W - 1);
    const int64_t cq = (int64_t)hq * K, ck = (int64_t)p.H * K + hq * K;

    // Loads of one value head: its gate row, dt_bias, beta and state rows
    // (the bulk of the bytes) are all issued before the v conv of the
    // wave's rows (lane l convolves row wave * RPW + l % RPW) and the gate
    // map use any of them.
    float4 x[IT][NV];
    float4 eg[NV];
    float vconv, bt;
    const int gmode = p.gate;
    auto load_head = [&](int h) {
        const TIn* ap = static_cast<const TIn*>(p.a) + r * p.as0 + h * K;
        const float alog = (p.A_log ? p.A_log : p.pool)[p.A_log ? h : 0];
        float4 a4[NV], dr[NV];
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            a4[u] = ld4(ap, u * HALF + 4 * j);
            dr[u] = ld4(p.dt_bias ? p.dt_bias : p.pool, p.dt_bias ? (int64_t)h * K + u * HALF + 4 * j : 0);
        }
        const float beta = ld(static_cast<const TIn*>(p.b) + r * p.bs0, h);
        // the state rows: nothing before the recurrence needs them
        const float* S = p.pool + (static_cast<int64_t>(slot) * p.HV + h) * (int64_t)V * K;
#pragma unroll
        for (int it = 0; it < IT; ++it)
#pragma unroll
            for (int u = 0; u < NV; ++u) x[it][u] = ld4(S, (int64_t)(row0 + it * RPI) * K + u * HALF + 4 * j);
        const int64_t cv = 2 * (int64_t)p.H * K + (int64_t)h * V + wave * RPW;
        vconv = conv_channel<TIn, W>(p, xrow, st, cv + lane % RPW, cvalid);
        const float expA = gmode != kGateRaw ? __expf(alog) : 0.0f;
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const float4 d4 = p.dt_bias ? dr[u] : make_float4(0.f, 0.f, 0.f, 0.f);
            eg[u] = make_float4(gate_decay(a4[u].x, gmode, expA, d4.x, p.lb), gate_decay(a4[u].y, gmode, expA, d4.y, p.lb),
                                gate_decay(a4[u].z, gmode, expA, d4.z, p.lb), gate_decay(a4[u].w, gmode, expA, d4.w, p.lb));
        }
        bt = p.beta_is_raw ? sigmoidf(beta) : beta;
    };
    load_head(h0);

    // q and k of head hq: the 2K conv outputs in K / 2 groups of 4 channels,
    // one group per thread (GPW per wave: wave w takes groups GPW w ..
    // GPW w + GPW - 1), shared through LDS; the thread that convolved a group
    // rolls its state (it alone reads it, and its arithmetic has used the
    // loads)
    constexpr int GPW = (K / 2 + Sh::WAVES - 1) / Sh::WAVES;
    __shared__ __attribute__((aligned(16))) float s_qk[2 * K];
    {
        const int g4 = wave * GPW + lane;
        if (lane < GPW && g4 < K / 2) {
            const int64_t c = (g4 < K / 4 ? cq : ck - K) + 4 * (int64_t)g4;
            float y[4];
            conv_group4<TIn, W>(p, xrow, st, c, cvalid, y);
            *reinterpret_cast<float4*>(&s_qk[4 * g4]) = make_float4(y[0], y[1], y[2], y[3]);
            if (cvalid) roll_group4<TIn, W>(xrow, st, c);
        }
    }
    lds_barrier();
    float qv[NV][4], kv[NV][4];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        const float4 q4 = *reinterpret_cast<const float4*>(&s_qk[u * HALF + 4 * j]);
        const float4 k4 = *reinterpret_cast<const float4*>(&s_qk[K + u * HALF + 4 * j]);
        qv[u][0] = q4.x; qv[u][1] = q4.y; qv[u][2] = q4.z; qv[u][3] = q4.w;
        kv[u][0] = k4.x; kv[u][1] = k4.y; kv[u][2] = k4.z; kv[u][3] = k4.w;
    }
    float sq = 0.f, sk = 0.f, sqk = 0.f;
    float4 kk[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sq = fmaf(qv[u][e], qv[u][e], sq);
            sk = fmaf(kv[u][e], kv[u][e], sk);
            sqk = fmaf(qv[u][e], kv[u][e], sqk);
        }
        kk[u] = make_float4(kv[u][0], kv[u][1], kv[u][2], kv[u][3]);
    }
    sq = lane_sum<LPR>(sq);
    sk = lane_sum<LPR>(sk);
    sqk = lane_sum<LPR>(sqk);
    const float rq = p.l2norm ? rsqrtf(sq + kL2Eps) : 1.0f;
    const float rk = p.l2norm ? rsqrtf(sk + kL2Eps) : 1.0f;
    const float qk = sqk * rq * rk;

    const int ngroup = kGrouped ? p.group : 1;
    for (int hh = 0; hh < ngroup; ++hh) {
        const int h = h0 + hh;
        if (kGrouped && hh > 0) load_head(h);
        float* S = p.pool + (static_cast<int64_t>(slot) * p.HV + h) * (int64_t)V * K;
        // this lane's rows take their v from the lanes that convolved them;
        // each v channel is then rolled by the lane that convolved its first
        // copy, after the shuffles used every copy
        float vv[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) vv[it] = __shfl(vconv, rs + it * RPI, 64);
        const int64_t cv = 2 * (int64_t)p.H * K + (int64_t)h * V + wave * RPW;
        if (cvalid && lane < RPW) roll_channel<TIn, W>(xrow, st, cv + lane);
        TIn* o = static_cast<TIn*>(p.o) + r * p.os0 + h * p.os1;
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
            const float d = bt * (vv[it] - kx);
            const float dk = d * rk;
            const int row = row0 + it * RPI;
#pragma unroll
            for (int u = 0; u < NV; ++u) st4(S + (int64_t)row * K + u * HALF + 4 * j, f4fma(kk[u], dk, xd[u]));
            if (j == 0) o[row] = from_f32<TIn>(p.scale * (qx + d * qk));
        }
    }
}

// Without grouped heads the bf16 body fits 80 registers, six waves per
// SIMD: three blocks of 8 waves per CU, so the 768 blocks of 48 requests x
// 16 heads run in one round (float32 inputs, with twice the conv operand
// registers, keep the compiler's choice).
template <typename TIn>
constexpr int flat_waves_per_eu() { return sizeof(TIn) == 2 ? 6 : 1; }

template <typename TIn, int K, int V, int W>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(flat_waves_per_eu<TIn>()))) void
decode_conv_kernel(const DecodeConvParams p) {
    decode_conv_body<TIn, K, V, W, false>(p);
}

template <typename TIn, int K, int V, int W>
__global__ __launch_bounds__(512) void decode_conv_grouped_kernel(const DecodeConvParams p) {
    decode_conv_body<TIn, K, V, W, true>(p);
}

template <typename TIn, int K, int V, int W>
hipError_t launch_kvw(const kda_decode_conv_args& a, const DecodeConvParams& p, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(a.B * a.H)), block(64 * DecodeConvShape<K, V>::WAVES);
    if (a.HV > a.H) klaunch(decode_conv_grouped_kernel<TIn, K, V, W>, grid, block, 0, s, p);
    else klaunch(decode_conv_kernel<TIn, K, V, W>, grid, block, 0, s, p);
    return hipGetLastError();
}

template <typename TIn, int K, int V>
hipError_t launch_kv(const kda_decode_conv_args& a, const DecodeConvParams& p, hipStream_t s) {
    switch (a.conv_width) {
        case 2: return launch_kvw<TIn, K, V, 2>(a, p, s);
        case 3: return launch_kvw<TIn, K, V, 3>(a, p, s);
        default: return launch_kvw<TIn, K, V, 4>(a, p, s);
    }
}

template <typename TIn, int K>
hipError_t launch_k(const kda_decode_conv_args& a, const DecodeConvParams& p, hipStream_t s) {
    switch (a.V) {
        case 32: return launch_kv<TIn, K, 32>(a, p, s);
        case 64: return launch_kv<TIn, K, 64>(a, p, s);
        default: return launch_kv<TIn, K, 128>(a, p, s);
    }
}

template <typename TIn>
hipError_t launch_t(const kda_decode_conv_args& a, const DecodeConvParams& p, hipStream_t s) {
    switch (a.K) {
        case 32: return launch_k<TIn, 32>(a, p, s);
        case 64: return launch_k<TIn, 64>(a, p, s);
        default: return launch_k<TIn, 128>(a, p, s);
    }
}

}  // namespace

hipError_t launch_decode_conv(const kda_decode_conv_args& a, hipStream_t s) {
    DecodeConvParams p;
    p.x = a.mixed_qkv; p.xs = a.mixed_stride;
    p.w = a.conv_weight; p.bias = a.conv_bias; p.cs = a.conv_state; p.cidx = a.conv_state_indices;
    p.conv_dim = 2 * a.H * a.K + a.HV * a.V;
    p.num_conv_slots = static_cast<int>(a.num_conv_slots);
    p.act = a.conv_activation;
    p.o = a.o; p.a = a.a; p.b = a.b;
    p.os0 = a.o_stride[0]; p.os1 = a.o_stride[1]; p.as0 = a.a_stride; p.bs0 = a.b_stride;
    p.A_log = a.A_log; p.dt_bias = a.dt_bias; p.lb = a.lower_bound; p.scale = a.scale;
    p.gate = gate_mode(a.A_log, a.has_lower_bound); p.beta_is_raw = a.beta_is_raw; p.l2norm = a.use_qk_l2norm;
    p.H = static_cast<int>(a.H); p.HV = static_cast<int>(a.HV);
    p.group = static_cast<int>(a.HV / a.H);
    p.num_slots = static_cast<int>(a.num_slots);
    p.pool = a.state_pool; p.idx = a.state_indices;
    return a.dtype == KDA_BF16 ? launch_t<bf16>(a, p, s) : launch_t<float>(a, p, s);
}

}  // namespace kda
