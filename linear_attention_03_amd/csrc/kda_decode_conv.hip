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

// The conv's inputs are loaded apart from its arithmetic, so that a kernel
// can issue every load before it needs any (a use waits for every load
// issued before it).  Loads are branch-free: the state address is valid
// whatever `valid` says, and the bias address whatever p.bias is.

// One channel: its new input, weights, state (oldest first) and bias.
template <typename T, int W>
struct ChanIn {
    T x, w[W], s[W - 1];
    float b;
};

template <typename T, int W>
__device__ __forceinline__ ChanIn<T, W> load_channel(const DecodeConvParams& p, const T* xrow, const T* st,
                                                     int64_t c) {
    ChanIn<T, W> in;
    const T* wc = static_cast<const T*>(p.w) + c * W;
    in.x = xrow[c];
#pragma unroll
    for (int t = 0; t < W; ++t) in.w[t] = wc[t];
#pragma unroll
    for (int t = 0; t < W - 1; ++t) in.s[t] = st[c * (W - 1) + t];
    const T* bp = p.bias ? static_cast<const T*>(p.bias) : static_cast<const T*>(p.w);
    const float braw = ld(bp, p.bias ? c : 0);
    in.b = p.bias ? braw : 0.0f;
    return in;
}

// Conv of one channel: window = conv state (oldest first) then the new
// input, newest tap first as in the conv update and verify kernels, then
// the activation.
template <typename T, int W>
__device__ __forceinline__ float conv_channel(const DecodeConvParams& p, const ChanIn<T, W>& in, bool valid) {
    float acc = fmaf(to_f32(in.w[W - 1]), to_f32(in.x), in.b);
#pragma unroll
    for (int t = W - 2; t >= 0; --t) acc = fmaf(to_f32(in.w[t]), to_f32(in.s[t]), acc);
    if (p.act == KDA_ACT_SILU) acc = acc * sigmoidf(acc);
    return valid ? acc : 0.0f;
}

// Roll of one channel: the state keeps the window's last W-1 entries.
template <typename T, int W>
__device__ __forceinline__ void roll_channel(const ChanIn<T, W>& in, T* st, int64_t c) {
#pragma unroll
    for (int t = 0; t < W - 2; ++t) st[c * (W - 1) + t] = in.s[t + 1];
    st[c * (W - 1) + W - 2] = in.x;
}

// The 4 consecutive channels c .. c+3 (c a multiple of 4): input, weights
// and state of the group are contiguous, so they come in 8-byte loads.
template <typename T, int W>
struct Group4In {
    Span<T, 4> x;
    Span<T, 4 * W> w;
    Span<T, 4 * (W - 1)> s;
    float b[4];
};

template <typename T, int W>
__device__ __forceinline__ Group4In<T, W> load_group4(const DecodeConvParams& p, const T* xrow, const T* st,
                                                      int64_t c) {
    Group4In<T, W> in;
    in.x = load_span<T, 4>(xrow + c);
    in.w = load_span<T, 4 * W>(static_cast<const T*>(p.w) + c * W);
    in.s = load_span<T, 4 * (W - 1)>(st + c * (W - 1));
    const T* bp = p.bias ? static_cast<const T*>(p.bias) : static_cast<const T*>(p.w);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float braw = ld(bp, p.bias ? c + e : 0);
        in.b[e] = p.bias ? braw : 0.0f;
    }
    return in;
}

// Same arithmetic as conv_channel, per channel of the group.
template <typename T, int W>
__device__ __forceinline__ void conv_group4(const DecodeConvParams& p, const Group4In<T, W>& in, bool valid,
                                            float out[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float acc = fmaf(to_f32(in.w.e[e * W + W - 1]), to_f32(in.x.e[e]), in.b[e]);
#pragma unroll
        for (int t = W - 2; t >= 0; --t) acc = fmaf(to_f32(in.w.e[e * W + t]), to_f32(in.s.e[e * (W - 1) + t]), acc);
        if (p.act == KDA_ACT_SILU) acc = acc * sigmoidf(acc);
        out[e] = valid ? acc : 0.0f;
    }
}

// Roll of the group: one contiguous span of states, written in 8-byte units.
template <typename T, int W>
__device__ __forceinline__ void roll_group4(const Group4In<T, W>& in, T* st, int64_t c) {
    constexpr int NS = 4 * (W - 1);
    Span<T, NS> n;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int t = 0; t < W - 2; ++t) n.e[e * (W - 1) + t] = in.s.e[e * (W - 1) + t + 1];
        n.e[e * (W - 1) + W - 2] = in.x.e[e];
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

    // Every load comes before any use: first the q and k conv inputs of
    // this thread's group of 4 channels (GPW groups per wave: wave w takes
    // groups GPW w .. GPW w + GPW - 1; a thread without a group loads the
    // last one again and leaves it unused), then per value head its gate
    // row, dt_bias, beta, the v conv inputs of the wave's rows (lane l
    // convolves row wave * RPW + l % RPW) and the state rows (the bulk of
    // the bytes, needed last).
    constexpr int GPW = (K / 2 + Sh::WAVES - 1) / Sh::WAVES;
    const int g4 = wave * GPW + lane;
    const bool own_group = lane < GPW && g4 < K / 2;
    const int g4c = min(g4, K / 2 - 1);
    const int64_t cg = (g4c < K / 4 ? cq : ck - K) + 4 * (int64_t)g4c;
    const Group4In<TIn, W> gin = load_group4<TIn, W>(p, xrow, st, cg);
    float4 x[IT][NV];
    float4 eg[NV];
    float vconv, bt;
    ChanIn<TIn, W> vin;
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
        const int64_t cv = 2 * (int64_t)p.H * K + (int64_t)h * V + wave * RPW;
        vin = load_channel<TIn, W>(p, xrow, st, cv + lane % RPW);
        __builtin_amdgcn_sched_barrier(0);      // the state loads stay behind these
        const float* S = p.pool + (static_cast<int64_t>(slot) * p.HV + h) * (int64_t)V * K;
#pragma unroll
        for (int it = 0; it < IT; ++it)
#pragma unroll
            for (int u = 0; u < NV; ++u) x[it][u] = ld4(S, (int64_t)(row0 + it * RPI) * K + u * HALF + 4 * j);
        vconv = conv_channel<TIn, W>(p, vin, cvalid);
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

    // q and k of head hq: the 2K conv outputs, one group of 4 channels per
    // owning thread, shared through LDS; the owner rolls its group's state
    // (the only other reads of it are the unused loads of threads without a
    // group, whose values do not matter)
    __shared__ __attribute__((aligned(16))) float s_qk[2 * K];
    if (own_group) {
        float y[4];
        conv_group4<TIn, W>(p, gin, cvalid, y);
        *reinterpret_cast<float4*>(&s_qk[4 * g4]) = make_float4(y[0], y[1], y[2], y[3]);
        if (cvalid) roll_group4<TIn, W>(gin, st, cg);
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
        if (cvalid && lane < RPW) roll_channel<TIn, W>(vin, st, cv + lane);
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

// Without grouped heads the bf16 body is held to 96 registers, five waves
// per SIMD (float32 inputs, with twice the conv operand registers, keep the
// compiler's choice).  Measured on 48 x 1: at 80 registers (six waves, the
// 768 blocks in one round) the q / k conv inputs, loaded up front with
// everything else, spilled and the call took 23.6 / 34.1 us hot / cold; at
// 96, 17.0 / 23.7 us, against 17.1 / 26.6 us with those inputs loaded only
// after the v conv had waited for the state.
template <typename TIn>
constexpr int flat_waves_per_eu() { return sizeof(TIn) == 2 ? 5 : 1; }

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
