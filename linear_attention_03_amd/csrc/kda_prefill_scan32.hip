// Inter-chunk scan of the general prefill path on fp32 matrix tiles
// (v_mfma_f32_16x16x4f32, fp32 products and accumulation).  It reads the
// general prep's workspace as those kernels write it (fp32 W, U', P, Qt,
// Kt^T and e^G_last per chunk and head, in the read order of ws_run and
// ws_tile in kda_prefill_common.h) and computes, chunk after chunk,
//     U = U' - W S;  O = scale (Qt S + P U);  S <- e^G_last * S + Kt^T U
// for one sequence, one head and 16 state columns per block.
//
// Waves 0-3 ("state" waves) keep the state in MFMA accumulator tiles: wave
// w holds S rows 16 t .. 16 t + 15 for its tiles t = w, w + 4 (K / 16 tiles
// in all) and computes U rows 16 w .. 16 w + 15 (C / 16 tiles).  Waves 4-7
// ("output" waves) compute O rows 16 j .. 16 j + 15.  S and U pass between
// waves through LDS (transposed: one row per state column), two barriers
// per chunk; each chunk's operands are loaded during the previous one.
//
// Contraction order: a 16 x 16 x 4 tile product takes four contraction
// indices per step, one per 16-lane group.  Over a contraction of length L
// the lanes of group g take the indices L/4 g .. L/4 g + L/4 - 1, one per
// step, so every lane's operand run is one run of the workspace layout (W,
// Qt, P and Kt^T as row runs) or a row of S^T or U^T in LDS, read with
// 16-byte loads.

#include "kda_prefill_common.h"

namespace kda {
namespace {

typedef float f32x4m __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4m mfma_f32(float a, float b, f32x4m c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

constexpr int kScan32Waves = 8;

template <int C, int K>
struct Scan32Shape {
    static constexpr int NS = K / 16;            // state tiles
    static constexpr int NU = C / 16;            // corrected-value and output tiles
    static constexpr int SPW = (NS + 3) / 4;     // state tiles per state wave
    static constexpr int KQ = K / 4;             // contraction slots per lane group, channels
    static constexpr int CQ = C / 4;             // contraction slots per lane group, tokens
    static constexpr int LDS_S = K + 4;          // S^T row stride (16-byte rows, groups on distinct banks)
    static constexpr int LDS_U = C + 4;
};

template <int C, int K>
struct StateOps {                                // one chunk's operands of a state wave
    float w[Scan32Shape<C, K>::KQ];              // W row 16 w + l16, this lane group's channels
    float up[4];                                 // U' rows 16 w + 4 sub + i, this lane's column
    float kt[Scan32Shape<C, K>::SPW][Scan32Shape<C, K>::CQ];   // Kt at this lane group's tokens, channel 16 t + l16
    float4 gl[Scan32Shape<C, K>::SPW];           // e^G_last of this lane's state rows
};

template <int C, int K>
struct OutOps {
    float qt[Scan32Shape<C, K>::KQ];             // Qt row 16 j + l16, this lane group's channels
    float pp[Scan32Shape<C, K>::CQ];             // P row 16 j + l16, this lane group's tokens
};

// The N values this lane reads from a row block of a row-run operand
// (ws_run: N = L/4): float4 q of the lane at blk + 4 (64 q + lane), so each
// load of the wave is 1 KiB of consecutive memory.
template <int N>
__device__ __forceinline__ void load_runs(float* dst, const float* blk, int lane) {
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(blk + 4 * (64 * q + lane));
        dst[4 * q] = v.x; dst[4 * q + 1] = v.y; dst[4 * q + 2] = v.z; dst[4 * q + 3] = v.w;
    }
}

template <typename TIn, int C, int K, int V, bool kInter>
__global__ __launch_bounds__(64 * kScan32Waves) void scan32_kernel(const PrefillParams p) {
    using SH = Scan32Shape<C, K>;
    constexpr int NVS = V / 16;
    __shared__ __attribute__((aligned(16))) float sS[2][16 * SH::LDS_S];
    __shared__ __attribute__((aligned(16))) float sU[2][16 * SH::LDS_U];
    __shared__ int s_cstart;

    const int blk = blockIdx.x;
    const int vsl = blk % NVS;
    const int h = (blk / NVS) % p.HV;
    const int n = blk / (NVS * p.HV);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int sub = lane >> 4, l16 = lane & 15;
    const int col0 = vsl * 16;

    int b, t0, len, cstart;
    if (p.cu) {
        b = 0;
        t0 = cu_at(p.cu, n, p.T);
        len = seq_len(p.cu, n, p.T);
        cstart = 0;
        if (tid < 64) cstart = chunks_before(p.cu, n, p.T, C);
        if (tid == 0) s_cstart = cstart;
        __syncthreads();
        cstart = s_cstart;
    } else {
        b = n;
        t0 = 0;
        len = p.T;
        cstart = n * ceil_div(p.T, C);
    }
    const int nch = min(ceil_div(len, C), max(p.max_chunks - cstart, 0));
    const int slot = p.idx[n];
    if (slot < 0 || slot >= p.num_slots) return;   // index out of range: nothing is touched

    // workspace of chunk cc of this sequence and head (layout of the general prep)
    const int64_t cf = p.chunk_floats;
    auto chunk = [&](int cc) { return p.ws + ((int64_t)(cstart + cc) * p.HV + h) * cf; };
    constexpr int OFF_UP = C * K, OFF_P = C * (K + V), OFF_QT = C * (K + V + C), OFF_KT = C * (2 * K + V + C),
                  OFF_GL = C * (3 * K + V + C);
    const int w = wave & 3;

    if (wave >= 4) {
        // ---- output waves: O rows 16 w .. 16 w + 15
        const bool has_o = w < SH::NU;
        TIn* og = static_cast<TIn*>(p.o) + b * p.os[0] + h * p.os[2] + col0 + l16;
        auto load = [&](OutOps<C, K>& o, int cc) {
            if (!has_o) return;
            const float* ws = chunk(cc);
            load_runs<SH::KQ>(o.qt, ws + OFF_QT + (int64_t)w * SH::KQ * 64, lane);
            load_runs<SH::CQ>(o.pp, ws + OFF_P + (int64_t)w * SH::CQ * 64, lane);
        };
        // the next chunk's operands go into the other set first: its registers
        // were last read by the previous step's products
        auto step = [&](const OutOps<C, K>& o, OutOps<C, K>& nx, int cc, int buf) {
            load(nx, min(cc + 1, nch - 1));
            lds_barrier();                                  // S of chunk cc published
            f32x4m a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0, a3 = a0;
            if (has_o) {
                const float* srow = &sS[buf][l16 * SH::LDS_S + SH::KQ * sub];
#pragma unroll
                for (int j = 0; j < SH::KQ; j += 4) {
                    const float4 sv = *reinterpret_cast<const float4*>(srow + j);
                    a0 = mfma_f32(o.qt[j], sv.x, a0);
                    a1 = mfma_f32(o.qt[j + 1], sv.y, a1);
                    a2 = mfma_f32(o.qt[j + 2], sv.z, a2);
                    a3 = mfma_f32(o.qt[j + 3], sv.w, a3);
                }
            }
            lds_barrier();                                  // U of chunk cc published
            if (has_o) {
                const float* urow = &sU[buf][l16 * SH::LDS_U + SH::CQ * sub];
#pragma unroll
                for (int j = 0; j < SH::CQ; j += 4) {
                    const float4 uv = *reinterpret_cast<const float4*>(urow + j);
                    a0 = mfma_f32(o.pp[j], uv.x, a0);
                    a1 = mfma_f32(o.pp[j + 1], uv.y, a1);
                    a2 = mfma_f32(o.pp[j + 2], uv.z, a2);
                    a3 = mfma_f32(o.pp[j + 3], uv.w, a3);
                }
                // rows past the chunk (all rows of a padding step) store into
                // the sink: the stores carry no branch, which would make the
                // compiler wait for every load in flight at the merge
                const f32x4m ov = (a0 + a1) + (a2 + a3);
                const int clen = min(C, len - cc * C);
                TIn* const sink = reinterpret_cast<TIn*>(p.sink) + 4 * lane;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * w + 4 * sub + i;
                    TIn* const dst = r < clen ? og + (int64_t)(t0 + cc * C + r) * p.os[1] : sink + i;
                    *dst = from_f32<TIn>(p.scale * ov[i]);
                }
            }
        };
        if (nch <= 0) return;
        OutOps<C, K> oa, ob;
        load(oa, 0);
        for (int cc = 0; cc < nch; cc += 2) {
            step(oa, ob, cc, 0);
            step(ob, oa, cc + 1, 1);
        }
        return;
    }

    // ---- state waves
    const bool has_u = w < SH::NU;
    float* pool_h = p.pool + ((int64_t)slot * p.HV + h) * (int64_t)V * K + (int64_t)(col0 + l16) * K + 4 * sub;
    f32x4m S[SH::SPW];
#pragma unroll
    for (int si = 0; si < SH::SPW; ++si) {
        const int t = w + 4 * si;
        S[si] = f32x4m{0.f, 0.f, 0.f, 0.f};
        if (t < SH::NS) {
            const float4 v = *reinterpret_cast<const float4*>(pool_h + 16 * t);
            S[si] = f32x4m{v.x, v.y, v.z, v.w};
        }
    }
    if (nch <= 0) return;                            // empty sequence: the slot keeps its state
    auto load_u = [&](StateOps<C, K>& o, int cc) {
        if (!has_u) return;
        const float* ws = chunk(cc);
        load_runs<SH::KQ>(o.w, ws + (int64_t)w * SH::KQ * 64, lane);
        const float4 u = *reinterpret_cast<const float4*>(ws + OFF_UP + ws_tile(16 * w + 4 * sub, col0 + l16, V));
        o.up[0] = u.x; o.up[1] = u.y; o.up[2] = u.z; o.up[3] = u.w;
    };
    auto load_s = [&](StateOps<C, K>& o, int cc) {
        const float* ws = chunk(cc);
#pragma unroll
        for (int si = 0; si < SH::SPW; ++si) {
            const int t = w + 4 * si;
            if (t < SH::NS) {
                load_runs<SH::CQ>(o.kt[si], ws + OFF_KT + (int64_t)t * SH::CQ * 64, lane);
                o.gl[si] = *reinterpret_cast<const float4*>(ws + OFF_GL + 16 * t + 4 * sub);
            }
        }
    };
    auto step = [&](const StateOps<C, K>& o, StateOps<C, K>& nx, int cc, int buf) {
        const bool live = cc < nch;
        const int nxt = min(cc + 1, nch - 1);
#pragma unroll
        for (int si = 0; si < SH::SPW; ++si) {
            const int t = w + 4 * si;
            if (t < SH::NS) {
                if (kInter && live) {
                    float* dst = p.inter + ((int64_t)(cstart + cc) * p.HV + h) * (int64_t)V * K +
                                 (int64_t)(col0 + l16) * K + 16 * t + 4 * sub;
                    *reinterpret_cast<float4*>(dst) = make_float4(S[si][0], S[si][1], S[si][2], S[si][3]);
                }
                *reinterpret_cast<float4*>(&sS[buf][l16 * SH::LDS_S + 16 * t + 4 * sub]) =
                    make_float4(S[si][0], S[si][1], S[si][2], S[si][3]);
            }
        }
        lds_barrier();                                  // S of chunk cc published
        if (has_u) {
            // U = U' - W S, rows 16 w .. 16 w + 15 (four independent chains)
            f32x4m a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0, a3 = a0;
            const float* srow = &sS[buf][l16 * SH::LDS_S + SH::KQ * sub];
#pragma unroll
            for (int j = 0; j < SH::KQ; j += 4) {
                const float4 sv = *reinterpret_cast<const float4*>(srow + j);
                a0 = mfma_f32(o.w[j], sv.x, a0);
                a1 = mfma_f32(o.w[j + 1], sv.y, a1);
                a2 = mfma_f32(o.w[j + 2], sv.z, a2);
                a3 = mfma_f32(o.w[j + 3], sv.w, a3);
            }
            const f32x4m ws4 = (a0 + a1) + (a2 + a3);
            const float4 u = make_float4(o.up[0] - ws4[0], o.up[1] - ws4[1], o.up[2] - ws4[2], o.up[3] - ws4[3]);
            *reinterpret_cast<float4*>(&sU[buf][l16 * SH::LDS_U + 16 * w + 4 * sub]) = u;
            load_u(nx, nxt);
        }
        lds_barrier();                                  // U of chunk cc published
        // S <- e^G_last * S + Kt^T U
        const float* urow = &sU[buf][l16 * SH::LDS_U + SH::CQ * sub];
        float4 uv[SH::CQ / 4];
#pragma unroll
        for (int q = 0; q < SH::CQ / 4; ++q) uv[q] = *reinterpret_cast<const float4*>(urow + 4 * q);
#pragma unroll
        for (int si = 0; si < SH::SPW; ++si) {
            const int t = w + 4 * si;
            if (t < SH::NS) {
                f32x4m a0 = {S[si][0] * o.gl[si].x, S[si][1] * o.gl[si].y, S[si][2] * o.gl[si].z,
                             S[si][3] * o.gl[si].w};
                f32x4m a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < SH::CQ / 4; ++q) {
                    a0 = mfma_f32(o.kt[si][4 * q], uv[q].x, a0);
                    a1 = mfma_f32(o.kt[si][4 * q + 1], uv[q].y, a1);
                    a0 = mfma_f32(o.kt[si][4 * q + 2], uv[q].z, a0);
                    a1 = mfma_f32(o.kt[si][4 * q + 3], uv[q].w, a1);
                }
                if (live) S[si] = a0 + a1;
            }
        }
        load_s(nx, nxt);
    };
    StateOps<C, K> oa, ob;
    load_u(oa, 0);
    load_s(oa, 0);
    // steps in pairs (two operand sets); for an odd count the last step of
    // the last pair re-reads the last chunk, keeps S and stores nothing
    for (int cc = 0; cc < nch; cc += 2) {
        step(oa, ob, cc, 0);
        step(ob, oa, cc + 1, 1);
    }
#pragma unroll
    for (int si = 0; si < SH::SPW; ++si) {
        const int t = w + 4 * si;
        if (t < SH::NS)
            *reinterpret_cast<float4*>(pool_h + 16 * t) = make_float4(S[si][0], S[si][1], S[si][2], S[si][3]);
    }
}

}  // namespace

template <typename TIn, int C, int K, int V>
hipError_t launch_scan32(const kda_prefill_args& a, const PrefillParams& p, hipStream_t s) {
    const int64_t nblk = a.num_seqs * a.HV * (V / 16);
    if (p.inter)
        klaunch(scan32_kernel<TIn, C, K, V, true>, dim3(static_cast<unsigned>(nblk)), dim3(64 * kScan32Waves), 0, s, p);
    else
        klaunch(scan32_kernel<TIn, C, K, V, false>, dim3(static_cast<unsigned>(nblk)), dim3(64 * kScan32Waves), 0, s, p);
    return hipGetLastError();
}

#define KDA_SCAN32(T, C, K, V) template hipError_t launch_scan32<T, C, K, V>(const kda_prefill_args&, const PrefillParams&, hipStream_t);
#define KDA_SCAN32_V(T, C, K) KDA_SCAN32(T, C, K, 32) KDA_SCAN32(T, C, K, 64) KDA_SCAN32(T, C, K, 128)
#define KDA_SCAN32_K(T, C) KDA_SCAN32_V(T, C, 32) KDA_SCAN32_V(T, C, 64) KDA_SCAN32_V(T, C, 128)
KDA_SCAN32_K(float, 16) KDA_SCAN32_K(float, 64) KDA_SCAN32_K(bf16, 16) KDA_SCAN32_K(bf16, 64)
#undef KDA_SCAN32_K
#undef KDA_SCAN32_V
#undef KDA_SCAN32

}  // namespace kda
