// Prep of the general prefill path on fp32 matrix tiles (v_mfma_f32_16x16x4f32)
// for chunk C = 64 and K, V in {32, 64, 128}: one block of 4 waves per
// chunk x head.  (The chunk-16 prep, one wave per chunk x head, follows it.)
// It writes the general path's workspace (row-major fp32 W, U', P, Qt, Kt
// and e^G_last), which the fp32 scan then reads.
//
// 1. per row (wave s: rows 16 s .. 16 s + 15; lane (l16, g): row 16 s + l16,
//    key channels K/4 g .. K/4 g + K/4 - 1, value channels likewise): q, k,
//    gate and beta; the L2 norms.
// 2. G = in-chunk cumulative log-decay (base-2 units): an inclusive scan
//    over the 16 rows of each wave (DPP row shifts), then the totals of the
//    waves before through LDS.
// 3. with the reference row m = 16 s + 7 of the row block,
//      E1 = e^(G_r - G_m), E2 = e^(G_m - G_r)
//    give the Gram operands q-hat E1, k-hat E1 (row side) and k-hat E2 (key
//    side), and with per-channel factors
//      Qt = q-hat E1 e^G_m, R = k-hat E1 e^G_m, Kt = k-hat E2 e^(G_last - G_m).
// 4. gated Grams: block (s, u) is one product over the K channels of row
//    block s's operands and key block u's, the latter rescaled per channel
//    from u's reference row to m(s) (through u's last row, so no factor
//    underflows where the operand is large); P -> workspace, A -> LDS.
// 5. (I + A)^-1: 16 x 16 diagonal blocks by substitution (one per wave),
//    then two levels of block merges.
// 6. W = Tm diag(beta) R and U' = Tm diag(beta) V, column tiles dealt
//    round robin over the waves.
// A chunk whose factors could leave the float32 range (a decay span above
// 80 inside half a block, or any g > 0) is flagged and left to the exact
// per-element prep, launched after this one for the flagged chunks only.

#include "kda_prefill_common.h"

namespace kda {
namespace {

typedef float f32x4p __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4p mfma32(float a, float b, f32x4p c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

constexpr float kLog2eP = 1.4426950408889634f;
constexpr float kMaxSpanP2 = 80.0f * kLog2eP;       // largest |G_r - G_m| of the fast path (base 2)

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// N (a multiple of 8) consecutive elements of a row as float: 16-byte loads
// when every row of the tensor is 16-byte aligned (kVec), element loads
// otherwise.
template <bool kVec, int N>
__device__ __forceinline__ void load_row(float* dst, const float* src, bool valid) {
    if constexpr (kVec) {
#pragma unroll
        for (int j = 0; j < N; j += 4) {
            const float4 v = valid ? *reinterpret_cast<const float4*>(src + j) : make_float4(0.f, 0.f, 0.f, 0.f);
            dst[j] = v.x; dst[j + 1] = v.y; dst[j + 2] = v.z; dst[j + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < N; ++j) dst[j] = valid ? src[j] : 0.0f;
    }
}
template <bool kVec, int N>
__device__ __forceinline__ void load_row(float* dst, const bf16* src, bool valid) {
    if constexpr (kVec) {
#pragma unroll
        for (int j = 0; j < N; j += 8) {
            const uint4 u = valid ? *reinterpret_cast<const uint4*>(src + j) : make_uint4(0, 0, 0, 0);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dst[j + 2 * e] = __uint_as_float(w[e] << 16);
                dst[j + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < N; ++j) dst[j] = valid ? ld(src, j) : 0.0f;
    }
}

// x from the lane `off` rows earlier in the same 16-lane row, 0 for the first lanes.
template <int kCtrl>
__device__ __forceinline__ float row_shift(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}

template <typename TIn, bool kVec, int K, int V>
__global__ __launch_bounds__(256, 1) void prep32_kernel(const PrefillParams p) {
    constexpr int C = 64;
    constexpr int NCH = K / 4, NVC = V / 4;  // key and value channels per lane
    constexpr int NQ = NCH / 4;              // float4 of key operand per lane
    constexpr int LDA = C + 1;              // A and Tm row stride (floats)
    constexpr int LDR = K + 4;              // staged R rows (floats); 16-byte rows, groups on distinct banks
    constexpr int LDV = V + 4;              // staged V rows
    constexpr int KEYS = 3 * NCH * 64;      // key operands of blocks 0..2 (floats)
    constexpr int XF = KEYS + 9 * K > C * LDV ? KEYS + 9 * K : C * LDV;
    static_assert(K % 32 == 0 && V % 32 == 0 && K <= 128 && V <= 128, "channel split");
    __shared__ __attribute__((aligned(16))) float s_X[XF];        // key operands + factor tables; then V rows
    __shared__ __attribute__((aligned(16))) float s_R[C * LDR];   // R rows
    __shared__ float s_A[C * LDA];
    __shared__ float s_T[C * LDA];
    __shared__ __attribute__((aligned(16))) float s_tot[4 * K];   // per-wave totals of g
    __shared__ __attribute__((aligned(16))) float s_gref[4 * 2 * K];   // G at rows 16 s + 7 and 16 s + 15
    __shared__ float s_beta[C];
    __shared__ int s_flag[4];

    const int item = blockIdx.x;
    const int h = item % p.HV;
    const int ci = item / p.HV;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int sub = lane >> 4, l16 = lane & 15;

    int b, t0, len;
    if (p.cu) {
        int n, cstart;
        if (!locate_chunk(p.cu, p.num_seqs, p.T, C, ci, n, cstart)) return;
        b = 0;
        t0 = cu_at(p.cu, n, p.T) + (ci - cstart) * C;
        len = min(C, cu_at(p.cu, n, p.T) + seq_len(p.cu, n, p.T) - t0);
    } else {
        const int cpb = ceil_div(p.T, C);
        b = ci / cpb;
        t0 = (ci % cpb) * C;
        len = min(C, p.T - t0);
    }
    float* ws = p.ws + ((int64_t)ci * p.HV + h) * p.chunk_floats;
    float* gW = ws;
    float* gUp = gW + C * K;
    float* gP = gUp + C * V;
    float* gQt = gP + C * C;
    float* gKt = gQt + C * K;
    float* gGl = gKt + C * K;

    // ---- 1. rows
    const int ra = 16 * wave + l16;
    const int c0 = NCH * sub, cv0 = NVC * sub;
    const bool valid = ra < len;
    const int64_t t = t0 + min(ra, len - 1);
    const int hq = h / p.group;
    const TIn* qg = static_cast<const TIn*>(p.q) + b * p.qs[0] + hq * p.qs[2] + t * p.qs[1] + c0;
    const TIn* kg = static_cast<const TIn*>(p.k) + b * p.ks[0] + hq * p.ks[2] + t * p.ks[1] + c0;
    const TIn* gg = static_cast<const TIn*>(p.g) + b * p.gs[0] + h * p.gs[2] + t * p.gs[1] + c0;
    const TIn* vg = static_cast<const TIn*>(p.v) + b * p.vs[0] + h * p.vs[2] + t * p.vs[1] + cv0;
    float qv[NCH], kv[NCH], G[NCH];
    load_row<kVec, NCH>(qv, qg, valid);
    load_row<kVec, NCH>(kv, kg, valid);
    load_row<kVec, NCH>(G, gg, valid);
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        sq = fmaf(qv[j], qv[j], sq);
        sk = fmaf(kv[j], kv[j], sk);
    }
    sq += __shfl_xor(sq, 16, 64);
    sq += __shfl_xor(sq, 32, 64);
    sk += __shfl_xor(sk, 16, 64);
    sk += __shfl_xor(sk, 32, 64);
    const float rq = p.l2norm ? rsqrtf(sq + kL2Eps) : 1.0f, rk = p.l2norm ? rsqrtf(sk + kL2Eps) : 1.0f;
    const int gmode = p.gate;
    const float expA = gmode != kGateRaw ? __expf(p.A_log[h]) : 0.0f;
    bool unsafe = false;
    float dtv[NCH];
    if (p.dt_bias) load_row<true, NCH>(dtv, p.dt_bias + h * K + c0, true);    // dt_bias rows are 16-byte aligned
    else {
#pragma unroll
        for (int j = 0; j < NCH; ++j) dtv[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        qv[j] *= rq;
        kv[j] *= rk;
        const float gl = valid ? log_gate(G[j], gmode, expA, dtv[j], p.lb) * kLog2eP : 0.0f;
        unsafe |= gl > 0.0f;
        G[j] = gl;
    }
    if (sub == 0) {
        const TIn* bg = static_cast<const TIn*>(p.beta) + b * p.bs[0] + h + t * p.bs[1];
        float bt = valid ? ld(bg, 0) : 0.0f;
        if (valid && p.beta_is_raw) bt = sigmoidf(bt);
        s_beta[ra] = bt;
    }

    // ---- 2. cumulative G: rows of this wave, then the waves before
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        float x = G[j];
        x += row_shift<0x111>(x);
        x += row_shift<0x112>(x);
        x += row_shift<0x114>(x);
        x += row_shift<0x118>(x);
        G[j] = x;
    }
    if (l16 == 15) {
#pragma unroll
        for (int j = 0; j < NCH; j += 4)
            *reinterpret_cast<float4*>(&s_tot[wave * K + c0 + j]) = make_float4(G[j], G[j + 1], G[j + 2], G[j + 3]);
    }
    lds_barrier();
    float glast[NCH];
#pragma unroll
    for (int j = 0; j < NCH; j += 4) {
        float4 off = make_float4(0.f, 0.f, 0.f, 0.f), all = off;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
            const float4 tv = *reinterpret_cast<const float4*>(&s_tot[w2 * K + c0 + j]);
            if (w2 < wave) { off.x += tv.x; off.y += tv.y; off.z += tv.z; off.w += tv.w; }
            all.x += tv.x; all.y += tv.y; all.z += tv.z; all.w += tv.w;
        }
        G[j] += off.x; G[j + 1] += off.y; G[j + 2] += off.z; G[j + 3] += off.w;
        glast[j] = all.x; glast[j + 1] = all.y; glast[j + 2] = all.z; glast[j + 3] = all.w;
    }
    if (l16 == 7 || l16 == 15) {
        float* dst = &s_gref[(2 * wave + (l16 == 15)) * K + c0];
#pragma unroll
        for (int j = 0; j < NCH; j += 4)
            *reinterpret_cast<float4*>(dst + j) = make_float4(G[j], G[j + 1], G[j + 2], G[j + 3]);
    }
    if (wave == 0 && l16 == 0) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) gGl[c0 + j] = ex2(glast[j]);
    }
    // V rows of this lane (staged after the Grams)
    float vv[NVC];
    load_row<kVec, NVC>(vv, vg, valid);
    lds_barrier();

    // factor tables for the off-diagonal Gram blocks (after the key operands in s_X)
    float* s_f = s_X + KEYS;                 // [3][K]  f(u) = e^(G_l(u) - G_m(u))
    float* s_d = s_f + 3 * K;                // [6][K]  d(s, u) = e^(G_m(s) - G_l(u))
    for (int e = tid; e < 9 * K; e += 256) {
        const int c = e % K, r = e / K;
        if (r < 3) {
            s_f[r * K + c] = ex2(s_gref[(2 * r + 1) * K + c] - s_gref[(2 * r) * K + c]);
        } else {
            const int pr = r - 3;                              // pair s (s - 1) / 2 + u
            const int sb = pr < 1 ? 1 : (pr < 3 ? 2 : 3);
            const int u = pr - sb * (sb - 1) / 2;
            s_d[pr * K + c] = ex2(s_gref[(2 * sb) * K + c] - s_gref[(2 * u + 1) * K + c]);
        }
    }

    // ---- 3. operands
    float aq[NCH], ak[NCH], bk[NCH];
    {
        const float* gm = &s_gref[(2 * wave) * K + c0];
#pragma unroll
        for (int j = 0; j < NCH; j += 4) {
            const float4 m4 = *reinterpret_cast<const float4*>(gm + j);
            const float mv[4] = {m4.x, m4.y, m4.z, m4.w};
            float qt[4], kt[4], rr[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float dl = G[j + e] - mv[e];
                unsafe |= fabsf(dl) > kMaxSpanP2;
                const float e1 = ex2(dl), e2 = ex2(-dl);
                const float egm = ex2(mv[e]), eglm = ex2(glast[j + e] - mv[e]);
                aq[j + e] = qv[j + e] * e1;
                ak[j + e] = kv[j + e] * e1;
                bk[j + e] = kv[j + e] * e2;
                qt[e] = aq[j + e] * egm;
                rr[e] = ak[j + e] * egm;
                kt[e] = bk[j + e] * eglm;
            }
            *reinterpret_cast<float4*>(&gQt[ws_run(ra, c0 + j, K)]) = make_float4(qt[0], qt[1], qt[2], qt[3]);
#pragma unroll
            for (int e = 0; e < 4; ++e) gKt[ws_run(c0 + j + e, ra, C)] = kt[e];     // Kt^T
            *reinterpret_cast<float4*>(&s_R[ra * LDR + c0 + j]) = make_float4(rr[0], rr[1], rr[2], rr[3]);
        }
        if (wave < 3) {
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                *reinterpret_cast<float4*>(&s_X[((wave * NQ + q) * 64 + lane) * 4]) =
                    make_float4(bk[4 * q], bk[4 * q + 1], bk[4 * q + 2], bk[4 * q + 3]);
        }
        const int any = __ballot(unsafe) != 0 ? 1 : 0;
        if (lane == 0) s_flag[wave] = any;
    }
    lds_barrier();
    const bool block_unsafe = (s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3]) != 0;
    if (tid == 0) p.flags[item] = block_unsafe ? 1 : 0;
    if (block_unsafe) return;                 // every wave leaves here: the exact prep redoes the chunk

    // ---- 4. gated Grams; wave s: row block s against key blocks u <= s
    {
        const int s = wave;
        for (int nt = 0; nt < 4; ++nt) {
            f32x4p p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0, a0 = p0, a1 = p0;
            if (nt <= s) {
                if (nt == s) {
#pragma unroll
                    for (int j = 0; j < NCH; j += 2) {
                        p0 = mfma32(aq[j], bk[j], p0);
                        a0 = mfma32(ak[j], bk[j], a0);
                        p1 = mfma32(aq[j + 1], bk[j + 1], p1);
                        a1 = mfma32(ak[j + 1], bk[j + 1], a1);
                    }
                } else {
                    const float* fp = s_f + nt * K + c0;
                    const float* dp = s_d + (s * (s - 1) / 2 + nt) * K + c0;
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        const float4 kb = *reinterpret_cast<const float4*>(&s_X[((nt * NQ + q) * 64 + lane) * 4]);
                        const float4 f4 = *reinterpret_cast<const float4*>(fp + 4 * q);
                        const float4 d4 = *reinterpret_cast<const float4*>(dp + 4 * q);
                        const float bv[4] = {(kb.x * f4.x) * d4.x, (kb.y * f4.y) * d4.y,
                                             (kb.z * f4.z) * d4.z, (kb.w * f4.w) * d4.w};
                        p0 = mfma32(aq[4 * q], bv[0], p0);
                        a0 = mfma32(ak[4 * q], bv[0], a0);
                        p1 = mfma32(aq[4 * q + 1], bv[1], p1);
                        a1 = mfma32(ak[4 * q + 1], bv[1], a1);
                        p0 = mfma32(aq[4 * q + 2], bv[2], p0);
                        a0 = mfma32(ak[4 * q + 2], bv[2], a0);
                        p1 = mfma32(aq[4 * q + 3], bv[3], p1);
                        a1 = mfma32(ak[4 * q + 3], bv[3], a1);
                    }
                }
            }
            // lane (l16, sub) holds rows 16 s + 4 sub + i of column 16 nt + l16
            const int j = 16 * nt + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * s + 4 * sub + i;
                gP[ws_run(r, j, C)] = j <= r ? p0[i] + p1[i] : 0.0f;
                s_A[r * LDA + j] = j < r ? s_beta[r] * (a0[i] + a1[i]) : 0.0f;
            }
        }
    }
    lds_barrier();

    // ---- 5. (I + A)^-1: diagonal blocks by forward substitution, one per
    //         wave (lane (c, sub) solves column c, keeps rows 4 sub .. + 3);
    //         V rows into s_X meanwhile (the key operands are no longer read)
#pragma unroll
    for (int j = 0; j < NVC; j += 4)
        *reinterpret_cast<float4*>(&s_X[ra * LDV + cv0 + j]) = make_float4(vv[j], vv[j + 1], vv[j + 2], vv[j + 3]);
    {
        const int d0 = 16 * wave;
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float acc = rr == l16 ? 1.0f : 0.0f;
#pragma unroll
            for (int tt = 0; tt < rr; ++tt) acc = fmaf(-s_A[(d0 + rr) * LDA + d0 + tt], x[tt], acc);
            x[rr] = acc;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = sub == 0 ? x[i] : sub == 1 ? x[4 + i] : sub == 2 ? x[8 + i] : x[12 + i];
            s_T[(d0 + 4 * sub + i) * LDA + d0 + l16] = v;
        }
    }
    lds_barrier();
    // blocks below the diagonal: the inverse of [[L1, 0], [B, L2]] has the
    // lower left block -L2^-1 B L1^-1; a product whose right operand is a
    // previous result takes it from registers (k-step j: row 4 sub + j)
    auto prod_at = [&](int rb, int ub, int cb, f32x4p acc) {      // += A[rb][ub] T[ub][cb]
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kk = 4 * j + sub;
            acc = mfma32(s_A[(16 * rb + l16) * LDA + 16 * ub + kk], s_T[(16 * ub + kk) * LDA + 16 * cb + l16], acc);
        }
        return acc;
    };
    auto prod_treg = [&](int rb, int mb, f32x4p y, f32x4p acc) {  // += T[rb][mb] Y
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mfma32(s_T[(16 * rb + l16) * LDA + 16 * mb + 4 * sub + j], y[j], acc);
        return acc;
    };
    auto store_neg = [&](int rb, int cb, f32x4p x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s_T[(16 * rb + 4 * sub + i) * LDA + 16 * cb + l16] = -x[i];
    };
    if (wave & 1) {
        const f32x4p zero = {0.f, 0.f, 0.f, 0.f};
        const f32x4p y = prod_at(wave, wave - 1, wave - 1, zero);
        store_neg(wave, wave - 1, prod_treg(wave, wave, y, zero));
    }
    lds_barrier();
    {
        const int rb = 2 + (wave >> 1), cb = wave & 1;
        const f32x4p zero = {0.f, 0.f, 0.f, 0.f};
        f32x4p x = zero;
        for (int m = 2; m <= rb; ++m) {
            f32x4p y = zero;
            for (int u = cb; u < 2; ++u) y = prod_at(m, u, cb, y);
            x = prod_treg(rb, m, y, x);
        }
        store_neg(rb, cb, x);
    }
    lds_barrier();

    // ---- 6. W = Tm diag(beta) R, U' = Tm diag(beta) V: column tiles
    //         w, w + 4, ... of each, every row block (k-step j: token
    //         4 j + sub; Tm is lower triangular, so row block mt needs
    //         4 (mt + 1) steps)
    // the tile goes to W as row runs, to U' as a whole accumulator tile
    auto tile = [&](const float* src, int ld, int nt, int mt, const float (&tb)[16], bool to_w) {
        f32x4p a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
        for (int j = 0; j < 4 * (mt + 1); j += 2) {
            const int k0 = 4 * j + sub, k1 = k0 + 4;
            a0 = mfma32(tb[j], src[k0 * ld + 16 * nt + l16], a0);
            a1 = mfma32(tb[j + 1], src[k1 * ld + 16 * nt + l16], a1);
        }
        if (to_w) {
#pragma unroll
            for (int i = 0; i < 4; ++i) gW[ws_run(16 * mt + 4 * sub + i, 16 * nt + l16, K)] = a0[i] + a1[i];
        } else {
            *reinterpret_cast<float4*>(&gUp[ws_tile(16 * mt + 4 * sub, 16 * nt + l16, V)]) =
                make_float4(a0[0] + a1[0], a0[1] + a1[1], a0[2] + a1[2], a0[3] + a1[3]);
        }
    };
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        float tb[16];
#pragma unroll
        for (int j = 0; j < 4 * (mt + 1); ++j) {
            const int kk = 4 * j + sub;
            tb[j] = s_T[(16 * mt + l16) * LDA + kk] * s_beta[kk];
        }
#pragma unroll
        for (int n2 = 0; n2 < (K / 16 + 3) / 4; ++n2)
            if (wave + 4 * n2 < K / 16) tile(s_R, LDR, wave + 4 * n2, mt, tb, true);
#pragma unroll
        for (int n2 = 0; n2 < (V / 16 + 3) / 4; ++n2)
            if (wave + 4 * n2 < V / 16) tile(s_X, LDV, wave + 4 * n2, mt, tb, false);
    }
}

// LDS hand-off between the lanes of one wave: a wave's LDS operations
// complete in order, so only the compiler's reordering needs a fence.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Prep of the general path at chunk C = 16 on fp32 matrix tiles: one wave
// per (chunk, head) item, four items per block.  The chunk-64 prep's steps
// for a single 16-row block, all inside the wave: rows (lane (l16, g): row
// l16, K/4 key and V/4 value channels), the cumulative log-decay by DPP row
// shifts, the reference row 7 (E1 = e^(G_r - G_7), E2 = e^(G_7 - G_r)), the
// Grams as one tile product, (I + A)^-1 by substitution, W and U' as column
// tiles.  Chunks whose factors could leave the float32 range are flagged to
// the exact prep, as at chunk 64.
template <typename TIn, bool kVec, int K, int V>
__global__ __launch_bounds__(256) void prep16_kernel(const PrefillParams p) {
    constexpr int C = 16;
    constexpr int NCH = K / 4, NVC = V / 4;  // key and value channels per lane
    constexpr int LDA = C + 1;
    constexpr int LDR = K + 4, LDV = V + 4;
    struct WaveLds {
        float R[C * LDR];                    // R rows
        float Vr[C * LDV];                   // V rows
        float A[C * LDA];                    // beta-scaled strict lower A
        float T[C * LDA];                    // (I + A)^-1
        float gref[2 * K];                   // G at rows 7 and 15
        float beta[C];
    };
    __shared__ __attribute__((aligned(16))) WaveLds sw[4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int sub = lane >> 4, l16 = lane & 15;
    WaveLds& L = sw[wave];
    const int64_t item = (int64_t)blockIdx.x * 4 + wave;
    if (item >= (int64_t)p.max_chunks * p.HV) return;      // per wave: nothing below waits for the block
    const int h = static_cast<int>(item % p.HV);
    const int ci = static_cast<int>(item / p.HV);

    int b, t0, len;
    if (p.cu) {
        int n, cstart;
        if (!locate_chunk(p.cu, p.num_seqs, p.T, C, ci, n, cstart)) return;
        b = 0;
        t0 = cu_at(p.cu, n, p.T) + (ci - cstart) * C;
        len = min(C, cu_at(p.cu, n, p.T) + seq_len(p.cu, n, p.T) - t0);
    } else {
        const int cpb = ceil_div(p.T, C);
        b = ci / cpb;
        t0 = (ci % cpb) * C;
        len = min(C, p.T - t0);
    }
    float* ws = p.ws + (int64_t)item * p.chunk_floats;
    float* gW = ws;
    float* gUp = gW + C * K;
    float* gP = gUp + C * V;
    float* gQt = gP + C * C;
    float* gKt = gQt + C * K;
    float* gGl = gKt + C * K;

    // ---- 1. rows, norms, gate map, beta
    const int ra = l16;
    const int c0 = NCH * sub, cv0 = NVC * sub;
    const bool valid = ra < len;
    const int64_t t = t0 + min(ra, len - 1);
    const int hq = h / p.group;
    const TIn* qg = static_cast<const TIn*>(p.q) + b * p.qs[0] + hq * p.qs[2] + t * p.qs[1] + c0;
    const TIn* kg = static_cast<const TIn*>(p.k) + b * p.ks[0] + hq * p.ks[2] + t * p.ks[1] + c0;
    const TIn* gg = static_cast<const TIn*>(p.g) + b * p.gs[0] + h * p.gs[2] + t * p.gs[1] + c0;
    const TIn* vg = static_cast<const TIn*>(p.v) + b * p.vs[0] + h * p.vs[2] + t * p.vs[1] + cv0;
    float qv[NCH], kv[NCH], G[NCH], vv[NVC];
    load_row<kVec, NCH>(qv, qg, valid);
    load_row<kVec, NCH>(kv, kg, valid);
    load_row<kVec, NCH>(G, gg, valid);
    load_row<kVec, NVC>(vv, vg, valid);
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        sq = fmaf(qv[j], qv[j], sq);
        sk = fmaf(kv[j], kv[j], sk);
    }
    sq += __shfl_xor(sq, 16, 64);
    sq += __shfl_xor(sq, 32, 64);
    sk += __shfl_xor(sk, 16, 64);
    sk += __shfl_xor(sk, 32, 64);
    const float rq = p.l2norm ? rsqrtf(sq + kL2Eps) : 1.0f, rk = p.l2norm ? rsqrtf(sk + kL2Eps) : 1.0f;
    const int gmode = p.gate;
    const float expA = gmode != kGateRaw ? __expf(p.A_log[h]) : 0.0f;
    bool unsafe = false;
    float dtv[NCH];
    if (p.dt_bias) load_row<true, NCH>(dtv, p.dt_bias + h * K + c0, true);    // dt_bias rows are 16-byte aligned
    else {
#pragma unroll
        for (int j = 0; j < NCH; ++j) dtv[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        qv[j] *= rq;
        kv[j] *= rk;
        const float gl = valid ? log_gate(G[j], gmode, expA, dtv[j], p.lb) * kLog2eP : 0.0f;
        unsafe |= gl > 0.0f;
        G[j] = gl;
    }
    if (sub == 0) {
        const TIn* bg = static_cast<const TIn*>(p.beta) + b * p.bs[0] + h + t * p.bs[1];
        float bt = valid ? ld(bg, 0) : 0.0f;
        if (valid && p.beta_is_raw) bt = sigmoidf(bt);
        L.beta[ra] = bt;
    }

    // ---- 2. cumulative G over the 16 rows; rows 7 and 15 to LDS
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        float x = G[j];
        x += row_shift<0x111>(x);
        x += row_shift<0x112>(x);
        x += row_shift<0x114>(x);
        x += row_shift<0x118>(x);
        G[j] = x;
    }
    if (l16 == 7 || l16 == 15) {
        float* dst = &L.gref[(l16 == 15 ? K : 0) + c0];
#pragma unroll
        for (int j = 0; j < NCH; j += 4)
            *reinterpret_cast<float4*>(dst + j) = make_float4(G[j], G[j + 1], G[j + 2], G[j + 3]);
    }
    wave_lds_sync();

    // ---- 3. operands: Gram operands, Qt and Kt to the workspace, R and V rows to LDS
    float aq[NCH], ak[NCH], bk[NCH];
#pragma unroll
    for (int j = 0; j < NCH; j += 4) {
        const float4 m4 = *reinterpret_cast<const float4*>(&L.gref[c0 + j]);
        const float4 l4 = *reinterpret_cast<const float4*>(&L.gref[K + c0 + j]);
        const float mv[4] = {m4.x, m4.y, m4.z, m4.w}, lv[4] = {l4.x, l4.y, l4.z, l4.w};
        float qt[4], kt[4], rr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float dl = G[j + e] - mv[e];
            unsafe |= fabsf(dl) > kMaxSpanP2;
            const float e1 = ex2(dl), e2 = ex2(-dl);
            const float egm = ex2(mv[e]), eglm = ex2(lv[e] - mv[e]);
            aq[j + e] = qv[j + e] * e1;
            ak[j + e] = kv[j + e] * e1;
            bk[j + e] = kv[j + e] * e2;
            qt[e] = aq[j + e] * egm;
            rr[e] = ak[j + e] * egm;
            kt[e] = bk[j + e] * eglm;
        }
        *reinterpret_cast<float4*>(&gQt[ws_run(ra, c0 + j, K)]) = make_float4(qt[0], qt[1], qt[2], qt[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) gKt[ws_run(c0 + j + e, ra, C)] = kt[e];         // Kt^T
        *reinterpret_cast<float4*>(&L.R[ra * LDR + c0 + j]) = make_float4(rr[0], rr[1], rr[2], rr[3]);
        if (l16 == 0) {
            *reinterpret_cast<float4*>(&gGl[c0 + j]) = make_float4(ex2(lv[0]), ex2(lv[1]), ex2(lv[2]), ex2(lv[3]));
        }
    }
#pragma unroll
    for (int j = 0; j < NVC; j += 4)
        *reinterpret_cast<float4*>(&L.Vr[ra * LDV + cv0 + j]) = make_float4(vv[j], vv[j + 1], vv[j + 2], vv[j + 3]);
    const bool any_unsafe = __ballot(unsafe) != 0;
    if (lane == 0) p.flags[item] = any_unsafe ? 1 : 0;
    if (any_unsafe) return;                  // the exact prep redoes this chunk

    // ---- 4. Grams: one tile product over the K channels
    {
        f32x4p p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0, a0 = p0, a1 = p0;
#pragma unroll
        for (int j = 0; j < NCH; j += 2) {
            p0 = mfma32(aq[j], bk[j], p0);
            a0 = mfma32(ak[j], bk[j], a0);
            p1 = mfma32(aq[j + 1], bk[j + 1], p1);
            a1 = mfma32(ak[j + 1], bk[j + 1], a1);
        }
        // lane (l16, sub) holds rows 4 sub + i of column l16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * sub + i;
            gP[ws_run(r, l16, C)] = l16 <= r ? p0[i] + p1[i] : 0.0f;
            L.A[r * LDA + l16] = l16 < r ? L.beta[r] * (a0[i] + a1[i]) : 0.0f;
        }
    }
    wave_lds_sync();

    // ---- 5. (I + A)^-1 by forward substitution: lane (c, sub) solves column
    //         c and keeps rows 4 sub .. 4 sub + 3
    {
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float acc = rr == l16 ? 1.0f : 0.0f;
#pragma unroll
            for (int tt = 0; tt < rr; ++tt) acc = fmaf(-L.A[rr * LDA + tt], x[tt], acc);
            x[rr] = acc;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = sub == 0 ? x[i] : sub == 1 ? x[4 + i] : sub == 2 ? x[8 + i] : x[12 + i];
            L.T[(4 * sub + i) * LDA + l16] = v;
        }
    }
    wave_lds_sync();

    // ---- 6. W = Tm diag(beta) R and U' = Tm diag(beta) V (k-step j: token 4 j + sub)
    float tb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int kk = 4 * j + sub;
        tb[j] = L.T[l16 * LDA + kk] * L.beta[kk];
    }
    // the tile goes to W as row runs, to U' as a whole accumulator tile
    auto tile = [&](const float* src, int ld, int nt, bool to_w) {
        f32x4p a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
            const int k0 = 4 * j + sub, k1 = k0 + 4;
            a0 = mfma32(tb[j], src[k0 * ld + 16 * nt + l16], a0);
            a1 = mfma32(tb[j + 1], src[k1 * ld + 16 * nt + l16], a1);
        }
        if (to_w) {
#pragma unroll
            for (int i = 0; i < 4; ++i) gW[ws_run(4 * sub + i, 16 * nt + l16, K)] = a0[i] + a1[i];
        } else {
            *reinterpret_cast<float4*>(&gUp[ws_tile(4 * sub, 16 * nt + l16, V)]) =
                make_float4(a0[0] + a1[0], a0[1] + a1[1], a0[2] + a1[2], a0[3] + a1[3]);
        }
    };
#pragma unroll
    for (int nt = 0; nt < K / 16; ++nt) tile(L.R, LDR, nt, true);
#pragma unroll
    for (int nt = 0; nt < V / 16; ++nt) tile(L.Vr, LDV, nt, false);
}

}  // namespace

template <typename TIn, int K, int V>
hipError_t launch_prep32(const kda_prefill_args& a, const PrefillParams& p, hipStream_t s) {
    const int64_t items = prefill_max_chunks(a) * a.HV;
    const int elem = sizeof(TIn);
    const bool vec = aligned_rows(a.q, a.q_stride, 3, elem) && aligned_rows(a.k, a.k_stride, 3, elem) &&
                     aligned_rows(a.g, a.g_stride, 3, elem) && aligned_rows(a.v, a.v_stride, 3, elem);
    if (vec) klaunch(prep32_kernel<TIn, true, K, V>, dim3(static_cast<unsigned>(items)), dim3(256), 0, s, p);
    else klaunch(prep32_kernel<TIn, false, K, V>, dim3(static_cast<unsigned>(items)), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <typename TIn, int K, int V>
hipError_t launch_prep16(const kda_prefill_args& a, const PrefillParams& p, hipStream_t s) {
    const int64_t items = prefill_max_chunks(a) * a.HV;
    const int elem = sizeof(TIn);
    const bool vec = aligned_rows(a.q, a.q_stride, 3, elem) && aligned_rows(a.k, a.k_stride, 3, elem) &&
                     aligned_rows(a.g, a.g_stride, 3, elem) && aligned_rows(a.v, a.v_stride, 3, elem);
    const dim3 grid(static_cast<unsigned>((items + 3) / 4));
    if (vec) klaunch(prep16_kernel<TIn, true, K, V>, grid, dim3(256), 0, s, p);
    else klaunch(prep16_kernel<TIn, false, K, V>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

#define KDA_PREP32(T, K, V) template hipError_t launch_prep32<T, K, V>(const kda_prefill_args&, const PrefillParams&, hipStream_t); \
    template hipError_t launch_prep16<T, K, V>(const kda_prefill_args&, const PrefillParams&, hipStream_t);
#define KDA_PREP32_T(T) KDA_PREP32(T, 32, 32) KDA_PREP32(T, 32, 64) KDA_PREP32(T, 32, 128) \
    KDA_PREP32(T, 64, 32) KDA_PREP32(T, 64, 64) KDA_PREP32(T, 64, 128) \
    KDA_PREP32(T, 128, 32) KDA_PREP32(T, 128, 64) KDA_PREP32(T, 128, 128)
KDA_PREP32_T(float)
KDA_PREP32_T(bf16)
#undef KDA_PREP32_T
#undef KDA_PREP32

}  // namespace kda
