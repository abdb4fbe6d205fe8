// Target verify without snapshots (A8 + A9, outputs only) on fp32 matrix
// tiles.  One block of 4 waves per (request, head).
//
// With no per-node state to write, the draft is one small chunk.  With S0
// the pool state (K x V), G_i the log-decay summed along the path root .. i
// (per channel), q-hat / k-hat the normalised conv outputs and anc(i) the
// strict ancestors of node i:
//   x_i = S0^T (e^{G_i} k-hat_i),   y_i = S0^T (e^{G_i} q-hat_i)
//   u_i = beta_i (v_i - x_i) - sum_{j in anc(i)} beta_i (k-hat_i . e^{G_i - G_j} k-hat_j) u_j
//   o_i = scale (y_i + sum_{j in anc(i) + i} (q-hat_i . e^{G_i - G_j} k-hat_j) u_j)
// which is the token recurrence (decay, delta correction, read-out) of
// "[KDA] Support Helion MTP verification and harden prefill, decode"
// (Modifications: tree drafts) unrolled from S0: the state after node i is
// e^{G_i} S0 plus the rank-one terms e^{G_i - G_j} k-hat_j u_j^T of the
// path, so S_i^T k and S_i^T q need S0 only through x and y.
//
// The two K-long contractions with S0 are the only large products.  They
// run as v_mfma_f32_16x16x4f32 (fp32 operands and sums), with the e^G k-hat
// rows and e^G q-hat rows stacked in one 16-row operand when N <= 8 (two
// operands for N <= 16) and the state read once from the pool as B
// fragments: lane (j, g) of a 16-column tile holds state row v0 + j at
// channels 16 q + 4 g .. + 3, so k-step (q, e) contracts channel 16 q + 4 g + e
// in lane group g of both operands.  The node-pair Grams are one more tile
// product, [e^G k-hat; e^G q-hat] (e^-G k-hat)^T, when every |G| of the
// block is at most 60 (e^G and e^-G then stay normal floats), and take exact
// per-element exponentials otherwise; the solve for u and the outputs are
// a few fused multiply-adds per column.
//
// Prologue as in the snapshot launch: conv1d over the node's path, then the
// request's conv state, SiLU, L2 norms of q and k; the gate map and beta.
// The state is loaded after the conv: issued with the prologue's small
// loads, the state requests of every block queue ahead of them.  The pool
// is only read.  A padded request (state index < 0, or an index out of
// range) gets zero outputs.

#include "kda_verify_kernel.h"

namespace kda {
namespace {

// Largest |G| (cumulative log-decay along a path) for which the Grams use
// e^G and e^-G as separate factors: both stay normal floats with room for
// the vector magnitudes.
constexpr float kFactorSpan = 60.0f;

// Largest value over the wave, in every lane: the lane exchanges of
// lane_sum (quad permutes, row mirrors, the swizzle across 16-lane rows),
// then the two 32-lane halves.
template <int kCtrl>
__device__ __forceinline__ float dpp_max(float v) {
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false)));
}

__device__ __forceinline__ float wave_max(float x) {
    x = dpp_max<0xB1>(x);     // quad permute: lane ^ 1
    x = dpp_max<0x4E>(x);     // quad permute: lane ^ 2
    x = dpp_max<0x141>(x);    // half-row mirror
    x = dpp_max<0x140>(x);    // row mirror
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F)));
    return fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)),
                 __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)));
}

template <typename TIn, int K, int V, int NMAX, bool CHAIN>
__global__ __launch_bounds__(256) void verify_tile_kernel(const VerifyParams p) {
    constexpr int CH = 2 * K + V;                    // conv channels of a (request, head)
    constexpr int NCS = (CH + 255) / 256;
    constexpr int NT = V / 16;                       // 16-column value tiles
    constexpr int TPW = (NT + kWaves - 1) / kWaves;  // tiles per wave
    constexpr int NQ = K / 16;                       // float4 per lane and operand row
    constexpr bool STACK = NMAX <= 8;                // x rows 0..7, y rows 8..15 of one operand
    constexpr int NOP = STACK ? 1 : 2;
    constexpr int YOFF = STACK ? 8 : 16;             // first y row of the hand-off
    constexpr int KP = K + 4;                        // padded operand row (bank spread)
    constexpr int XP = TPW * 16 + 1;
    constexpr int NPT = 256 / K;                     // threads per channel in the operand pass
    constexpr int kPO = STACK ? 0 : 1, kPR = STACK ? 8 : 0;   // tile and first row of the q Grams
    static_assert(NMAX == 8 || NMAX == 16, "node count build");
    static_assert(V % 16 == 0 && K % 16 == 0 && K <= 256, "tile shape");

    __shared__ float s_q[NMAX][K];                   // q-hat
    __shared__ float s_k[NMAX][K];                   // k-hat
    __shared__ float s_G[NMAX][K];                   // cumulative log-decay along the path
    __shared__ float s_v[NMAX][V];
    __shared__ float s_op[NOP][16][KP];              // e^G k-hat rows [, e^G q-hat rows]
    __shared__ float s_x[kWaves][16 * NOP][XP];      // x / y tiles of each wave
    __shared__ float s_gp[kWaves][NOP][16][16];      // Gram partial tiles of each wave
    __shared__ float s_beta[NMAX], s_rq[NMAX], s_rk[NMAX], s_gmax[kWaves];
    __shared__ unsigned s_anc[NMAX];                 // ancestors and self, as a bit mask
    // trees: node inputs, then the conv state by age (conv phase only); then
    // the k-hat e^-G rows of the factored Grams, in the same bytes
    constexpr int kInBytes = CHAIN ? 0 : (NMAX + kMaxWidth - 1) * CH * (int)sizeof(TIn);
    constexpr int kKiBytes = 16 * KP * (int)sizeof(float);
    __shared__ __attribute__((aligned(16))) char s_buf[kInBytes > kKiBytes ? kInBytes : kKiBytes];
    auto s_in = reinterpret_cast<TIn (*)[CH]>(s_buf);
    auto s_ki = reinterpret_cast<float (*)[KP]>(s_buf);
    __shared__ int s_par[kWaves][NMAX];

    const int bh = blockIdx.x;
    const int h = bh % p.HV;
    const int r = bh / p.HV;
    const int hq = h / p.group;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int N = p.N;
    const int W = p.W;
    const int64_t conv_dim = 2 * (int64_t)p.H * K + (int64_t)p.HV * V;

    TIn* o = static_cast<TIn*>(p.o);
    const int slot = p.idx[r];
    const int cslot = p.cidx ? p.cidx[r] : slot;
    if (slot < 0 || slot >= p.num_slots || cslot < 0 || cslot >= p.num_conv_slots) {
        for (int t = tid; t < N * V; t += 256) {
            const int i = t / V, vv = t % V;
            o[((int64_t)r * N + i) * p.os0 + h * p.os1 + vv] = from_f32<TIn>(0.0f);
        }
        return;
    }

    // ---- the prologue's global loads, all issued before any use.  The
    // state is loaded once they have arrived (after the conv): issued
    // together, the state's bytes from every block delay these small loads
    // by several microseconds. ----

    // parents; a parent outside [-1, i) is treated as a root
    int par[NMAX];
#pragma unroll
    for (int i = 0; i < NMAX; ++i) {
        const int pi = CHAIN ? i - 1 : p.parents[(int64_t)r * N + min(i, N - 1)];
        par[i] = (i < N && pi >= -1 && pi < i) ? pi : -1;
    }
    const int lpar_raw = CHAIN ? lane - 1 : p.parents[(int64_t)r * N + min(lane, N - 1)];

    // conv inputs of this thread's channels (all nodes), the conv state and
    // the weights by age (age 0 = the node itself; state age 1 = its newest entry)
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
                        : 2 * (int64_t)p.H * K + h * V + (cc - 2 * K);
#pragma unroll
        for (int i = 0; i < NMAX; ++i) raw[sl][i] = mixed_r[(int64_t)min(i, N - 1) * p.ms + c];
#pragma unroll
        for (int m = 0; m < kMaxWidth - 1; ++m) cs_age[sl][m] = cs_base[c * (W - 1) + max(W - 2 - m, 0)];
#pragma unroll
        for (int m = 0; m < kMaxWidth; ++m) w_age[sl][m] = ld(cw, c * W + max(W - 1 - m, 0));
        bias_raw[sl] = cb[has_bias ? c : 0];
    }

    // gate inputs of channel tid % K at every node, and beta
    const int gc = tid % K;
    float graw[NMAX];
#pragma unroll
    for (int i = 0; i < NMAX; ++i)
        graw[i] = ld(static_cast<const TIn*>(p.a), ((int64_t)r * N + min(i, N - 1)) * p.as0 + h * K + gc);
    const float gdt_raw = (p.dt_bias ? p.dt_bias : p.pool)[p.dt_bias ? h * K + gc : 0];
    const float gdt = p.dt_bias ? gdt_raw : 0.0f;
    const float braw = ld(static_cast<const TIn*>(p.b), ((int64_t)r * N + min(tid, N - 1)) * p.bs0 + h);
    const int gmode = p.gate;
    const float alog = (p.A_log ? p.A_log : p.pool)[p.A_log ? h : 0];
    const float expA = gmode != kGateRaw ? __expf(alog) : 0.0f;

    // ---- conv + SiLU per channel and node.  Branch-free per node: the
    // activation is a select, and each channel slot's LDS row (q, k or v)
    // is fixed before the node loop. ----
    const bool silu = p.act == KDA_ACT_SILU;
    float* cdst[NCS];
    int cstride[NCS];
#pragma unroll
    for (int sl = 0; sl < NCS; ++sl) {
        const int cc = min(tid + 256 * sl, CH - 1);
        cdst[sl] = cc < K ? &s_q[0][cc] : cc < 2 * K ? &s_k[0][cc - K] : &s_v[0][cc - 2 * K];
        cstride[sl] = cc < 2 * K ? K : V;
    }
    if constexpr (CHAIN) {
        // tap m of node i reads node i - m, or conv-state age m - i once the
        // draft is exhausted; taps at or beyond W leave the sum unchanged
#pragma unroll
        for (int sl = 0; sl < NCS; ++sl) {
            const int cc = tid + 256 * sl;
            if (cc < CH) {
#pragma unroll
                for (int i = 0; i < NMAX; ++i) {
                    if (i >= N) break;
                    float acc = fmaf(w_age[sl][0], to_f32(raw[sl][i]), has_bias ? to_f32(bias_raw[sl]) : 0.0f);
#pragma unroll
                    for (int m = 1; m < kMaxWidth; ++m) {
                        const float x = i - m >= 0 ? to_f32(raw[sl][i - m >= 0 ? i - m : 0])
                                                   : to_f32(cs_age[sl][m - i - 1 >= 0 ? m - i - 1 : 0]);
                        const float t = fmaf(w_age[sl][m], x, acc);
                        acc = m < W ? t : acc;
                    }
                    const float act = acc * sigmoidf(acc);
                    cdst[sl][i * cstride[sl]] = silu ? act : acc;
                }
            }
        }
    }
    if constexpr (!CHAIN) {
        // each thread walks its channel's ancestor path through LDS (its own
        // columns and its wave's parent copy only, so no barrier is needed)
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
                                    a = s_par[wave][a];
                                } else {
                                    src = row_cs++;
                                }
                                acc = fmaf(w_age[sl][m], to_f32(s_in[src][cc]), acc);
                            }
                        }
                        const float act = acc * sigmoidf(acc);
                        cdst[sl][i * cstride[sl]] = silu ? act : acc;
                    }
                }
            }
        }
    }

    // ---- log-decay summed along each node's path, per channel, on the
    // last K threads (the first ones convolve a second channel slot) ----
    float gabs = 0.0f;
    if (tid >= 256 - K) {
        // the gate map with the mode decided once, outside the node loops
        float gl[NMAX];
        if (gmode == kGateBounded) {
#pragma unroll
            for (int i = 0; i < NMAX; ++i) gl[i] = log_gate(graw[i], kGateBounded, expA, gdt, p.lb);
        } else if (gmode == kGateUnbounded) {
#pragma unroll
            for (int i = 0; i < NMAX; ++i) gl[i] = log_gate(graw[i], kGateUnbounded, expA, gdt, p.lb);
        } else {
#pragma unroll
            for (int i = 0; i < NMAX; ++i) gl[i] = graw[i];
        }
        float G[NMAX];
#pragma unroll
        for (int i = 0; i < NMAX; ++i) {
            float gp = 0.0f;
            if constexpr (CHAIN) {
                if (i > 0) gp = G[i > 0 ? i - 1 : 0];
            } else {
#pragma unroll
                for (int jn = 0; jn < NMAX - 1; ++jn)
                    if (jn < i && par[i] == jn) gp = G[jn];
            }
            G[i] = gp + gl[i];
            s_G[i][gc] = G[i];
            gabs = i < N ? fmaxf(gabs, fabsf(G[i])) : gabs;
        }
    }
    gabs = wave_max(gabs);
    if (lane == 0) s_gmax[wave] = gabs;
    if (tid < N) s_beta[tid] = p.beta_is_raw ? sigmoidf(braw) : braw;
    if (tid == 0) {
        unsigned anc[NMAX];
#pragma unroll
        for (int i = 0; i < NMAX; ++i) {
            unsigned a = 0u;
#pragma unroll
            for (int jn = 0; jn < NMAX - 1; ++jn)
                if (jn < i && par[i] == jn) a = anc[jn];
            anc[i] = a | (1u << i);
            s_anc[i] = anc[i];
        }
    }
    lds_barrier();

    // ---- the state: B fragments of this wave's tiles (a wave past the
    // last tile of a narrow head loads the last one again and leaves it
    // unused) ----
    const float* S = p.pool + ((int64_t)slot * p.HV + h) * (int64_t)V * K;
    float4 sb[TPW][NQ];
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
        const int vt = min(wave + kWaves * m, NT - 1);
#pragma unroll
        for (int q = 0; q < NQ; ++q) sb[m][q] = ld4(S, (int64_t)(vt * 16 + l16) * K + 16 * q + 4 * lg);
    }

    // matrix-core Grams when every |G| is small enough for e^G and e^-G to
    // stay normal floats (the products then need no exponential per pair)
    const bool factored = fmaxf(fmaxf(s_gmax[0], s_gmax[1]), fmaxf(s_gmax[2], s_gmax[3])) <= kFactorSpan;

    // ---- L2 norms of q and k: wave w takes nodes w, w + 4, ... ----
    for (int i = wave; i < N; i += kWaves) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int kk = lane; kk < K; kk += 64) {
            const float qv = s_q[i][kk], kv = s_k[i][kk];
            sq = fmaf(qv, qv, sq);
            sk = fmaf(kv, kv, sk);
        }
        if (K >= 64) {
            sq = wave_sum(sq); sk = wave_sum(sk);
        } else {
            sq = lane_sum<32>(sq); sk = lane_sum<32>(sk);
        }
        if (lane == 0) {
            s_rq[i] = p.l2norm ? rsqrtf(sq + kL2Eps) : 1.0f;
            s_rk[i] = p.l2norm ? rsqrtf(sk + kL2Eps) : 1.0f;
        }
    }
    lds_barrier();

    // ---- q-hat, k-hat and the operand rows e^G k-hat, e^G q-hat ----
    {
        const int c = tid % K;
#pragma unroll
        for (int i = tid / K; i < 16; i += NPT) {
            float kr = 0.f, qr = 0.f, ki = 0.f;
            if (i < N) {
                const float qh = s_q[i][c] * s_rq[i], kh = s_k[i][c] * s_rk[i];
                s_q[i][c] = qh;
                s_k[i][c] = kh;
                const float G = s_G[i][c];
                const float e = __expf(G);
                kr = kh * e;
                qr = qh * e;
                if (factored) ki = kh * __expf(-G);
            }
            s_ki[i][c] = ki;
            if (STACK) {
                if (i < 8) {
                    s_op[0][i][c] = kr;
                    s_op[0][8 + i][c] = qr;
                }
            } else {
                s_op[0][i][c] = kr;
                s_op[NOP - 1][i][c] = qr;
            }
        }
    }
    lds_barrier();

    // ---- node-pair Grams, exact exponentials (when |G| is too large to
    // factor): pair n of the list (t, j <= t) goes to wave n mod 4, into
    // the first partial tile ----
    if (!factored) {
        int n = 0;
        for (int t = 0; t < N; ++t) {
            const unsigned at = s_anc[t];
            for (int j = 0; j <= t; ++j, ++n) {
                if ((n & (kWaves - 1)) != wave) continue;
                float pq = 0.f, pk = 0.f;
                if ((at >> j) & 1u) {
#pragma unroll
                    for (int c = lane; c < K; c += 64) {
                        const float kj = s_k[j][c] * __expf(s_G[t][c] - s_G[j][c]);
                        pq = fmaf(s_q[t][c], kj, pq);
                        pk = fmaf(s_k[t][c], kj, pk);
                    }
                    if (K >= 64) {
                        pq = wave_sum(pq); pk = wave_sum(pk);
                    } else {
                        pq = lane_sum<32>(pq); pk = lane_sum<32>(pk);
                    }
                }
                if (lane == 0) {
                    s_gp[0][0][t][j] = pk;
                    s_gp[0][kPO][kPR + t][j] = pq;
                }
            }
        }
    }

    // ---- x and y of this wave's tiles on the matrix cores ----
    {
        float4 ak[NQ], aq[STACK ? 1 : NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            ak[q] = *reinterpret_cast<const float4*>(&s_op[0][l16][16 * q + 4 * lg]);
            if constexpr (!STACK) aq[q] = *reinterpret_cast<const float4*>(&s_op[NOP - 1][l16][16 * q + 4 * lg]);
        }
        f32x4 ax[TPW], ay[STACK ? 1 : TPW];
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
            ax[m] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (!STACK) ay[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const float av[4] = {ak[q].x, ak[q].y, ak[q].z, ak[q].w};
#pragma unroll
            for (int m = 0; m < TPW; ++m) {
                const float bv[4] = {sb[m][q].x, sb[m][q].y, sb[m][q].z, sb[m][q].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) ax[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bv[e], ax[m], 0, 0, 0);
                if constexpr (!STACK) {
                    const float qv[4] = {aq[q].x, aq[q].y, aq[q].z, aq[q].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) ay[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[e], bv[e], ay[m], 0, 0, 0);
                }
            }
        }
        // factored Grams: [e^G k-hat; e^G q-hat] (e^-G k-hat)^T over this
        // wave's quarter of the channels, one partial tile per wave
        if (factored) {
            f32x4 ga = f32x4{0.f, 0.f, 0.f, 0.f}, gq = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < K / 16; ++st) {
                const int c = (K / 4) * wave + 4 * st + lg;
                const float bk = s_ki[l16][c];
                ga = __builtin_amdgcn_mfma_f32_16x16x4f32(s_op[0][l16][c], bk, ga, 0, 0, 0);
                if constexpr (!STACK) gq = __builtin_amdgcn_mfma_f32_16x16x4f32(s_op[NOP - 1][l16][c], bk, gq, 0, 0, 0);
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                s_gp[wave][0][4 * lg + rr][l16] = ga[rr];
                if constexpr (!STACK) s_gp[wave][NOP - 1][4 * lg + rr][l16] = gq[rr];
            }
        }
        // result tile: lane (j, g) holds rows 4 g .. 4 g + 3 of column j
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                s_x[wave][4 * lg + rr][16 * m + l16] = ax[m][rr];
                if constexpr (!STACK) s_x[wave][16 + 4 * lg + rr][16 * m + l16] = ay[m][rr];
            }
        }
    }
    lds_barrier();

    // ---- the Gram coefficients: partial tiles summed, pairs off the
    // ancestor path zeroed, into the first partial (entry e of each tile is
    // read and written by thread e only) ----
    {
        const int nparts = factored ? kWaves : 1;
        const int row = tid >> 4, j = tid & 15;
#pragma unroll
        for (int ot = 0; ot < NOP; ++ot) {
            float g = s_gp[0][ot][row][j];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) {
                const float x = s_gp[w][ot][row][j];
                g += w < nparts ? x : 0.0f;
            }
            // row of tile ot: node t = row - 8 of the q Grams when stacked
            const bool qrow = STACK ? row >= 8 : ot == 1;
            const int t = STACK ? row & 7 : row;
            const bool on = t < N && j < N && ((s_anc[min(t, NMAX - 1)] >> j) & 1u) && (qrow || j < t);
            s_gp[0][ot][row][j] = on ? g : 0.0f;
        }
    }
    lds_barrier();

    // ---- u and the outputs, one value column per lane ----
    if (lane < TPW * 16) {
        const int vt = wave + kWaves * (lane >> 4);
        if (vt < NT) {
            const int vc = vt * 16 + (lane & 15);
            float u[NMAX];
#pragma unroll
            for (int t = 0; t < NMAX; ++t) {
                if (t < N) {
                    float acc = s_v[t][vc] - s_x[wave][t][lane];
#pragma unroll
                    for (int j = 0; j < t; ++j) acc = fmaf(-s_gp[0][0][t][j], u[j], acc);
                    u[t] = s_beta[t] * acc;
                    float ov = s_x[wave][YOFF + t][lane];
#pragma unroll
                    for (int j = 0; j <= t; ++j) ov = fmaf(s_gp[0][kPO][kPR + t][j], u[j], ov);
                    o[((int64_t)r * N + t) * p.os0 + h * p.os1 + vc] = from_f32<TIn>(p.scale * ov);
                }
            }
        }
    }
}

template <typename TIn, int K, int V, int NMAX>
hipError_t launch_tile_kvn(const kda_verify_args& a, const VerifyParams& p, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(a.B * a.HV));
    if (p.parents) klaunch(verify_tile_kernel<TIn, K, V, NMAX, false>, grid, dim3(256), 0, s, p);
    else klaunch(verify_tile_kernel<TIn, K, V, NMAX, true>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

template <typename TIn, int K, int V>
hipError_t launch_tile_kv(const kda_verify_args& a, const VerifyParams& p, hipStream_t s) {
    return a.N <= 8 ? launch_tile_kvn<TIn, K, V, 8>(a, p, s) : launch_tile_kvn<TIn, K, V, 16>(a, p, s);
}

template <typename TIn, int K>
hipError_t launch_tile_k(const kda_verify_args& a, const VerifyParams& p, hipStream_t s) {
    switch (a.V) {
        case 32: return launch_tile_kv<TIn, K, 32>(a, p, s);
        case 64: return launch_tile_kv<TIn, K, 64>(a, p, s);
        default: return launch_tile_kv<TIn, K, 128>(a, p, s);
    }
}

}  // namespace

hipError_t launch_verify_outputs(const kda_verify_args& a, hipStream_t s) {
    const VerifyParams p = make_verify_params(a);
    auto by_k = [&](auto tin) -> hipError_t {
        using TIn = decltype(tin);
        switch (a.K) {
            case 32: return launch_tile_k<TIn, 32>(a, p, s);
            case 64: return launch_tile_k<TIn, 64>(a, p, s);
            default: return launch_tile_k<TIn, 128>(a, p, s);
        }
    };
    return a.dtype == KDA_BF16 ? by_k(bf16{}) : by_k(float{});
}

}  // namespace kda
