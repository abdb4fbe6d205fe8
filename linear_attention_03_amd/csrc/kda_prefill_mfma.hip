// Chunked prefill on MFMA tiles (chunk C = 64, K = V = 128): the path the
// 16-head x 128 workloads take.  Same two-launch structure and algebra as
// the general path, with every chunk-sized product on the matrix cores
// (v_mfma_f32_16x16x32_bf16 / _f16, fp32 accumulate).
//
// prep (persistent blocks of 4 waves, one chunk x head at a time)
//   1. tokens -> LDS: q, k (with their L2 norms), gate g, beta.
//   2. G = in-chunk cumulative g per channel (base-2 units), and per-channel
//      factors of the reference rows m(s) = 16 s + 7 of the 16-row blocks s.
//   3. per row (wave s: rows 16 s .. 16 s + 15, one row per lane group, 32
//      channels per lane): E1 = exp(G_r - G_m), E2 = exp(G_m - G_r) give the
//      Gram operands q-hat E1, k-hat E1 and k-hat E2 (every one <= exp(span),
//      span the largest decay inside half a block: up to 8 fp16, up to 80
//      bf16), and with the per-channel factors, without more exponentials,
//      Qt = q-hat e^G, R = k-hat e^G and Kt = k-hat e^(G_last - G) (fp16).
//      A chunk with span > 80 or any g > 0 takes exact per-element
//      exponentials instead (Qt, R and Kt hold e^G up to the chunk's
//      cumulative log-decay, so a positive gate given directly must keep it
//      below ~11; a bounded gate with a positive lower bound never comes here).
//   4. gated Grams A (strict lower, beta-scaled) and P (lower): block (s, u)
//      is one MFMA product of row block s's operands and key block u's,
//      rescaled per channel from u's reference row to m(s).
//   5. Tm = (I + A)^-1 in fp32: 16 x 16 diagonal blocks by substitution, one
//      per wave, then two levels of block merges on fp32 MFMA tiles.
//   6. W = Tm diag(beta) (K-hat e^G)  (fp16 MFMA)
//      U' = Tm diag(beta) V           (Tm diag(beta) split bf16 hi + lo; V is exact in bf16)
//   Qt, Kt^T, P, W, U' and e^G_last go to the workspace.
// scan (one block of 8 waves per sequence x head x 16 state columns)
//   per chunk, with S (128 x 16, fp32) spread over the 4 state waves as
//   MFMA accumulator tiles:
//     U  = U' - W S                 (state wave w: rows 16w..16w+15)
//     S <- e^G_last * S + Kt^T U    (state wave w: rows 32w..32w+31; U split hi + lo)
//     O  = scale (Qt S + P U)       (output wave 4+j: rows 16j..16j+15)
//   all on fp16 tiles.  S and U pass between waves through double-buffered
//   LDS tiles, two barriers per chunk; the next chunk's operands are loaded
//   while the current one computes.
// Operand precision was chosen by emulating the chunked form against the
// fp64 recurrence.  Every fp16 operand is bounded by the algebra under a
// decaying gate (|Kt|, |Qt|, |K-hat e^G|, |P|, |A| <= 1; Gram factors <=
// e^8 on the fp16 path; S and U of the size of the values), and fp16's
// 11-bit significand keeps the state within ~4e-4 of the recurrence even
// when the decay is slow and no rounding error is forgotten; bf16 operands
// in W S or the state update left up to ~2e-3.  U' keeps a split left
// operand (bf16 hi + lo) against bf16 V.

#include <type_traits>

#include "kda_prefill_mfma.h"

namespace kda {
namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));

// Eight consecutive rows k0..k0+7 of column n0 + (lane % 16) of a row-major
// bf16 matrix in LDS (row stride ld elements, ld and n0 multiples of 4), as
// one MFMA operand fragment.  Built from two transposing LDS reads: in each
// group of 16 lanes, lane L addresses row k + L / 4, columns n0 + 4 (L % 4),
// and lane l receives element l % 4 of the rows addressed by lanes 4 j + l / 4.
__device__ __forceinline__ bf16x8 lds_col8(const __bf16* base, int ld, int k0, int n0, int l16) {
    const __bf16* p0 = base + (k0 + (l16 >> 2)) * ld + n0 + 4 * (l16 & 3);
    const short4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4_t*)(p0));
    const short4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4_t*)(p0 + 4 * ld));
    const short8_t ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, ab);
}

// One (chunk, head) of the prep: chunk index ci (global over the batch or
// the packed sequences), head h, and the chunk's tokens [t0, t0 + len) of
// batch row b.
struct PrepItem {
    int ci, h, b, t0, len;
};

__device__ __forceinline__ bool prep_locate(const PrefillParams& p, int64_t item, PrepItem& it) {
    if (item >= (int64_t)p.max_chunks * p.HV) return false;
    it.h = static_cast<int>(item % p.HV);
    it.ci = static_cast<int>(item / p.HV);
    if (p.cu) {
        int n, cstart;
        if (!locate_chunk(p.cu, p.num_seqs, p.T, C, it.ci, n, cstart)) return false;
        it.b = 0;
        it.t0 = cu_at(p.cu, n, p.T) + (it.ci - cstart) * C;
        it.len = min(C, cu_at(p.cu, n, p.T) + seq_len(p.cu, n, p.T) - it.t0);
    } else {
        const int cpb = ceil_div(p.T, C);
        it.b = it.ci / cpb;
        it.t0 = (it.ci % cpb) * C;
        it.len = min(C, p.T - it.t0);
    }
    return true;
}

// Activations of one item as this lane loads them: rows 16 w + 4 it + sub,
// channels c8..c8+7 of q, k, g (v separately); beta of those rows; dt_bias
// of the channels.  Rows past the chunk re-read its last row (zeroed on use).
struct PrepIn {
    uint4 q[4], k[4], g[4];
    float beta[4];
    float dt[8];
    float a_log;
};

struct VRows {
    uint4 v[4];
};

__device__ __forceinline__ VRows prep_issue_v(const PrefillParams& p, const PrepItem& it, int wave, int sub, int c8) {
    const bf16* vg = static_cast<const bf16*>(p.v) + it.b * p.vs[0] + it.h * p.vs[2] + c8;
    VRows r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = it.t0 + min(16 * wave + 4 * i + sub, it.len - 1);
        r.v[i] = *reinterpret_cast<const uint4*>(vg + t * p.vs[1]);
    }
    return r;
}

// With `dummy` every row index is the chunk's first row: the load stays
// unconditional (simple waits) but reads lines already in cache.
template <typename TIn>
__device__ __forceinline__ void prep_issue(const PrefillParams& p, const PrepItem& it, PrepIn& in,
                                           int wave, int sub, int c8, bool dummy = false) {
    const int hq = it.h / p.group;       // q/k head of this value head
    const bf16* qg = static_cast<const bf16*>(p.q) + it.b * p.qs[0] + hq * p.qs[2] + c8;
    const bf16* kg = static_cast<const bf16*>(p.k) + it.b * p.ks[0] + hq * p.ks[2] + c8;
    const bf16* gg = static_cast<const bf16*>(p.g) + it.b * p.gs[0] + it.h * p.gs[2] + c8;
    const TIn* bg = static_cast<const TIn*>(p.beta) + it.b * p.bs[0] + it.h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = it.t0 + (dummy ? 0 : min(16 * wave + 4 * i + sub, it.len - 1));
        in.q[i] = *reinterpret_cast<const uint4*>(qg + t * p.qs[1]);
        in.k[i] = *reinterpret_cast<const uint4*>(kg + t * p.ks[1]);
        in.g[i] = *reinterpret_cast<const uint4*>(gg + t * p.gs[1]);
        in.beta[i] = ld(bg, t * p.bs[1]);
    }
    in.a_log = p.gate != kGateRaw ? p.A_log[it.h] : 0.0f;
    if (p.dt_bias) {
        const float4 d0 = ld4(p.dt_bias, (int64_t)it.h * K + c8);
        const float4 d1 = ld4(p.dt_bias, (int64_t)it.h * K + c8 + 4);
        in.dt[0] = d0.x; in.dt[1] = d0.y; in.dt[2] = d0.z; in.dt[3] = d0.w;
        in.dt[4] = d1.x; in.dt[5] = d1.y; in.dt[6] = d1.z; in.dt[7] = d1.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) in.dt[e] = 0.0f;
    }
}

// prep: persistent blocks of 4 waves, one (chunk, head) at a time; under
// 80 KiB of LDS so two blocks share a CU.  q and k stay in LDS as the input bf16 values with
// their per-row norms; A is kept in fp16; beta is folded into the inverse,
// Tm' = (I + A)^-1 diag(beta), so U' = Tm' V takes V exactly as bf16.
template <typename TIn>
__global__ __launch_bounds__(256, 2) void prep_mfma_kernel(const PrefillParams p) {
    constexpr int LDG = K + 4;                  // fp32 row stride (16-byte rows; a 16-lane row walk is conflict-free)
    constexpr int LDQ = K + 8;                  // bf16 row stride of q, k (16-byte aligned, staggered)
    constexpr int LDA = C + 4;                  // fp16 row stride of A (8-byte aligned rows)
    constexpr int QK = C * LDQ;
    static_assert(C * (C + 1) <= C * LDG, "Tm fits where G was");
    __shared__ __attribute__((aligned(16))) __bf16 s_q[QK];    // q rows; then Kt (fp16 bits); then V rows
    __shared__ __attribute__((aligned(16))) __bf16 s_k[QK];    // k rows; then K-hat e^G rows
    __shared__ float s_G[C * LDG];                             // g, cumulative G; then Tm
    __shared__ _Float16 s_A[C * LDA];                          // A (|A| < 1), fp16
    __shared__ __attribute__((aligned(16))) float s_beta[C];
    __shared__ __attribute__((aligned(16))) float s_rq[C];
    __shared__ __attribute__((aligned(16))) float s_rk[C];
    float* s_T = s_G;                                          // [C][C + 1]

    const int gmode = p.gate;
    __shared__ int s_flag[4];

    // Persistent: block b takes items b, b + gridDim.x, ... (item = chunk *
    // HV + head, so the items of a block only grow and the first one past the
    // last chunk ends the loop).  The next item's activations are loaded while
    // the current one is computed.
    int64_t item = blockIdx.x;
    PrepItem cur;
    if (!prep_locate(p, item, cur)) return;
    PrepIn in;
    {
        const int w0 = threadIdx.x >> 6, s0 = (threadIdx.x >> 4) & 3, c0 = (threadIdx.x & 15) * 8;
        prep_issue<TIn>(p, cur, in, w0, s0, c0);
    }
    // wait once for the first item: left pending into the loop, its
    // registers would make the loop-head wait cover every store in flight
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    for (;;) {
    // The thread index goes through an opaque move each item, so the many
    // per-thread addresses derived from it are computed inside the loop
    // rather than hoisted out of it and held in registers for its whole run.
    int tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"(static_cast<int>(threadIdx.x)));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int sub = lane >> 4;
    const int l16 = lane & 15;
    const int c8 = l16 * 8;
    const int h = cur.h, len = cur.len;
    char* ws = reinterpret_cast<char*>(p.ws) + ((int64_t)cur.ci * p.HV + h) * CHUNK_BYTES;
    __bf16* gW = reinterpret_cast<__bf16*>(ws + OFF_W);
    __bf16* gKt = reinterpret_cast<__bf16*>(ws + OFF_KT);         // fp16 bits
    __bf16* gQt = reinterpret_cast<__bf16*>(ws + OFF_QT);
    __bf16* gP = reinterpret_cast<__bf16*>(ws + OFF_P);
    float* gUp = reinterpret_cast<float*>(ws + OFF_UP);
    float* gGl = reinterpret_cast<float*>(ws + OFF_GL);

    // ---- 1. tokens -> LDS: wave w rows 16w + 4 it + sub, 16 lanes x 8 channels per row
    const float expA = gmode != kGateRaw ? __expf(in.a_log) : 0.0f;
    const float nA2 = -expA * kLog2e;            // bounded: sigmoid(expA x) = 1 / (1 + 2^(nA2 x))
    const float lb2 = p.lb * kLog2e;
    bool unsafe = false, wide = false;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int r = 16 * wave + 4 * it + sub;
        const bool valid = r < len;
        const uint4 zero = make_uint4(0, 0, 0, 0);
        const uint4 qr = valid ? in.q[it] : zero, kr = valid ? in.k[it] : zero, gr = valid ? in.g[it] : zero;
        float qv[8], kv[8], gv[8];
        const uint32_t qw[4] = {qr.x, qr.y, qr.z, qr.w};
        const uint32_t kw[4] = {kr.x, kr.y, kr.z, kr.w};
        const uint32_t gw[4] = {gr.x, gr.y, gr.z, gr.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qv[2 * e] = __uint_as_float(qw[e] << 16); qv[2 * e + 1] = __uint_as_float(qw[e] & 0xffff0000u);
            kv[2 * e] = __uint_as_float(kw[e] << 16); kv[2 * e + 1] = __uint_as_float(kw[e] & 0xffff0000u);
            gv[2 * e] = __uint_as_float(gw[e] << 16); gv[2 * e + 1] = __uint_as_float(gw[e] & 0xffff0000u);
        }
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) { sq += qv[e] * qv[e]; sk += kv[e] * kv[e]; }
        sq = lane_sum<16>(sq);
        sk = lane_sum<16>(sk);
        *reinterpret_cast<uint4*>(&s_q[r * LDQ + c8]) = qr;
        *reinterpret_cast<uint4*>(&s_k[r * LDQ + c8]) = kr;
        // one gate map per call (uniform branch), so the bounded path does
        // not also evaluate the softplus
        float glv[8];                           // g log2(e)
        if (gmode == kGateUnbounded) {
#pragma unroll
            for (int e = 0; e < 8; ++e) glv[e] = valid ? nA2 * softplusf(gv[e] + in.dt[e]) : 0.0f;
        } else if (gmode == kGateBounded) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                glv[e] = valid ? lb2 * __builtin_amdgcn_rcpf(1.0f + exp2_hw(nA2 * (gv[e] + in.dt[e]))) : 0.0f;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) glv[e] = valid ? gv[e] * kLog2e : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) unsafe |= glv[e] > 0.0f;
        *reinterpret_cast<float4*>(&s_G[r * LDG + c8]) = make_float4(glv[0], glv[1], glv[2], glv[3]);
        *reinterpret_cast<float4*>(&s_G[r * LDG + c8 + 4]) = make_float4(glv[4], glv[5], glv[6], glv[7]);
        if (l16 == 0) {
            s_rq[r] = p.l2norm ? rsqrtf(sq + kL2Eps) : 1.0f;
            s_rk[r] = p.l2norm ? rsqrtf(sk + kL2Eps) : 1.0f;
            float bt = valid ? in.beta[it] : 0.0f;
            if (valid && p.beta_is_raw) bt = sigmoidf(bt);
            s_beta[r] = bt;
        }
    }
    // v of this item (used after the Grams); then the next item's location
    __builtin_amdgcn_sched_barrier(0);
    const VRows vr = prep_issue_v(p, cur, wave, sub, c8);
    PrepItem nxt;
    const bool more = prep_locate(p, item + gridDim.x, nxt);
    lds_barrier();

    // ---- 2. cumulative log-decay per channel; decay spans inside half blocks;
    //         per-channel factors of the reference rows.  Thread t scans rows
    //         32 h .. 32 h + 31 of channel t % K (h = t / K); the first half's
    //         totals and rows 7, 15, 23, 31 reach the second half through LDS.
    //         With m(s) = 16 s + 7 and l(u) = 16 u + 15 (the last row of block u):
    //           e^G_m(s), e^(G_last - G_m(s))   LDS tables, read by the row phase
    //           f(u) = e^(G_l(u) - G_m(u)), d(s, u) = e^(G_m(s) - G_l(u)), u < s,
    //         kept in registers until the Gram phase (every factor is <= 1).
    float* const s_tot = reinterpret_cast<float*>(s_A);        // A is written only after the Gram phase
    const float* const s_tab = s_tot + 5 * K;                   // [8][K]: e^G_m(s), then e^(G_last - G_m(s))
    static_assert(13 * K * 4 <= C * LDA * 2, "totals and factor tables fit the space of A");
    const int cc = tid & (K - 1), hf = tid / K;                 // channel and half of the column threads
    float dfac[6];                                              // second half: d(s, u), pair s (s - 1) / 2 + u
    float ffac[2];                                              // first half: f(0), f(1); second half: f(2)
    {
        float* s_gx = s_tot + K;                                // [4][K]: G at rows 7, 15, 23, 31
        float G[C / 2];
        float run = 0.0f;
#pragma unroll
        for (int r = 0; r < C / 2; ++r) G[r] = s_G[(32 * hf + r) * LDG + cc];
#pragma unroll
        for (int r = 0; r < C / 2; ++r) { run += G[r]; G[r] = run; }
        // spans are differences inside a 16-row block: the half's offset cancels
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const float span = fmaxf(G[16 * s2] - G[16 * s2 + 7], G[16 * s2 + 7] - G[16 * s2 + 15]);
            unsafe |= span > kMaxSpan2;
            wide |= span > kF16Span2;
        }
        ffac[0] = exp2_hw(G[15] - G[7]);
        ffac[1] = exp2_hw(G[31] - G[23]);
        if (hf == 0) {
            s_tot[cc] = run;
            s_gx[cc] = G[7];
            s_gx[K + cc] = G[15];
            s_gx[2 * K + cc] = G[23];
            s_gx[3 * K + cc] = G[31];
        }
        lds_barrier();
        const float off = hf == 0 ? 0.0f : s_tot[cc];
#pragma unroll
        for (int r = 0; r < C / 2; ++r) s_G[(32 * hf + r) * LDG + cc] = G[r] + off;
        if (hf == 1) {
            const float gl = run + off;
            const float gm[4] = {s_gx[cc], s_gx[2 * K + cc], G[7] + off, G[23] + off};
            const float glast[3] = {s_gx[K + cc], s_gx[3 * K + cc], G[15] + off};
            gGl[cc] = exp2_hw(gl);
            float* tab = s_tot + 5 * K;
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                tab[sb * K + cc] = exp2_hw(gm[sb]);
                tab[(4 + sb) * K + cc] = exp2_hw(gl - gm[sb]);
            }
#pragma unroll
            for (int sb = 1; sb < 4; ++sb)
#pragma unroll
                for (int u = 0; u < sb; ++u) dfac[sb * (sb - 1) / 2 + u] = exp2_hw(gm[sb] - glast[u]);
        }
    }
    {   // block-wide ORs through LDS (a plain __syncthreads_or would also wait
        // for the next item's loads)
        const int any = (__ballot(unsafe) != 0 ? 1 : 0) | (__ballot(wide) != 0 ? 2 : 0);
        if (lane == 0) s_flag[wave] = any;
        lds_barrier();
        const int all = s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3];
        unsafe = (all & 1) != 0;
        wide = (all & 2) != 0;
    }

    // ---- 3. per row: wave w owns rows 16 w .. 16 w + 15, lane (l16, sub) row
    //         ra = 16 w + l16 at channels 32 ks + 8 sub .. + 7 (the layout of an
    //         MFMA operand fragment).  With the block's reference row m,
    //           E1 = e^(G_r - G_m), E2 = e^(G_m - G_r)  (both <= e^span)
    //         give the Gram operands q-hat E1, k-hat E1 (row side) and k-hat E2
    //         (key side), and without further exponentials
    //           Qt = q-hat e^G = q-hat E1 e^G_m          (-> workspace)
    //           R  = k-hat e^G = k-hat E1 e^G_m          (W's right-hand side)
    //           Kt = k-hat e^(G_last - G) = k-hat E2 e^(G_last - G_m).
    //         The Gram operands are fp16 or bf16 by span (bits kept as fp16).
    const int ra = 16 * wave + l16;
    f16x8 opq[4], opk[4], opb[4];
    f16x8 rrow[4], ktr[4];
    auto row_fast = [&](auto f16tag) {
        constexpr bool F16 = decltype(f16tag)::value;
        const int m = 16 * wave + 7;
        const float rqa = s_rq[ra], rka = s_rk[ra];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int k0 = 32 * ks + 8 * sub;
            const float4 g0 = *reinterpret_cast<const float4*>(&s_G[ra * LDG + k0]);
            const float4 g1 = *reinterpret_cast<const float4*>(&s_G[ra * LDG + k0 + 4]);
            const float4 m0 = *reinterpret_cast<const float4*>(&s_G[m * LDG + k0]);
            const float4 m1 = *reinterpret_cast<const float4*>(&s_G[m * LDG + k0 + 4]);
            const float4 x0 = *reinterpret_cast<const float4*>(&s_tab[wave * K + k0]);
            const float4 x1 = *reinterpret_cast<const float4*>(&s_tab[wave * K + k0 + 4]);
            const float4 y0 = *reinterpret_cast<const float4*>(&s_tab[(4 + wave) * K + k0]);
            const float4 y1 = *reinterpret_cast<const float4*>(&s_tab[(4 + wave) * K + k0 + 4]);
            const bf16x8 qr = *reinterpret_cast<const bf16x8*>(&s_q[ra * LDQ + k0]);
            const bf16x8 kr = *reinterpret_cast<const bf16x8*>(&s_k[ra * LDQ + k0]);
            const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
            const float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
            const float em[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            const float el[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
            f16x8 qt, rw, kt;
            float aq[8], ak[8], bk[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float dl = gv[e] - mv[e];
                const float e1 = exp2_hw(dl), e2 = exp2_hw(-dl);
                const float qn = static_cast<float>(qr[e]) * rqa, kn = static_cast<float>(kr[e]) * rka;
                aq[e] = qn * e1;
                ak[e] = kn * e1;
                bk[e] = kn * e2;
                qt[e] = static_cast<_Float16>(aq[e] * em[e]);
                rw[e] = static_cast<_Float16>(ak[e] * em[e]);
                kt[e] = static_cast<_Float16>(bk[e] * el[e]);
            }
            if constexpr (F16) {
                f16x8 a, b, c;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    a[e] = static_cast<_Float16>(aq[e]);
                    b[e] = static_cast<_Float16>(ak[e]);
                    c[e] = static_cast<_Float16>(bk[e]);
                }
                opq[ks] = a; opk[ks] = b; opb[ks] = c;
            } else {
                bf16x8 a, b, c;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    a[e] = tobf(aq[e]);
                    b[e] = tobf(ak[e]);
                    c[e] = tobf(bk[e]);
                }
                opq[ks] = __builtin_bit_cast(f16x8, a);
                opk[ks] = __builtin_bit_cast(f16x8, b);
                opb[ks] = __builtin_bit_cast(f16x8, c);
            }
            *reinterpret_cast<f16x8*>(gQt + afrag(ra, k0, K / 32)) = qt;
            rrow[ks] = rw;
            ktr[ks] = kt;
        }
    };
    // wide spans or a positive log-decay: Qt, R and Kt with their own
    // exponentials, and the Grams with exact per-element exponentials
    // (argument <= 0 for r >= j)
    auto row_exact = [&]() {
        const float rqa = s_rq[ra], rka = s_rk[ra];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int k0 = 32 * ks + 8 * sub;
            const bf16x8 qr = *reinterpret_cast<const bf16x8*>(&s_q[ra * LDQ + k0]);
            const bf16x8 kr = *reinterpret_cast<const bf16x8*>(&s_k[ra * LDQ + k0]);
            f16x8 qt, rw, kt;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float gv = s_G[ra * LDG + k0 + e], gl = s_G[(C - 1) * LDG + k0 + e];
                const float eg = exp2_hw(gv);
                const float qn = static_cast<float>(qr[e]) * rqa, kn = static_cast<float>(kr[e]) * rka;
                qt[e] = static_cast<_Float16>(qn * eg);
                rw[e] = static_cast<_Float16>(kn * eg);
                kt[e] = static_cast<_Float16>(kn * exp2_hw(gl - gv));
            }
            *reinterpret_cast<f16x8*>(gQt + afrag(ra, k0, K / 32)) = qt;
            rrow[ks] = rw;
            ktr[ks] = kt;
        }
        auto qhat = [&](int r, int c) { return static_cast<float>(s_q[r * LDQ + c]) * s_rq[r]; };
        auto khat = [&](int r, int c) { return static_cast<float>(s_k[r * LDQ + c]) * s_rk[r]; };
        for (int e = tid; e < C * C; e += 256) {
            const int r = e / C, j = e % C;
            float av = 0.f, pv = 0.f;
            if (j <= r) {
                for (int c = 0; c < K; ++c) {
                    const float kj = khat(j, c) * exp2_hw(s_G[r * LDG + c] - s_G[j * LDG + c]);
                    av = fmaf(khat(r, c), kj, av);
                    pv = fmaf(qhat(r, c), kj, pv);
                }
            }
            reinterpret_cast<_Float16*>(gP)[afrag(r, j, C / 32)] = static_cast<_Float16>(pv);
            s_A[r * LDA + j] = static_cast<_Float16>(j < r ? s_beta[r] * av : 0.0f);
        }
    };
    if (unsafe) row_exact();
    else if (wide) row_fast(std::false_type{});
    else row_fast(std::true_type{});
    lds_barrier();                              // q, k, G and the factor tables are no longer read

    // Kt rows (fp16) into the q space for the transposed reads; key-side Gram
    // operands of row blocks 0..2 and the factors f, d into the k space
    f16x8* const s_bk = reinterpret_cast<f16x8*>(s_k);                 // [3][4][64] fragments
    float* const s_d = reinterpret_cast<float*>(s_k) + 3 * 4 * 64 * 4;  // [6][K] d(s, u)
    float* const s_f = s_d + 6 * K;                                     // [3][K] f(u)
    static_assert(3 * 4 * 64 * 16 + 9 * K * 4 <= QK * 2, "key-side operands and factors fit the k space");
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) *reinterpret_cast<f16x8*>(&s_q[ra * LDQ + 32 * ks + 8 * sub]) = ktr[ks];
    if (!unsafe) {
        if (wave < 3) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) s_bk[(wave * 4 + ks) * 64 + lane] = opb[ks];
        }
        if (hf == 0) {
            s_f[cc] = ffac[0];
            s_f[K + cc] = ffac[1];
        } else {
            s_f[2 * K + cc] = ffac[0];
#pragma unroll
            for (int pr = 0; pr < 6; ++pr) s_d[pr * K + cc] = dfac[pr];
        }
    }
    lds_barrier();

    // ---- 4. gated Grams A (-> LDS, fp16) and P (-> workspace, fp16): wave s
    //         forms row block s against key blocks u <= s.  Key block u's
    //         operand has u's reference row; against row block s it is
    //         scaled per channel by f(u), to the block's last row, then by
    //         d(s, u), to m(s): e^(G_m(s) - G_j) = d(s, u) f(u) e^(G_m(u) - G_j).
    //         (d(s, u) f(u) alone can underflow where e^(G_m(u) - G_j) is
    //         large; after f(u) the operand is <= 1 and d(s, u) <= 1.)
    auto grams = [&](auto f16tag) {
        constexpr bool F16 = decltype(f16tag)::value;
        using OpT = typename std::conditional<F16, f16x8, bf16x8>::type;
        const int s = wave;
        const float ba = s_beta[ra];
        for (int nt = 0; nt < 4; ++nt) {
            // operands swapped: the tile comes out transposed, each lane holding
            // row ra of P and A at columns j0..j0+3
            f32x4_t accP = {0.f, 0.f, 0.f, 0.f}, accA = {0.f, 0.f, 0.f, 0.f};
            if (nt <= s) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    OpT bb;
                    if (nt == s) {
                        bb = __builtin_bit_cast(OpT, opb[ks]);
                    } else {
                        const OpT raw = __builtin_bit_cast(OpT, s_bk[(nt * 4 + ks) * 64 + lane]);
                        const float* dp = s_d + (s * (s - 1) / 2 + nt) * K + 32 * ks + 8 * sub;
                        const float* fp = s_f + nt * K + 32 * ks + 8 * sub;
                        const float4 d0 = *reinterpret_cast<const float4*>(dp);
                        const float4 d1 = *reinterpret_cast<const float4*>(dp + 4);
                        const float4 f0 = *reinterpret_cast<const float4*>(fp);
                        const float4 f1 = *reinterpret_cast<const float4*>(fp + 4);
                        const float dv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
                        const float fv[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float x = (static_cast<float>(raw[e]) * fv[e]) * dv[e];
                            if constexpr (F16) bb[e] = static_cast<_Float16>(x);
                            else bb[e] = tobf(x);
                        }
                    }
                    accP = mma(bb, __builtin_bit_cast(OpT, opq[ks]), accP);
                    accA = mma(bb, __builtin_bit_cast(OpT, opk[ks]), accA);
                }
            }
            const int j0 = 16 * nt + 4 * sub;
            f16x4 pv, av;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pv[i] = static_cast<_Float16>(j0 + i <= ra ? accP[i] : 0.0f);
                av[i] = static_cast<_Float16>(j0 + i < ra ? ba * accA[i] : 0.0f);
            }
            *reinterpret_cast<f16x4*>(gP + afrag(ra, j0, C / 32)) = pv;
            *reinterpret_cast<f16x4*>(&s_A[ra * LDA + j0]) = av;
        }
    };
    if (!unsafe) {
        if (wide) grams(std::false_type{});
        else grams(std::true_type{});
    }
    // Kt^T fragments by transposed LDS reads (16-bit lanes, so the fp16 bits
    // move unchanged): tile (16 channels, 32 tokens) kt, rt; wave w stores
    // tiles 4w..4w+3
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int tile = 4 * wave + u;          // tile = 2 * (channel block) + token block
        const int kt = tile >> 1, rt = tile & 1;
        const bf16x8 bits = lds_col8(s_q, LDQ, 32 * rt + 8 * sub, 16 * kt, l16);
        *reinterpret_cast<bf16x8*>(gKt + (tile * 64 + lane) * 8) = bits;
    }
    lds_barrier();

    // next item's q, k, g, beta, dt: they land while the rest runs; with no
    // next item one cached row of the current one is loaded instead (an
    // unconditional load keeps the waits simple)
    __builtin_amdgcn_sched_barrier(0);          // keep these loads here (register pressure)
    prep_issue<TIn>(p, more ? nxt : cur, in, wave, sub, c8, !more);

    // ---- 5. Tm = (I + A)^-1.  Diagonal 16 x 16 blocks, one per wave (wave w:
    //         block w), by forward substitution along the rows: lane (c, sub)
    //         solves column c (the four lane groups alike), reading row rr of A
    //         as four-element vectors, and keeps rows 4 sub .. 4 sub + 3 -- the
    //         layout of an MFMA result tile.  Meanwhile the right-hand sides go
    //         row-major into LDS: R into the k space, V into the q space.
    {
        const int d0 = 16 * wave;
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float acc = rr == l16 ? 1.0f : 0.0f;
#pragma unroll
            for (int t4 = 0; t4 < rr; t4 += 4) {
                const f16x4 a4 = *reinterpret_cast<const f16x4*>(&s_A[(d0 + rr) * LDA + d0 + t4]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (t4 + e < rr) acc = fmaf(-static_cast<float>(a4[e]), x[t4 + e], acc);
            }
            x[rr] = acc;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = sub == 0 ? x[i] : sub == 1 ? x[4 + i] : sub == 2 ? x[8 + i] : x[12 + i];
            s_T[(d0 + 4 * sub + i) * (C + 1) + d0 + l16] = v;
        }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) *reinterpret_cast<f16x8*>(&s_k[ra * LDQ + 32 * ks + 8 * sub]) = rrow[ks];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int r = 16 * wave + 4 * it + sub;
        *reinterpret_cast<uint4*>(&s_q[r * LDQ + c8]) = vr.v[it];
    }
    lds_barrier();
    //      Blocks below the diagonal by merging the inverses of halves:
    //      the inverse of [[L1, 0], [B, L2]] has the lower left block
    //      -L2^-1 B L1^-1 (first the 32 x 32 halves from the 16 x 16 blocks,
    //      then the whole).  fp32 MFMA tiles (16 x 16 x 4).  A product whose
    //      right operand is a previous result takes it from registers: in
    //      k-step j lane (l16, sub) holds row 4 sub + j of that tile, so the
    //      left operand is read at column 4 sub + j.
    auto prod_at = [&](int rb, int ub, int cb, f32x4_t acc) {      // += A[rb][ub] T[ub][cb]
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kk = 4 * j + sub;
            const float av = static_cast<float>(s_A[(16 * rb + l16) * LDA + 16 * ub + kk]);
            const float tv = s_T[(16 * ub + kk) * (C + 1) + 16 * cb + l16];
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, tv, acc, 0, 0, 0);
        }
        return acc;
    };
    auto prod_treg = [&](int rb, int mb, f32x4_t y, f32x4_t acc) {  // += T[rb][mb] Y
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float tv = s_T[(16 * rb + l16) * (C + 1) + 16 * mb + 4 * sub + j];
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(tv, y[j], acc, 0, 0, 0);
        }
        return acc;
    };
    auto store_neg = [&](int rb, int cb, f32x4_t x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s_T[(16 * rb + 4 * sub + i) * (C + 1) + 16 * cb + l16] = -x[i];
    };
    // level 1: T[1][0] = -T[1][1] A[1][0] T[0][0] (wave 1), T[3][2] likewise (wave 3)
    if (wave & 1) {
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        const f32x4_t y = prod_at(wave, wave - 1, wave - 1, zero);
        store_neg(wave, wave - 1, prod_treg(wave, wave, y, zero));
    }
    lds_barrier();
    // level 2: block (rb, cb), rb in {2, 3}, cb in {0, 1}, one per wave:
    //   T[rb][cb] = -sum_{m=2..rb} T[rb][m] sum_{u=cb..1} A[m][u] T[u][cb]
    {
        const int rb = 2 + (wave >> 1), cb = wave & 1;
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        f32x4_t x = zero;
        for (int m = 2; m <= rb; ++m) {
            f32x4_t y = zero;
            for (int u = cb; u < 2; ++u) y = prod_at(m, u, cb, y);
            x = prod_treg(rb, m, y, x);
        }
        store_neg(rb, cb, x);
    }
    lds_barrier();

    // ---- 6. W = Tm' (K-hat e^G) (fp16) and U' = Tm' V (Tm' split into bf16
    //         hi + lo; V is exact in bf16), Tm' = Tm diag(beta); wave w: rows 16w..16w+15
    {
        const int mt = wave;
        const int nks = mt < 2 ? 1 : 2;         // Tm is lower triangular
        bf16x8 th[2], tl[2];
        f16x8 tf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int j = 32 * ks + 8 * sub + jj;
                // blocks above the diagonal are zero (never written)
                const float tv = (j >> 4) <= mt ? s_T[(16 * mt + l16) * (C + 1) + j] * s_beta[j] : 0.0f;
                const __bf16 hi = tobf(tv);
                th[ks][jj] = hi;
                tl[ks][jj] = tobf(tv - static_cast<float>(hi));
                tf[ks][jj] = static_cast<_Float16>(tv);
            }
        }
        for (int nt = 0; nt < K / 16; ++nt) {
            f32x4_t accW = {0.f, 0.f, 0.f, 0.f}, accU = {0.f, 0.f, 0.f, 0.f};
            for (int ks = 0; ks < nks; ++ks) {
                const f16x8 bw = __builtin_bit_cast(f16x8, lds_col8(s_k, LDQ, 32 * ks + 8 * sub, 16 * nt, l16));
                const bf16x8 bv = lds_col8(s_q, LDQ, 32 * ks + 8 * sub, 16 * nt, l16);
                accW = mfma16(bw, tf[ks], accW);        // transposed: W[16 mt + l16][16 nt + 4 sub + i]
                accU = mfma(th[ks], bv, accU);
                accU = mfma(tl[ks], bv, accU);
            }
            f16x4 wv;
#pragma unroll
            for (int i = 0; i < 4; ++i) wv[i] = static_cast<_Float16>(-accW[i]);   // stored negated: the scan computes U' + (-W) S
            *reinterpret_cast<f16x4*>(gW + afrag(16 * mt + l16, 16 * nt + 4 * sub, K / 32)) = wv;
            *reinterpret_cast<float4*>(gUp + ((mt * (V / 16) + nt) * 64 + lane) * 4) =
                make_float4(accU[0], accU[1], accU[2], accU[3]);
        }
    }
    if (!more) break;
    item += gridDim.x;
    cur = nxt;
    lds_barrier();              // the next item's first phase overwrites every LDS array
    }
}

// Scan: one block of 8 waves per (sequence, head, 16 state columns).
//   waves 0-3 ("state" waves): wave w keeps state rows 32w..32w+31 of the
//     block's columns in two MFMA accumulator tiles, computes U rows
//     16w..16w+15 and updates its state tiles.  They only load.
//   waves 4-7 ("output" waves): output wave 4+j computes output rows
//     16j..16j+15 of chunk c from the S and U tiles of chunk c in LDS:
//     Qt S between the two barriers of step c, P U and the stores between
//     step c's second barrier and step c+1's first, so the output work is
//     split over both halves of a step.  With S and U double buffered, the
//     state waves overwrite a chunk's tiles only two steps later.
// Per chunk, two barriers: after S is published (before U) and after U is
// published (before the state update).
constexpr int kScanWaves = 8;
constexpr int LDS_S = K + 16;    // fp16 row stride of the S^T tile (16-byte aligned rows; +16 measured
                                 // fewer LDS bank-conflict cycles than +8 or +24)
constexpr int LDS_U = C + 16;

constexpr int kBufs = 2;
struct ScanShared {
    _Float16 St[kBufs][VS * LDS_S];  // S^T as fp16 [col][k], state wave w's rows scaled by 1 / sc[w]
    _Float16 Uh[kBufs][VS * LDS_U];  // U^T high part [col][r], fp16, rows of wave w scaled by 1 / sc[4 + w]
    _Float16 Ul[kBufs][VS * LDS_U];  // U^T low part
    float sc[kBufs][8];              // 2^e_S of state waves 0..3, then 2^e_U (range-safe pass)
    int over[4];                     // state wave w left the fp16 range in the first pass
};

// A fragment of a k-step over U rows (Kt^T, P) times the U factor of the
// state wave that owns the lane's rows (2 ks + sub / 2), in the range-safe
// pass.
__device__ __forceinline__ f16x8 scale_frag(f16x8 a, float f) {
    const _Float16 h = static_cast<_Float16>(f);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = a[e] * h;
    return a;
}

struct ScanCtx {
    const PrefillParams* p;
    ScanShared* sh;
    const char* wsh;             // workspace block of the sequence's first chunk, this head
    int64_t head_stride;         // bytes between consecutive chunks of this head
    int nch, len, t0, b, h, col0, cstart;
    int wave, sub, l16;
};

struct OpsState {                // operands of a state wave for one chunk
    f16x8 w[4];                  // -W rows 16w.., k-steps 0..3 (fp16)
    f16x8 kt[2][2];              // Kt^T rows 32w + 16 mi.., k-steps 0..1 (fp16)
    float up[4];                 // U' rows 16w + 4 sub + i, this lane's column
    float4 gl[2];                // e^G_last of this lane's state rows
};
struct OpsOut {                  // operands of an output wave for one chunk
    f16x8 qt[4];                 // Qt rows 16j.., k-steps 0..3 (fp16)
    f16x8 pp[2];                 // P rows 16j.., k-steps 0..1 (fp16)
};

template <typename T>
__device__ __forceinline__ T ldws(const char* base, uint32_t off) {
    return *reinterpret_cast<const T*>(base + off);
}

__device__ __forceinline__ uint32_t frag_off(int tile, const ScanCtx& x) {
    return (tile * 64 + x.l16 + 16 * x.sub) * 16;
}

__device__ __forceinline__ void load_u_side(OpsState& o, const char* cb, const ScanCtx& x) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) o.w[ks] = ldws<f16x8>(cb, OFF_W + frag_off(x.wave * 4 + ks, x));
    const float4 u = ldws<float4>(cb, OFF_UP + frag_off(x.wave * (V / 16) + x.col0 / 16, x));
    o.up[0] = u.x; o.up[1] = u.y; o.up[2] = u.z; o.up[3] = u.w;
}

__device__ __forceinline__ void load_s_side(OpsState& o, const char* cb, const ScanCtx& x) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            o.kt[mi][ks] = ldws<f16x8>(cb, OFF_KT + frag_off((2 * x.wave + mi) * 2 + ks, x));
        }
        o.gl[mi] = ldws<float4>(cb, OFF_GL + (32 * x.wave + 16 * mi + 4 * x.sub) * 4);
    }
}

// Operands of chunk c+1 are loaded, into the other of two register sets,
// right after chunk c's products that use the same operand group were
// issued: the loads never overwrite registers an MFMA in flight still
// reads, each has about a chunk step to arrive, and no wait covers a load
// issued after the value it waits for.
// kSafe selects the arithmetic for states and corrected values beyond the
// fp16 range (see the range notes in kda_prefill_mfma.h); without it the
// pass only notes, in `over`, whether any |S| or |U| of a live step reached
// 2^15 (off the critical path: the conversions do not wait for the test).
template <bool kInter, bool kSafe>
__device__ void scan_state_waves(const ScanCtx& x, f32x4_t* S, bool& over) {
    const PrefillParams& p = *x.p;
    ScanShared* sh = x.sh;
    int buf = 0;
    auto step = [&](const OpsState& o, OpsState& nx, int cc) {
        // next chunk's operands; the last step re-reads its own chunk so the
        // prefetch is unconditional (a conditional load would make every
        // later wait cover it on both paths)
        const char* nxt = x.wsh + (int64_t)min(cc + 1, x.nch - 1) * x.head_stride;
        const bool live = cc < x.nch;            // false for the padding step of an odd count
        if (kInter && live) {
            float* dst = p.inter + ((int64_t)(x.cstart + cc) * p.HV + x.h) * (int64_t)V * K +
                         (int64_t)(x.col0 + x.l16) * K + 32 * x.wave + 4 * x.sub;
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                *reinterpret_cast<float4*>(dst + 16 * mi) = make_float4(S[mi][0], S[mi][1], S[mi][2], S[mi][3]);
        }
        float ms = 0.f;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int i = 0; i < 4; ++i) ms = fmaxf(ms, fabsf(S[mi][i]));
        // S (fp16) -> LDS, transposed; the safe pass scales the wave's block
        // into the fp16 range and publishes the factor
        float fS = 1.0f;
        if constexpr (kSafe) {
            const int eS = range_exp(wave_max_nonneg(ms), kMaxExpS);
            fS = pow2f(-eS);
            if (x.l16 == 0 && x.sub == 0) sh->sc[buf][x.wave] = pow2f(eS);
        } else {
            over |= live && ms >= kRangeLimit;
        }
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            const f16x4 v4 = {static_cast<_Float16>(S[mi][0] * fS), static_cast<_Float16>(S[mi][1] * fS),
                              static_cast<_Float16>(S[mi][2] * fS), static_cast<_Float16>(S[mi][3] * fS)};
            *reinterpret_cast<f16x4*>(&sh->St[buf][x.l16 * LDS_S + 32 * x.wave + 16 * mi + 4 * x.sub]) = v4;
        }
        lds_barrier();
        // (phase fences: the scheduler would otherwise hoist the state
        // update's S * e^G_last next to the just-issued load of e^G_last)
        __builtin_amdgcn_sched_barrier(0);
        f32x4_t U;
        if constexpr (!kSafe) {
            // U = U' + (-W) S, rows 16w..16w+15 (two independent accumulator chains)
            f32x4_t Ua = {o.up[0], o.up[1], o.up[2], o.up[3]}, Ub = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ks += 2) {
                const f16x8 sa = *reinterpret_cast<const f16x8*>(&sh->St[buf][x.l16 * LDS_S + 32 * ks + 8 * x.sub]);
                const f16x8 sb = *reinterpret_cast<const f16x8*>(&sh->St[buf][x.l16 * LDS_S + 32 * ks + 32 + 8 * x.sub]);
                Ua = mfma16(o.w[ks], sa, Ua);
                Ub = mfma16(o.w[ks + 1], sb, Ub);
            }
            U = Ua + Ub;
        } else {
            // U = U' + sum_ks 2^e_S[ks] (-W_ks) S~_ks: one accumulator per
            // k-step (the rows of one state wave), factors on the fp32 sums
            const float4 es = *reinterpret_cast<const float4*>(&sh->sc[buf][0]);
            f32x4_t acc4[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const f16x8 sv = *reinterpret_cast<const f16x8*>(&sh->St[buf][x.l16 * LDS_S + 32 * ks + 8 * x.sub]);
                acc4[ks] = mfma16(o.w[ks], sv, f32x4_t{0.f, 0.f, 0.f, 0.f});
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                U[i] = fmaf(es.w, acc4[3][i],
                            fmaf(es.z, acc4[2][i], fmaf(es.y, acc4[1][i], fmaf(es.x, acc4[0][i], o.up[i]))));
        }
        load_u_side(nx, nxt, x);
        float mu = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) mu = fmaxf(mu, fabsf(U[i]));
        float fU = 1.0f;
        if constexpr (kSafe) {
            const int eU = range_exp(wave_max_nonneg(mu), kMaxExpU);
            fU = pow2f(-eU);
            if (x.l16 == 0 && x.sub == 0) sh->sc[buf][4 + x.wave] = pow2f(eU);
        } else {
            over |= live && mu >= kRangeLimit;
        }
        f16x4 uh, ul;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float us = U[i] * fU;
            uh[i] = static_cast<_Float16>(us);
            ul[i] = static_cast<_Float16>(us - static_cast<float>(uh[i]));
        }
        *reinterpret_cast<f16x4*>(&sh->Uh[buf][x.l16 * LDS_U + 16 * x.wave + 4 * x.sub]) = uh;
        *reinterpret_cast<f16x4*>(&sh->Ul[buf][x.l16 * LDS_U + 16 * x.wave + 4 * x.sub]) = ul;
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // S <- e^G_last * S + Kt^T (U_hi + U_lo) (fp16 products; in the safe
        // pass Kt^T carries the U factors of the rows it meets)
        f16x8 ubh[2], ubl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            ubh[ks] = *reinterpret_cast<const f16x8*>(&sh->Uh[buf][x.l16 * LDS_U + 32 * ks + 8 * x.sub]);
            ubl[ks] = *reinterpret_cast<const f16x8*>(&sh->Ul[buf][x.l16 * LDS_U + 32 * ks + 8 * x.sub]);
        }
        f16x8 kt[2][2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) kt[mi][ks] = o.kt[mi][ks];
        if constexpr (kSafe) {
            const float4 eu = *reinterpret_cast<const float4*>(&sh->sc[buf][4]);
            const float f0 = x.sub < 2 ? eu.x : eu.y, f1 = x.sub < 2 ? eu.z : eu.w;
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                kt[mi][0] = scale_frag(kt[mi][0], f0);
                kt[mi][1] = scale_frag(kt[mi][1], f1);
            }
        }
        // four independent chains of two (tile mi, k-step ks), summed at the end
        f32x4_t acc[2][2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            acc[mi][0] = f32x4_t{S[mi][0] * o.gl[mi].x, S[mi][1] * o.gl[mi].y,
                                 S[mi][2] * o.gl[mi].z, S[mi][3] * o.gl[mi].w};
            acc[mi][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) acc[mi][ks] = mfma16(kt[mi][ks], ubh[ks], acc[mi][ks]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) acc[mi][ks] = mfma16(kt[mi][ks], ubl[ks], acc[mi][ks]);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            const f32x4_t sn = acc[mi][0] + acc[mi][1];
            S[mi] = live ? sn : S[mi];
        }
        load_s_side(nx, nxt, x);
        buf = buf + 1 == kBufs ? 0 : buf + 1;
    };
    if (x.nch <= 0) return;                  // empty sequence: no chunk, no workspace read
    OpsState oa, ob;
    load_u_side(oa, x.wsh, x);
    load_s_side(oa, x.wsh, x);
    // Steps run in pairs with no branch inside (a conditional step would
    // make the waits at the loop head cover loads issued for the next
    // chunk); for an odd count the last step of the last pair is padding:
    // it re-reads the last chunk, keeps S and stores nothing.  The output
    // waves run the same number of steps (same barriers).
    for (int cc = 0; cc < x.nch; cc += 2) {
        step(oa, ob, cc);
        step(ob, oa, cc + 1);
    }
}

// Output rows 16j..16j+15 of chunk c: Qt S (after S of chunk c is
// published), then P U and the stores (after U of chunk c is published).
template <bool kSafe>
__device__ __forceinline__ f32x4_t output_qs(const ScanCtx& x, const OpsOut& o, int buf) {
    const ScanShared* sh = x.sh;
    if constexpr (!kSafe) {
        f32x4_t Oa = {0.f, 0.f, 0.f, 0.f}, Ob = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ks += 2) {
            const f16x8 sa = *reinterpret_cast<const f16x8*>(&sh->St[buf][x.l16 * LDS_S + 32 * ks + 8 * x.sub]);
            const f16x8 sb = *reinterpret_cast<const f16x8*>(&sh->St[buf][x.l16 * LDS_S + 32 * ks + 32 + 8 * x.sub]);
            Oa = mfma16(o.qt[ks], sa, Oa);
            Ob = mfma16(o.qt[ks + 1], sb, Ob);
        }
        return Oa + Ob;
    } else {
        const float4 es = *reinterpret_cast<const float4*>(&sh->sc[buf][0]);
        f32x4_t acc4[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const f16x8 sv = *reinterpret_cast<const f16x8*>(&sh->St[buf][x.l16 * LDS_S + 32 * ks + 8 * x.sub]);
            acc4[ks] = mfma16(o.qt[ks], sv, f32x4_t{0.f, 0.f, 0.f, 0.f});
        }
        f32x4_t O;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            O[i] = fmaf(es.w, acc4[3][i], fmaf(es.z, acc4[2][i], fmaf(es.y, acc4[1][i], es.x * acc4[0][i])));
        return O;
    }
}

// Raw buffer descriptor word 3 for gfx9-family raw (untyped) buffers.
constexpr int kBufferWord3 = 0x00020000;

// Output rows of chunk c go out through a buffer descriptor whose record
// count ends at the chunk's last valid row: the stores are unconditional
// (no branch for the wait analysis to merge) and the hardware drops the
// ones past a partial or padding chunk.
// PKS: k-steps of P the wave's rows need (P is lower triangular: rows
// 0..31 have zeros in columns 32..63).
template <typename TIn, int PKS, bool kSafe>
__device__ __forceinline__ void output_pu_store(const ScanCtx& x, const OpsOut& o, f32x4_t O, int buf, int c) {
    static_assert(sizeof(TIn) == 2, "the MFMA path writes bf16 outputs");
    const PrefillParams& p = *x.p;
    const ScanShared* sh = x.sh;
    f16x8 pp[PKS];
#pragma unroll
    for (int ks = 0; ks < PKS; ++ks) pp[ks] = o.pp[ks];
    if constexpr (kSafe) {          // P carries the U factors of the rows it meets
        const float4 eu = *reinterpret_cast<const float4*>(&sh->sc[buf][4]);
        const float fk[2] = {x.sub < 2 ? eu.x : eu.y, x.sub < 2 ? eu.z : eu.w};
#pragma unroll
        for (int ks = 0; ks < PKS; ++ks) pp[ks] = scale_frag(pp[ks], fk[ks]);
    }
#pragma unroll
    for (int ks = 0; ks < PKS; ++ks) {
        const f16x8 ub = *reinterpret_cast<const f16x8*>(&sh->Uh[buf][x.l16 * LDS_U + 32 * ks + 8 * x.sub]);
        O = mfma16(pp[ks], ub, O);
    }
    const int clen = min(C, x.len - c * C);
    const int rs = static_cast<int>(p.os[1]);          // row stride, elements (bounded on the host)
    TIn* base = static_cast<TIn*>(p.o) + x.b * p.os[0] + x.h * p.os[2] + x.col0 +
                (int64_t)(x.t0 + c * C) * p.os[1];
    const int records = clen > 0 ? ((clen - 1) * rs + VS) * 2 : 0;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(base, 0, records, kBufferWord3);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * (x.wave - 4) + 4 * x.sub + i;
        const int off = r < clen ? (r * rs + x.l16) * 2 : 0x7ffffff0;
        const __bf16 v = tobf(p.scale * O[i]);
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), rsrc, off, 0, 0);
    }
}

__device__ __forceinline__ void load_qt(OpsOut& o, const char* cb, const ScanCtx& x) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) o.qt[ks] = ldws<f16x8>(cb, OFF_QT + frag_off((x.wave - 4) * 4 + ks, x));
}

template <int PKS>
__device__ __forceinline__ void load_p(OpsOut& o, const char* cb, const ScanCtx& x) {
#pragma unroll
    for (int ks = 0; ks < PKS; ++ks) o.pp[ks] = ldws<f16x8>(cb, OFF_P + frag_off((x.wave - 4) * 2 + ks, x));
}

template <typename TIn, int PKS, bool kSafe>
__device__ void scan_output_waves(const ScanCtx& x) {
    if (x.nch <= 0) return;
    int buf = 0;
    auto step = [&](const OpsOut& cur, OpsOut& nx, int cc) {
        const char* nxt = x.wsh + (int64_t)min(cc + 1, x.nch - 1) * x.head_stride;
        lds_barrier();                                   // S of chunk cc published
        const f32x4_t O = output_qs<kSafe>(x, cur, buf);
        load_qt(nx, nxt, x);
        load_p<PKS>(nx, nxt, x);
        lds_barrier();                                   // U of chunk cc published
        output_pu_store<TIn, PKS, kSafe>(x, cur, O, buf, cc);   // no rows for a padding step
        buf = buf + 1 == kBufs ? 0 : buf + 1;
    };
    OpsOut oa, ob;
    load_qt(oa, x.wsh, x);
    load_p<PKS>(oa, x.wsh, x);
    // wait once for the first chunk's operands: left pending into the loop,
    // they would make the loop-head wait cover every store and prefetch
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    for (int cc = 0; cc < x.nch; cc += 2) {              // same steps as the state waves
        step(oa, ob, cc);
        step(ob, oa, cc + 1);
    }
}

// One scan block: run s of the two-level scan (a whole sequence when runs
// are not used), head h, state columns [col0, col0 + 16).  Blocks of one
// (run, head) pair share a block index modulo 8; MI355X deals consecutive
// blocks round-robin over its 8 XCDs, so the 8 blocks of a pair share one L2
// and each chunk's workspace leaves HBM once per pair.  A sequence of one
// run starts from its pool slot; otherwise every run starts from its entry
// state in the run area (passes A and B), and only the last run writes the
// final state back to the slot.
// kClaim: the block claims its compute unit's whole register file (its
// eight waves are declared at 256 VGPRs, two per SIMD), so no wave of
// another kernel running at the same time (another phase on another
// stream) is placed beside it.  The scan is bound by its CU's vector-memory
// path (~58 KB of operands per chunk step), and waves of a streaming kernel
// sharing that path slowed it 2.5x; the launch claims the CUs only when the
// grid has at most one block per CU, where the claim costs nothing.
template <typename TIn, bool kInter, bool kClaim>
__global__ __launch_bounds__(64 * kScanWaves) void scan_mfma_kernel(const PrefillParams p) {
    __shared__ __attribute__((aligned(16))) ScanShared sh;
    __shared__ int s_run[10];
    if constexpr (kClaim) asm volatile("" ::: "v255");    // register allocation reaches v255: 256 VGPRs

    const int blk = blockIdx.x;
    const int xcd = blk & 7;
    const int jdx = blk >> 3;
    const int vsl = jdx % NVS;
    const int unit = (jdx / NVS) * 8 + xcd;        // (run, head) pair
    if (unit >= p.max_segs * p.HV) return;
    ScanCtx x;
    x.p = &p;
    x.sh = &sh;
    x.h = unit % p.HV;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    x.wave = tid >> 6;
    x.sub = lane >> 4;
    x.l16 = lane & 15;
    x.col0 = vsl * VS;

    SegInfo g;
    if (p.cu) {
        // one wave locates the run (wave-wide prefix sums), the others read it
        if (tid < 64) {
            const bool found = locate_segment(p, unit / p.HV, g);
            if (tid == 0) {
                s_run[0] = found;
                s_run[1] = g.n; s_run[2] = g.b; s_run[3] = g.j; s_run[4] = g.nseg;
                s_run[5] = g.t0; s_run[6] = g.len; s_run[7] = g.cs; s_run[8] = g.seg0;
            }
        }
        lds_barrier();
        if (!s_run[0]) return;
        g.n = s_run[1]; g.b = s_run[2]; g.j = s_run[3]; g.nseg = s_run[4];
        g.t0 = s_run[5]; g.len = s_run[6]; g.cs = s_run[7]; g.seg0 = s_run[8];
    } else if (!locate_segment(p, unit / p.HV, g)) {
        return;
    }
    x.b = g.b;
    x.t0 = g.t0;
    x.len = g.len;
    x.cstart = g.cs;
    x.nch = min(ceil_div(x.len, C), max(p.max_chunks - g.cs, 0));
    const int slot = p.idx[g.n];
    if (slot < 0 || slot >= p.num_slots) return;
    if (g.nseg > 1 && g.seg0 + g.nseg > p.max_segs) return;   // only a malformed cu_seqlens gets here
    x.head_stride = (int64_t)p.HV * CHUNK_BYTES;
    x.wsh = reinterpret_cast<const char*>(p.ws) + ((int64_t)g.cs * p.HV + x.h) * CHUNK_BYTES;

    // A block whose state or corrected values left the fp16 range in its
    // first pass (some wave noted |S| or |U| >= 2^15) writes no final state
    // and runs its chunks again with the range-safe arithmetic; every wave
    // learns it at one more barrier after the first pass.
    if (x.wave >= 4) {
        // output rows 0..31 (waves 4, 5) see only the first 32 columns of P
        if (x.wave >= 6) scan_output_waves<TIn, 2, false>(x);
        else scan_output_waves<TIn, 1, false>(x);
        lds_barrier();
        if (sh.over[0] | sh.over[1] | sh.over[2] | sh.over[3]) {
            if (x.wave >= 6) scan_output_waves<TIn, 2, true>(x);
            else scan_output_waves<TIn, 1, true>(x);
        }
        return;
    }
    // state rows 32w + 16 mi + 4 sub + i, column col0 + l16 (S^T layout, as in the pool)
    const int64_t row_off = (int64_t)(x.col0 + x.l16) * K + 32 * x.wave + 4 * x.sub;
    float* pool_row = p.pool + ((int64_t)slot * p.HV + x.h) * (int64_t)V * K + row_off;
    const float* src = pool_row;
    if (g.nseg > 1)
        src = reinterpret_cast<const float*>(reinterpret_cast<const char*>(p.ws) + p.seg_off +
                                             ((int64_t)(g.seg0 + g.j) * p.HV + x.h) * SEG_BYTES + SEG_OFF_SIN) + row_off;
    f32x4_t S[2];
    auto load_state = [&]() {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            const float4 s0 = *reinterpret_cast<const float4*>(src + 16 * mi);
            S[mi] = f32x4_t{s0.x, s0.y, s0.z, s0.w};
        }
        // wait for the state here, once: left pending into the chunk loop, its
        // registers would make the loop-head wait cover every prefetch in flight
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    };
    load_state();
    bool over = false;
    scan_state_waves<kInter, false>(x, S, over);
    const bool wave_over = __ballot(over) != 0;      // every lane of the wave takes part
    if (lane == 0) sh.over[x.wave] = wave_over;
    lds_barrier();
    if (sh.over[0] | sh.over[1] | sh.over[2] | sh.over[3]) {
        load_state();
        scan_state_waves<kInter, true>(x, S, over);
    }
    if (g.j == g.nseg - 1) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
            *reinterpret_cast<float4*>(pool_row + 16 * mi) = make_float4(S[mi][0], S[mi][1], S[mi][2], S[mi][3]);
    }
}


// Chunks per run of the two-level scan (0: one run per sequence).  The
// default is one run: measured on the 16 x 128 workloads (1 x 4096, 1 x 8192,
// packed 8192) the composition of the run maps (pass A) cost more than the
// parallel runs saved over the single sequential scan.  A run longer than
// the longest possible sequence is one run as well.
int run_chunks(const kda_prefill_args& a) {
    const int64_t nch_bound = (a.T + C - 1) / C;     // chunks of the longest possible sequence
    if (a.run_chunks <= 0 || a.run_chunks >= nch_bound) return 0;
    return a.run_chunks;
}

int64_t max_runs(const kda_prefill_args& a, int L) {
    if (L <= 0) return a.num_seqs;
    if (a.cu_seqlens) return a.T / (C * L) + a.num_seqs;
    const int64_t nch = (a.T + C - 1) / C;
    return a.B * ((nch + L - 1) / L);
}

int64_t chunk_area_bytes(const kda_prefill_args& a) { return prefill_max_chunks(a) * a.HV * CHUNK_BYTES; }

template <typename TIn>
hipError_t launch_t(const kda_prefill_args& a, const PrefillParams& p, hipStream_t s) {
    const int64_t nchunks = prefill_max_chunks(a);
    // persistent prep blocks: two per compute unit (LDS-bound), at most one per item
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const int64_t items = nchunks * a.HV;
    const int64_t prep_blocks = items < 2 * (int64_t)cus ? items : 2 * (int64_t)cus;
    klaunch(prep_mfma_kernel<TIn>, dim3(static_cast<unsigned>(prep_blocks)), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.seg_len > 0) {
        if ((e = launch_seg_state(p, s)) != hipSuccess) return e;
        // a chain exists only where a sequence can have three runs or more
        if ((a.T + C - 1) / C > 2 * (int64_t)p.seg_len && (e = launch_seg_chain(p, s)) != hipSuccess) return e;
    }
    const int64_t units = (int64_t)p.max_segs * a.HV;
    const int64_t nblk = (units + 7) / 8 * 8 * NVS;     // whole groups of 8 pairs, see scan_mfma_kernel
    const dim3 grid(static_cast<unsigned>(nblk)), block(64 * kScanWaves);
    const bool claim = nblk <= cus;                     // one block per CU at most
    if (p.inter) {
        if (claim) klaunch(scan_mfma_kernel<TIn, true, true>, grid, block, 0, s, p);
        else klaunch(scan_mfma_kernel<TIn, true, false>, grid, block, 0, s, p);
    } else {
        if (claim) klaunch(scan_mfma_kernel<TIn, false, true>, grid, block, 0, s, p);
        else klaunch(scan_mfma_kernel<TIn, false, false>, grid, block, 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace

bool prefill_mfma_eligible(const kda_prefill_args& a) {
    // bf16 activations only: float32 inputs keep the float32 path, whose
    // results stay within 1e-4 of the fp64 recurrence
    if (a.dtype != KDA_BF16 || a.chunk_size != C || a.K != K || a.V != V) return false;
    // a positive lower bound makes every log-decay positive: the decay
    // factors would leave the fp16 operands' range, so the float32 path
    if (a.A_log != nullptr && a.has_lower_bound && a.lower_bound > 0.0f) return false;
    const int elem = 2;
    // 16-byte row loads of q, k, g and v; dt_bias rows are 16-byte aligned (host check)
    // output rows are addressed with 32-bit byte offsets inside a chunk
    if (a.o_stride[1] < VS || a.o_stride[1] > (1 << 22)) return false;
    return aligned_rows(a.q, a.q_stride, 3, elem) && aligned_rows(a.k, a.k_stride, 3, elem) &&
           aligned_rows(a.g, a.g_stride, 3, elem) && aligned_rows(a.v, a.v_stride, 3, elem);
}

size_t prefill_mfma_workspace_bytes(const kda_prefill_args& a) {
    const int L = run_chunks(a);
    const int64_t runs = L > 0 ? max_runs(a, L) * a.HV * SEG_BYTES : 0;
    return static_cast<size_t>(chunk_area_bytes(a) + runs);
}

hipError_t launch_prefill_mfma(const kda_prefill_args& a, const PrefillParams& p0, hipStream_t s) {
    PrefillParams p = p0;
    p.seg_len = run_chunks(a);
    p.max_segs = static_cast<int>(max_runs(a, p.seg_len));
    p.seg_off = chunk_area_bytes(a);
    return launch_t<bf16>(a, p, s);     // eligibility requires bf16 activations
}

}  // namespace kda
