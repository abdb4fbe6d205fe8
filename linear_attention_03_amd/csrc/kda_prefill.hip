// Chunked prefill (A1-A6) in two launches.
//
// prep (one block per chunk x head, all chunks in parallel): loads the
//   chunk's tokens, applies the L2 norm, the gate map and beta (A2), the
//   in-chunk cumulative log-decay G (A3), the gated Grams
//     A[r,j] = beta_r sum_c k_rc k_jc exp(G_rc - G_jc)   (j < r)
//     P[r,j] =        sum_c q_rc k_jc exp(G_rc - G_jc)   (j <= r)   (A4)
//   and the forward substitution (I + A) [W | U'] = diag(beta) [K e^G | V]
//   (A5).  It stores W, U', P, Qt = Q e^G, Kt = K e^(G_last - G) (as
//   Kt^T) and e^G_last in the workspace, in the scan's read order (ws_run,
//   ws_tile in kda_prefill_common.h).
// scan (one block per sequence x head x 16 state columns, on fp32 matrix
//   tiles; kda_prefill_scan32.hip): walks the sequence's chunks in order (A6):
//     U = U' - W S;  O = scale (Qt S + P U);  S <- e^G_last * S + Kt^T U
//   and writes S back to the sequence's pool slot.
//
// exp(G_r - G_j) is evaluated per element with r >= j, so its argument is
// <= 0 and nothing overflows however strong the decay.  Chunks never
// straddle sequences; rows past a chunk's last token are zero.
// Entry checks follow chunk_kda in the 35197 report (key code snippets):
// the indexed pool is required and gate / beta rows >= T are never read.

#include "kda_prefill_common.h"

namespace kda {
namespace {


template <typename TIn, int C, int K, int V>
__global__ __launch_bounds__(256) void prep_kernel(const PrefillParams p) {
    if (p.flags && p.flags[blockIdx.x] == 0) return;     // done by the matrix-core prep
    constexpr int KP = K + 1;                       // padded LDS row
    constexpr int QA = C * KP > C * C ? C * KP : C * C;
    __shared__ float s_q[QA];                       // q-hat, later A [C][C]
    __shared__ float s_k[C * KP];                   // k-hat
    __shared__ float s_G[C * KP];                   // g, then cumulative G
    __shared__ float s_beta[C];

    const int blk = blockIdx.x;
    const int h = blk % p.HV;
    const int ci = blk / p.HV;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

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

    const int hq = h / p.group;          // q/k head of this value head
    const TIn* qg = static_cast<const TIn*>(p.q) + b * p.qs[0] + hq * p.qs[2];
    const TIn* kg = static_cast<const TIn*>(p.k) + b * p.ks[0] + hq * p.ks[2];
    const TIn* gg = static_cast<const TIn*>(p.g) + b * p.gs[0] + h * p.gs[2];
    const TIn* bg = static_cast<const TIn*>(p.beta) + b * p.bs[0] + h;
    const int gmode = p.gate;
    const float expA = gmode != kGateRaw ? __expf(p.A_log[h]) : 0.0f;

    // A2: per-token preprocessing, one wave per row
    for (int r = wave; r < C; r += 4) {
        const bool valid = r < len;
        const int64_t t = t0 + r;
        float qv[(K + 63) / 64], kv[(K + 63) / 64];
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int m = 0; m < (K + 63) / 64; ++m) {
            const int c = lane + 64 * m;
            qv[m] = (valid && c < K) ? ld(qg, t * p.qs[1] + c) : 0.0f;
            kv[m] = (valid && c < K) ? ld(kg, t * p.ks[1] + c) : 0.0f;
            sq += qv[m] * qv[m];
            sk += kv[m] * kv[m];
        }
        float rq = 1.0f, rk = 1.0f;
        if (p.l2norm) {
            rq = rsqrtf(group_sum<64>(sq) + kL2Eps);
            rk = rsqrtf(group_sum<64>(sk) + kL2Eps);
        }
#pragma unroll
        for (int m = 0; m < (K + 63) / 64; ++m) {
            const int c = lane + 64 * m;
            if (c < K) {
                s_q[r * KP + c] = qv[m] * rq;
                s_k[r * KP + c] = kv[m] * rk;
                float gl = 0.0f;
                if (valid) {
                    const float dt = p.dt_bias ? p.dt_bias[h * K + c] : 0.0f;
                    gl = log_gate(ld(gg, t * p.gs[1] + c), gmode, expA, dt, p.lb);
                }
                s_G[r * KP + c] = gl;
            }
        }
        if (lane == 0) {
            float bt = valid ? ld(bg, t * p.bs[1]) : 0.0f;
            if (valid && p.beta_is_raw) bt = sigmoidf(bt);
            s_beta[r] = bt;
        }
    }
    __syncthreads();

    float* ws = p.ws + ((int64_t)ci * p.HV + h) * p.chunk_floats;
    float* W = ws;
    float* Up = W + C * K;
    float* P = Up + C * V;
    float* Qt = P + C * C;
    float* Kt = Qt + C * K;
    float* gl_out = Kt + C * K;

    // A3: cumulative log-decay per channel
    if (tid < K) {
        float acc = 0.0f;
        for (int r = 0; r < C; ++r) {
            acc += s_G[r * KP + tid];
            s_G[r * KP + tid] = acc;
        }
        gl_out[tid] = __expf(acc);
    }
    __syncthreads();

    for (int e = tid; e < C * K; e += 256) {
        const int r = e / K, c = e % K;
        const float G = s_G[r * KP + c];
        const float Gl = s_G[(C - 1) * KP + c];
        Qt[ws_run(r, c, K)] = s_q[r * KP + c] * __expf(G);
        Kt[ws_run(c, r, C)] = s_k[r * KP + c] * __expf(Gl - G);    // Kt^T
    }

    // A4: gated Grams; A stays in registers until q-hat is no longer needed
    constexpr int EPT = (C * C + 255) / 256;
    float a_reg[EPT];
#pragma unroll
    for (int m = 0; m < EPT; ++m) {
        const int e = tid + 256 * m;
        float av = 0.f, pv = 0.f;
        if (e < C * C) {
            const int r = e / C, jj = e % C;
            if (jj <= r) {
                for (int c = 0; c < K; ++c) {
                    const float ex = __expf(s_G[r * KP + c] - s_G[jj * KP + c]);
                    const float kj = s_k[jj * KP + c] * ex;
                    av = fmaf(s_k[r * KP + c], kj, av);
                    pv = fmaf(s_q[r * KP + c], kj, pv);
                }
            }
            P[ws_run(r, jj, C)] = pv;
            a_reg[m] = jj < r ? av * s_beta[r] : 0.0f;
        }
    }
    __syncthreads();
    float* s_A = s_q;                              // [C][C], row stride C
#pragma unroll
    for (int m = 0; m < EPT; ++m) {
        const int e = tid + 256 * m;
        if (e < C * C) s_A[e] = a_reg[m];
    }
    __syncthreads();

    // A5: forward substitution, one thread per column of [W | U'], in
    // blocks of 16 rows kept in registers; rows of earlier blocks are read
    // back from the thread's own column of the output.
    if (tid < K + V) {
        const bool is_w = tid < K;
        const int col = is_w ? tid : tid - K;
        const TIn* vg = static_cast<const TIn*>(p.v) + b * p.vs[0] + h * p.vs[2] + col;
        // element (row, col) of this thread's column of W or U'
        auto at = [&](int row) -> float& { return is_w ? W[ws_run(row, col, K)] : Up[ws_tile(row, col, V)]; };
        for (int r0 = 0; r0 < C; r0 += 16) {
            float x[16];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int r = r0 + rr;
                float acc;
                if (is_w) acc = s_beta[r] * s_k[r * KP + col] * __expf(s_G[r * KP + col]);
                else acc = r < len ? s_beta[r] * ld(vg, (int64_t)(t0 + r) * p.vs[1]) : 0.0f;
                for (int jj = 0; jj < r0; ++jj) acc = fmaf(-s_A[r * C + jj], at(jj), acc);
#pragma unroll
                for (int q2 = 0; q2 < rr; ++q2) acc = fmaf(-s_A[r * C + r0 + q2], x[q2], acc);
                x[rr] = acc;
            }
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) at(r0 + rr) = x[rr];
        }
    }
}

int64_t chunk_floats_rt(const kda_prefill_args& a) {
    return a.chunk_size * (3 * a.K + a.V + a.chunk_size) + a.K;
}

int64_t chunk_area_floats(const kda_prefill_args& a) { return prefill_max_chunks(a) * a.HV * chunk_floats_rt(a); }

// Byte offset of the general path's store sink in its workspace: after the
// chunk area and the flags, 256-byte aligned.
size_t general_sink_offset(const kda_prefill_args& a) {
    size_t bytes = static_cast<size_t>(chunk_area_floats(a)) * sizeof(float);
    bytes += static_cast<size_t>(prefill_max_chunks(a) * a.HV) * sizeof(int);   // flags of the fp32-tile prep
    return (bytes + 255) / 256 * 256;
}

// The fp32 matrix-core prep (chunk 64 or 16), then the exact prep for the
// chunks it flagged (their blocks return at once otherwise; not launched
// when no chunk can be flagged).
template <typename TIn, int C, int K, int V>
hipError_t launch_ckv(const kda_prefill_args& a, const PrefillParams& p0, hipStream_t s) {
    const int64_t nchunks = prefill_max_chunks(a);
    PrefillParams p = p0;
    hipError_t e;
    p.flags = reinterpret_cast<int*>(p.ws + chunk_area_floats(a));
    p.sink = reinterpret_cast<float*>(reinterpret_cast<char*>(p.ws) + general_sink_offset(a));
    if constexpr (C == 64) e = launch_prep32<TIn, K, V>(a, p, s);
    else e = launch_prep16<TIn, K, V>(a, p, s);
    if (e != hipSuccess) return e;
    // A bounded gate with lower_bound in [-8.75, 0] gives no positive
    // log-decay, and every span the fp32-tile prep checks (|G_r - G_m|, at
    // most 8 rows from a reference row) stays below 70 < 80: it flags no
    // chunk, and the exact prep's blocks would all return at once.
    const bool may_flag = !(p.gate == kGateBounded && p.lb <= 0.0f && p.lb >= -8.75f);
    if (may_flag) {
        klaunch(prep_kernel<TIn, C, K, V>, dim3(static_cast<unsigned>(nchunks * a.HV)), dim3(256), 0, s, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_scan32<TIn, C, K, V>(a, p, s);
}

template <typename TIn, int C, int K>
hipError_t launch_ck(const kda_prefill_args& a, const PrefillParams& p, hipStream_t s) {
    switch (a.V) {
        case 32: return launch_ckv<TIn, C, K, 32>(a, p, s);
        case 64: return launch_ckv<TIn, C, K, 64>(a, p, s);
        default: return launch_ckv<TIn, C, K, 128>(a, p, s);
    }
}

template <typename TIn, int C>
hipError_t launch_c(const kda_prefill_args& a, const PrefillParams& p, hipStream_t s) {
    switch (a.K) {
        case 32: return launch_ck<TIn, C, 32>(a, p, s);
        case 64: return launch_ck<TIn, C, 64>(a, p, s);
        default: return launch_ck<TIn, C, 128>(a, p, s);
    }
}

template <typename TIn>
hipError_t launch_t(const kda_prefill_args& a, const PrefillParams& p, hipStream_t s) {
    return a.chunk_size == 16 ? launch_c<TIn, 16>(a, p, s) : launch_c<TIn, 64>(a, p, s);
}

}  // namespace

int64_t prefill_max_chunks(const kda_prefill_args& a) {
    const int64_t C = a.chunk_size;
    if (a.cu_seqlens) return a.T / C + a.num_seqs;
    return a.B * ((a.T + C - 1) / C);
}

size_t prefill_workspace_bytes(const kda_prefill_args& a) {
    if (prefill_mfma_eligible(a)) return prefill_mfma_workspace_bytes(a);
    return general_sink_offset(a) + 256 * sizeof(float);
}

hipError_t launch_prefill(const kda_prefill_args& a, void* workspace, hipStream_t s) {
    PrefillParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o; p.g = a.g; p.beta = a.beta;
    for (int i = 0; i < 3; ++i) {
        p.qs[i] = a.q_stride[i]; p.ks[i] = a.k_stride[i]; p.vs[i] = a.v_stride[i];
        p.os[i] = a.o_stride[i]; p.gs[i] = a.g_stride[i];
    }
    p.bs[0] = a.beta_stride[0]; p.bs[1] = a.beta_stride[1];
    p.A_log = a.A_log; p.dt_bias = a.dt_bias; p.lb = a.lower_bound; p.scale = a.scale;
    p.gate = gate_mode(a.A_log, a.has_lower_bound); p.beta_is_raw = a.beta_is_raw; p.l2norm = a.use_qk_l2norm;
    p.group = static_cast<int>(a.HV / a.H);
    p.T = static_cast<int>(a.T); p.HV = static_cast<int>(a.HV); p.num_seqs = static_cast<int>(a.num_seqs);
    p.cu = a.cu_seqlens;
    p.num_slots = static_cast<int>(a.num_slots);
    p.max_chunks = static_cast<int>(prefill_max_chunks(a));
    p.pool = a.state_pool; p.idx = a.state_indices;
    p.inter = a.intermediate_states;
    p.ws = static_cast<float*>(workspace);
    p.chunk_floats = chunk_floats_rt(a);
    p.seg_len = 0;
    p.max_segs = static_cast<int>(a.num_seqs);
    p.seg_off = 0;
    p.flags = nullptr;
    p.sink = nullptr;
    if (prefill_mfma_eligible(a)) return launch_prefill_mfma(a, p, s);
    return a.dtype == KDA_BF16 ? launch_t<bf16>(a, p, s) : launch_t<float>(a, p, s);
}

}  // namespace kda
