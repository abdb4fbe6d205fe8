// Two-level scan of the matrix-core prefill: pass A (the affine map of each
// run of chunks) and pass B (the chain of run entry states).  Pass C, the
// chunk scan of every run from its entry state, is scan_mfma_kernel in
// kda_prefill_mfma.hip.
//
// The chunked form of the recurrence (chunk c of one head, entry state S)
// updates S <- D S + Kt^T (U' - W S) with D = Diag(e^G_last); per chunk the
// state map is affine, S -> (D - Kt^T W) S + Kt^T U'.  Composing the maps of
// the L chunks of a run gives S_out = M S_in + B, where M is the product of
// the chunks' linear parts and B the run's exit state from S_in = 0.  That
// is the chunk recurrence itself, applied to the K + V columns of
// Y = [I | 0]: the first K columns of the result are M and the last V are B.
// Pass A runs that recurrence for every run (except each sequence's last,
// whose map is never needed) with the first run started from the pool
// state, so that its B part is already the true entry state of run 1.
// Pass B then walks S_in(j+1) = M_j S_in(j) + B_j for j = 1 .. nseg - 2.
// Both use the operand precisions of the chunk scan: fp16 Y against fp16
// W, and Kt^T against U split into fp16 hi + lo; M enters pass B split into
// fp16 hi + lo as well, against S split the same way (three products).

#include "kda_prefill_mfma.h"

namespace kda {
namespace {

constexpr int kGroupCols = 64;              // columns of Y per pass-A block
constexpr int kGroups = (K + V) / kGroupCols;
constexpr int LDS_Y = K + 16;               // fp16 row stride of Y^T [col][k]
constexpr int LDS_UY = C + 16;              // fp16 row stride of U^T [col][r]
constexpr int LDS_MT = kGroupCols + 4;      // fp32 row stride of the M tile transpose

struct SegStateShared {
    union {
        struct {
            _Float16 Yt[kGroupCols * LDS_Y];
            _Float16 Uh[kGroupCols * LDS_UY];
            _Float16 Ul[kGroupCols * LDS_UY];
        } s;
        float Mt[K * LDS_MT];               // epilogue: this block's M columns, row-major
    };
};

struct SegOps {                             // one chunk's operands for one wave
    f16x8 w[4];                             // -W rows 16w.., k-steps 0..3
    f16x8 kt[2][2];                         // Kt^T rows 32w + 16mi.., k-steps 0..1
    float4 up[4];                           // U' rows 16w + 4sub.., col tiles 0..3 (B part only)
    float4 gl[2];                           // e^G_last of rows 32w + 16mi + 4sub..
};

// Operand loads of one chunk, in two groups issued at different points of
// the previous chunk's step (as in the chunk scan): the U side (-W, U') right
// after the previous U products, the state side (Kt^T, e^G_last) right after
// the previous state update, so each group has about half a step to arrive.
template <bool kB>
__device__ __forceinline__ void seg_load_u(SegOps& o, const char* cb, int wave, int lane, int tile0) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) o.w[ks] = *reinterpret_cast<const f16x8*>(cb + OFF_W + tile_frag(wave * 4 + ks, lane));
    if constexpr (kB) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
            o.up[nt] = *reinterpret_cast<const float4*>(cb + OFF_UP + tile_frag(wave * (V / 16) + tile0 + nt, lane));
    }
}

__device__ __forceinline__ void seg_load_s(SegOps& o, const char* cb, int wave, int lane, int sub) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            o.kt[mi][ks] = *reinterpret_cast<const f16x8*>(cb + OFF_KT + tile_frag((2 * wave + mi) * 2 + ks, lane));
        o.gl[mi] = *reinterpret_cast<const float4*>(cb + OFF_GL + (32 * wave + 16 * mi + 4 * sub) * 4);
    }
}

// One run x head x 64 columns of Y = [M | B].  Block of 4 waves; wave w
// keeps rows 32w..32w+31 of the block's columns as 2 x 4 accumulator tiles
// and computes rows 16w..16w+15 of U.  Two barriers per chunk (Y published,
// U published); the next chunk's operands are loaded during the current one.
template <bool kB>
__device__ void seg_state_run(const PrefillParams& p, SegStateShared& sh, const SegInfo& g, int h, int grp) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, sub = lane >> 4, l16 = lane & 15;
    const int col0 = kB ? (grp - K / kGroupCols) * kGroupCols : grp * kGroupCols;   // column of M or of the state
    char* seg_area = reinterpret_cast<char*>(p.ws) + p.seg_off;
    const int s_glob = g.seg0 + g.j;
    f32x4_t Y[2][4];
    if constexpr (kB) {
        if (g.j == 0) {
            // the run starts from the pool state; it is also run 0's entry
            // state for pass C (which must not read the pool slot that the
            // sequence's last run writes)
            const int slot = p.idx[g.n];
            const float* src = p.pool + ((int64_t)slot * p.HV + h) * (int64_t)V * K;
            float* sin0 = reinterpret_cast<float*>(seg_area + ((int64_t)s_glob * p.HV + h) * SEG_BYTES + SEG_OFF_SIN);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const int64_t off = (int64_t)(col0 + 16 * nt + l16) * K + 32 * wave + 16 * mi + 4 * sub;
                    const float4 v = *reinterpret_cast<const float4*>(src + off);
                    Y[mi][nt] = f32x4_t{v.x, v.y, v.z, v.w};
                    *reinterpret_cast<float4*>(sin0 + off) = v;
                }
        } else {
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) Y[mi][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    } else {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Y[mi][nt][i] = (32 * wave + 16 * mi + 4 * sub + i == col0 + 16 * nt + l16) ? 1.0f : 0.0f;
    }

    const int nch = min(ceil_div(g.len, C), max(p.max_chunks - g.cs, 0));
    if (nch <= 0) return;
    const int64_t head_stride = (int64_t)p.HV * CHUNK_BYTES;
    const char* wsh = reinterpret_cast<const char*>(p.ws) + ((int64_t)g.cs * p.HV + h) * CHUNK_BYTES;
    const int tile0 = kB ? col0 / 16 : 0;

    auto step = [&](const SegOps& o, SegOps& nx, int cc) {
        const char* nxt = wsh + (int64_t)min(cc + 1, nch - 1) * head_stride;
        const bool live = cc < nch;            // false for the padding step of an odd count
        // Y (fp16) -> LDS, transposed
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const f16x4 v4 = {static_cast<_Float16>(Y[mi][nt][0]), static_cast<_Float16>(Y[mi][nt][1]),
                                  static_cast<_Float16>(Y[mi][nt][2]), static_cast<_Float16>(Y[mi][nt][3])};
                *reinterpret_cast<f16x4*>(&sh.s.Yt[(16 * nt + l16) * LDS_Y + 32 * wave + 16 * mi + 4 * sub]) = v4;
            }
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // U = [0 | U'] + (-W) Y, rows 16w..16w+15
        f32x4_t U[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            if constexpr (kB) U[nt] = f32x4_t{o.up[nt].x, o.up[nt].y, o.up[nt].z, o.up[nt].w};
            else U[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const f16x8 b = *reinterpret_cast<const f16x8*>(&sh.s.Yt[(16 * nt + l16) * LDS_Y + 32 * ks + 8 * sub]);
                U[nt] = mfma16(o.w[ks], b, U[nt]);
            }
        seg_load_u<kB>(nx, nxt, wave, lane, tile0);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            f16x4 uh, ul;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uh[i] = static_cast<_Float16>(U[nt][i]);
                ul[i] = static_cast<_Float16>(U[nt][i] - static_cast<float>(uh[i]));
            }
            *reinterpret_cast<f16x4*>(&sh.s.Uh[(16 * nt + l16) * LDS_UY + 16 * wave + 4 * sub]) = uh;
            *reinterpret_cast<f16x4*>(&sh.s.Ul[(16 * nt + l16) * LDS_UY + 16 * wave + 4 * sub]) = ul;
        }
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // Y <- e^G_last * Y + Kt^T (U_hi + U_lo)
        f32x4_t acc[2][4];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                acc[mi][nt] = f32x4_t{Y[mi][nt][0] * o.gl[mi].x, Y[mi][nt][1] * o.gl[mi].y,
                                      Y[mi][nt][2] * o.gl[mi].z, Y[mi][nt][3] * o.gl[mi].w};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const f16x8 bh = *reinterpret_cast<const f16x8*>(&sh.s.Uh[(16 * nt + l16) * LDS_UY + 32 * ks + 8 * sub]);
                const f16x8 bl = *reinterpret_cast<const f16x8*>(&sh.s.Ul[(16 * nt + l16) * LDS_UY + 32 * ks + 8 * sub]);
#pragma unroll
                for (int mi = 0; mi < 2; ++mi) {
                    acc[mi][nt] = mfma16(o.kt[mi][ks], bh, acc[mi][nt]);
                    acc[mi][nt] = mfma16(o.kt[mi][ks], bl, acc[mi][nt]);
                }
            }
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) Y[mi][nt] = live ? acc[mi][nt] : Y[mi][nt];
        seg_load_s(nx, nxt, wave, lane, sub);
    };
    SegOps oa, ob;
    seg_load_u<kB>(oa, wsh, wave, lane, tile0);
    seg_load_s(oa, wsh, wave, lane, sub);
    // wait once for the first operands: left pending into the loop, they would
    // make the loop-head wait cover every prefetch in flight
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    for (int cc = 0; cc < nch; cc += 2) {      // pairs: no branch between steps
        step(oa, ob, cc);
        step(ob, oa, cc + 1);
    }

    if constexpr (kB) {
        // run 0: its exit state is run 1's entry state; later runs: B
        const int dst_seg = g.j == 0 ? s_glob + 1 : s_glob;
        float* dst = reinterpret_cast<float*>(seg_area + ((int64_t)dst_seg * p.HV + h) * SEG_BYTES +
                                              (g.j == 0 ? SEG_OFF_SIN : SEG_OFF_B));
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int64_t off = (int64_t)(col0 + 16 * nt + l16) * K + 32 * wave + 16 * mi + 4 * sub;
                *reinterpret_cast<float4*>(dst + off) = make_float4(Y[mi][nt][0], Y[mi][nt][1], Y[mi][nt][2], Y[mi][nt][3]);
            }
    } else {
        // M columns col0..col0+63 as A fragments of M (rows = output state
        // rows, k = these columns): transpose through LDS, split hi + lo
        lds_barrier();                          // every wave is done with Uh / Ul
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sh.Mt[(32 * wave + 16 * mi + 4 * sub + i) * LDS_MT + 16 * nt + l16] = Y[mi][nt][i];
        lds_barrier();
        char* mbase = seg_area + ((int64_t)s_glob * p.HV + h) * SEG_BYTES;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int idx = tid + 256 * f;      // 16 tiles (8 row tiles x 2 k-steps) x 64 lanes
            const int fl = idx & 63, tile = idx >> 6;
            const int mt = tile >> 1, ksl = tile & 1;
            const int row = 16 * mt + (fl & 15);
            const int kl = 32 * ksl + 8 * (fl >> 4);
            const float4 a = *reinterpret_cast<const float4*>(&sh.Mt[row * LDS_MT + kl]);
            const float4 b = *reinterpret_cast<const float4*>(&sh.Mt[row * LDS_MT + kl + 4]);
            const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            f16x8 hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                hi[e] = static_cast<_Float16>(v[e]);
                lo[e] = static_cast<_Float16>(v[e] - static_cast<float>(hi[e]));
            }
            const int ks = col0 / 32 + ksl;
            const uint32_t off = tile_frag(mt * 4 + ks, fl);
            *reinterpret_cast<f16x8*>(mbase + SEG_OFF_MH + off) = hi;
            *reinterpret_cast<f16x8*>(mbase + SEG_OFF_ML + off) = lo;
        }
    }
}

// Pass A: blocks (run, head, column group); the 4 groups of a (run, head)
// pair and the pairs of a group of 8 share a block index modulo 8 (one XCD,
// one L2), so each chunk's operands leave HBM once per pair.
__global__ __launch_bounds__(256) void seg_state_kernel(const PrefillParams p) {
    __shared__ __attribute__((aligned(16))) SegStateShared sh;
    const int blk = blockIdx.x;
    const int xcd = blk & 7;
    const int jdx = blk >> 3;
    const int grp = jdx % kGroups;
    const int unit = (jdx / kGroups) * 8 + xcd;
    if (unit >= p.max_segs * p.HV) return;
    const int h = unit % p.HV;
    SegInfo g;
    if (!locate_segment(p, unit / p.HV, g)) return;
    // no map for a sequence's last run; run 0 needs only its B part (from the pool state)
    if (g.nseg <= 1 || g.j == g.nseg - 1 || (g.j == 0 && grp < K / kGroupCols)) return;
    if (p.idx[g.n] < 0 || p.idx[g.n] >= p.num_slots) return;
    if (g.seg0 + g.nseg > p.max_segs) return;   // only a malformed cu_seqlens gets here
    if (grp >= K / kGroupCols) seg_state_run<true>(p, sh, g, h, grp);
    else seg_state_run<false>(p, sh, g, h, grp);
}

// Pass B: one block of 4 waves per (sequence, head, 16 state columns); wave
// w computes rows 32w..32w+31.  S_in(j+1) = M_j S_in(j) + B_j, j = 1 .. nseg-2,
// with M and S both split into fp16 hi + lo (hi hi + hi lo + lo hi).
constexpr int LDS_SC = K + 16;

struct ChainOps {
    f16x8 mh[2][4], ml[2][4];               // M rows 32w + 16mi.., k-steps 0..3
    float4 b[2];                            // B rows 32w + 16mi + 4sub.., column col0 + l16
};

__device__ __forceinline__ void chain_load(ChainOps& o, const char* seg, int wave, int lane, int sub, int l16, int col0) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint32_t off = tile_frag((2 * wave + mi) * 4 + ks, lane);
            o.mh[mi][ks] = *reinterpret_cast<const f16x8*>(seg + SEG_OFF_MH + off);
            o.ml[mi][ks] = *reinterpret_cast<const f16x8*>(seg + SEG_OFF_ML + off);
        }
        o.b[mi] = *reinterpret_cast<const float4*>(seg + SEG_OFF_B + ((int64_t)(col0 + l16) * K + 32 * wave + 16 * mi + 4 * sub) * 4);
    }
}

__global__ __launch_bounds__(256) void seg_chain_kernel(const PrefillParams p) {
    __shared__ __attribute__((aligned(16))) _Float16 s_sh[2][VS * LDS_SC];
    __shared__ __attribute__((aligned(16))) _Float16 s_sl[2][VS * LDS_SC];
    const int blk = blockIdx.x;
    const int xcd = blk & 7;
    const int jdx = blk >> 3;
    const int vsl = jdx % NVS;
    const int pair = (jdx / NVS) * 8 + xcd;     // (sequence, head)
    if (pair >= p.num_seqs * p.HV) return;
    const int h = pair % p.HV, n = pair / p.HV;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, sub = lane >> 4, l16 = lane & 15;
    const int col0 = vsl * VS;
    // the sequence's first run: its runs are global runs seg0 .. seg0 + nseg - 1
    SegInfo g;
    {
        // find run 0 of sequence n: walk the runs of the sequences before it
        int seg0 = 0, nseg = 0;
        if (!p.cu) {
            nseg = runs_of(ceil_div(p.T, C), p.seg_len);
            seg0 = n * nseg;
        } else {
            const int L = p.seg_len;
            int tot = 0;
            for (int m0 = 0; m0 < n; m0 += 64) {
                const int m = m0 + lane;
                const int cnt = m < n ? runs_of(ceil_div(seq_len(p.cu, m, p.T), C), L) : 0;
                tot += group_sum_int(cnt);
            }
            seg0 = tot;
            nseg = runs_of(ceil_div(seq_len(p.cu, n, p.T), C), L);
        }
        g.seg0 = seg0;
        g.nseg = nseg;
    }
    if (g.nseg <= 2) return;
    if (p.idx[n] < 0 || p.idx[n] >= p.num_slots) return;
    if (g.seg0 + g.nseg > p.max_segs) return;   // only a malformed cu_seqlens gets here
    const char* area = reinterpret_cast<const char*>(p.ws) + p.seg_off;
    float* sin_base = reinterpret_cast<float*>(reinterpret_cast<char*>(p.ws) + p.seg_off);
    auto seg_ptr = [&](int j) { return area + ((int64_t)(g.seg0 + j) * p.HV + h) * SEG_BYTES; };
    auto sin_ptr = [&](int j) {
        return reinterpret_cast<float*>(reinterpret_cast<char*>(sin_base) + ((int64_t)(g.seg0 + j) * p.HV + h) * SEG_BYTES +
                                        SEG_OFF_SIN);
    };
    // S_in(1), rows 32w + 16mi + 4sub + i, column col0 + l16
    f32x4_t S[2];
    {
        const float* src = sin_ptr(1);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            const float4 v = *reinterpret_cast<const float4*>(src + (int64_t)(col0 + l16) * K + 32 * wave + 16 * mi + 4 * sub);
            S[mi] = f32x4_t{v.x, v.y, v.z, v.w};
        }
    }
    const int last = g.nseg - 2;                // maps j = 1 .. last
    int buf = 0;
    auto step = [&](const ChainOps& o, ChainOps& nx, int j) {
        const bool live = j <= last;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            f16x4 hi, lo;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                hi[i] = static_cast<_Float16>(S[mi][i]);
                lo[i] = static_cast<_Float16>(S[mi][i] - static_cast<float>(hi[i]));
            }
            *reinterpret_cast<f16x4*>(&s_sh[buf][l16 * LDS_SC + 32 * wave + 16 * mi + 4 * sub]) = hi;
            *reinterpret_cast<f16x4*>(&s_sl[buf][l16 * LDS_SC + 32 * wave + 16 * mi + 4 * sub]) = lo;
        }
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        f32x4_t acc[2][2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            acc[mi][0] = f32x4_t{o.b[mi].x, o.b[mi].y, o.b[mi].z, o.b[mi].w};
            acc[mi][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const f16x8 bh = *reinterpret_cast<const f16x8*>(&s_sh[buf][l16 * LDS_SC + 32 * ks + 8 * sub]);
            const f16x8 bl = *reinterpret_cast<const f16x8*>(&s_sl[buf][l16 * LDS_SC + 32 * ks + 8 * sub]);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                acc[mi][ks & 1] = mfma16(o.mh[mi][ks], bh, acc[mi][ks & 1]);
                acc[mi][ks & 1] = mfma16(o.mh[mi][ks], bl, acc[mi][ks & 1]);
                acc[mi][ks & 1] = mfma16(o.ml[mi][ks], bh, acc[mi][ks & 1]);
            }
        }
        chain_load(nx, seg_ptr(min(j + 1, last)), wave, lane, sub, l16, col0);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            const f32x4_t sn = acc[mi][0] + acc[mi][1];
            S[mi] = live ? sn : S[mi];
        }
        if (live) {
            float* dst = sin_ptr(j + 1);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                *reinterpret_cast<float4*>(dst + (int64_t)(col0 + l16) * K + 32 * wave + 16 * mi + 4 * sub) =
                    make_float4(S[mi][0], S[mi][1], S[mi][2], S[mi][3]);
        }
        buf ^= 1;
    };
    ChainOps oa, ob;
    chain_load(oa, seg_ptr(1), wave, lane, sub, l16, col0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    for (int j = 1; j <= last; j += 2) {
        step(oa, ob, j);
        step(ob, oa, j + 1);
    }
}

}  // namespace

hipError_t launch_seg_state(const PrefillParams& p, hipStream_t s) {
    const int64_t units = (int64_t)p.max_segs * p.HV;
    const int64_t nblk = (units + 7) / 8 * 8 * kGroups;
    klaunch(seg_state_kernel, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_seg_chain(const PrefillParams& p, hipStream_t s) {
    const int64_t pairs = (int64_t)p.num_seqs * p.HV;
    const int64_t nblk = (pairs + 7) / 8 * 8 * NVS;
    klaunch(seg_chain_kernel, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace kda
