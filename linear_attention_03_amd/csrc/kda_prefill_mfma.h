// Pieces shared by the matrix-core prefill kernels (chunk C = 64,
// K = V = 128): operand types, the MFMA wrappers, the layout of the
// per-(chunk, head) workspace the prep writes and the scans read, and the
// runs ("segments") of the two-level scan.
#pragma once

#include "kda_prefill_common.h"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int C = 64;
constexpr int K = 128;
constexpr int V = 128;
constexpr int VS = 16;          // state columns per scan block
constexpr int NVS = V / VS;

// Workspace of one (chunk, head), in bytes.  Matrices the scan feeds to
// the matrix cores are stored fragment-major: a 16-row x 32-column operand
// tile is the 64 lanes' 16-byte fragments back to back (1 KiB), so every
// scan load is 1 KiB of contiguous, fully used cache lines.
constexpr int OFF_W = 0;                      // fp16 -W    [C][K], A fragments
constexpr int OFF_KT = OFF_W + C * K * 2;     // fp16 Kt^T  [K][C], A fragments
constexpr int OFF_QT = OFF_KT + K * C * 2;    // fp16 Qt    [C][K], A fragments
constexpr int OFF_P = OFF_QT + C * K * 2;     // fp16 P     [C][C], A fragments
constexpr int OFF_UP = OFF_P + C * C * 2;     // f32  U'    [C][V], accumulator fragments
constexpr int OFF_GL = OFF_UP + C * V * 4;    // f32  e^G_last [K]
constexpr int CHUNK_BYTES = ((OFF_GL + K * 4) + 255) / 256 * 256;

// The prep keeps the cumulative log-decay in base-2 units, G2 = G log2(e),
// so every factor e^(G_a - G_b) is one hardware exp2 of a difference.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaxSpan = 80.0f;               // natural-log units
constexpr float kMaxSpan2 = kMaxSpan * kLog2e;
// Spans up to this (natural-log units) keep every Gram factor <= e^8, so the
// normalised Gram operands fit fp16 (11-bit significand); wider spans take
// bf16 operands (8 bits, fp32 range).  The fp16 operands matter where the
// decay is slow: there the state forgets no rounding error, and the Gram
// feeds (I + A)^-1 and so every U.
constexpr float kF16Span2 = 8.0f * kLog2e;

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left at their
// maxima (no wait): vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
constexpr int kWaitVmcnt0 = (7 << 4) | (15 << 8);

__device__ __forceinline__ f32x4_t mfma(bf16x8 a, bf16x8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __bf16 tobf(float x) { return static_cast<__bf16>(x); }

// fp16 products: Kt^T U (state update) and P U (output).  Both operands are
// bounded there (|Kt| <= |k-hat| = 1 and |P| <= 1 under decaying gates), so
// fp16's 11-bit significand is used where bf16's 8 bits would need a split.
__device__ __forceinline__ f32x4_t mfma16(f16x8 a, f16x8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma(bf16x8 a, bf16x8 b, f32x4_t c) { return mfma(a, b, c); }
__device__ __forceinline__ f32x4_t mma(f16x8 a, f16x8 b, f32x4_t c) { return mfma16(a, b, c); }

// Element index of (row, col) in the A-fragment layout of a matrix with
// nks 32-column k-steps: lane (row % 16) + 16 ((col % 32) / 8) of tile
// (row / 16, col / 32) holds columns 8 ((col % 32) / 8) .. +7 of the row.
__device__ __forceinline__ int afrag(int row, int col, int nks) {
    return (((row >> 4) * nks + (col >> 5)) * 64 + (row & 15) + 16 * ((col & 31) >> 3)) * 8 + (col & 7);
}

// ---- fp16 range of the scan's state and corrected values ------------------
//
// The scan feeds S (state) and U (corrected values) to the matrix cores as
// fp16.  Where a wave's block of S or U reaches 2^15 in magnitude, the wave
// scales it by 2^-e before the conversion (e the smallest exponent that
// brings the block's maximum below 2^15; 0 otherwise, so values of ordinary
// size are converted as they are) and publishes 2^e with it.  The S factor
// is undone on the fp32 accumulator of the k-step that wave's rows form; the
// U factor is applied to the other operand (Kt^T or P, both at most 1), so
// e_U is capped at 14.

// Maximum over the 64 lanes of a wave of x >= 0, in every lane: DPP within
// each 16-lane row, then the four row maxima through scalar reads (no LDS
// instruction, so no LDS wait where the callers' paths merge).
__device__ __forceinline__ float wave_max_nonneg(float x) {
    constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kXor1, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kXor2, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kHalfMirror, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kMirror, 0xF, 0xF, false)));
    const float a = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)),
                          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16)));
    const float b = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)),
                          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48)));
    return fmaxf(a, b);
}

// Smallest e >= 0 (at most cap) with m 2^-e < 2^15.
__device__ __forceinline__ int range_exp(float m, int cap) {
    const int ex = static_cast<int>((__float_as_uint(m) >> 23) & 0xffu) - 127;   // floor(log2 m)
    return min(max(ex - 14, 0), cap);
}

// 2^e for e in [-126, 127], exactly.
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float(static_cast<uint32_t>(127 + e) << 23); }

constexpr float kRangeLimit = 32768.0f;   // 2^15: blocks below it are converted as they are
constexpr int kMaxExpS = 100;   // S: undone on fp32 accumulators
constexpr int kMaxExpU = 14;    // U: carried by Kt^T or P (|.| <= 1) in fp16

// ---- two-level scan ------------------------------------------------------
//
// A sequence of n chunks is cut into runs of L = seg_len chunks.  Per chunk
// the state map is affine, S -> (D - Kt^T W) S + Kt^T U', so a run maps its
// entry state S_in to M S_in + B, with M the product of its chunks' K x K
// factors and B its exit state from a zero entry state.  Pass A computes M
// and B of every run but the last (all runs at once), pass B chains
// S_in(j+1) = M_j S_in(j) + B_j over the runs of a sequence, and pass C is
// the chunk scan of every run from its S_in, again all at once.
//
// Per-(run, head) area, after the chunk workspace:
//   M as fp16 hi and lo parts, MFMA A fragments [8 row tiles][4 k-steps][64 lanes][8]
//   B        fp32 [V][K] (pool layout, S^T)
//   S_in     fp32 [V][K] (pool layout): the state entering the run
constexpr int SEG_OFF_MH = 0;
constexpr int SEG_OFF_ML = SEG_OFF_MH + K * K * 2;
constexpr int SEG_OFF_B = SEG_OFF_ML + K * K * 2;
constexpr int SEG_OFF_SIN = SEG_OFF_B + V * K * 4;
constexpr int SEG_BYTES = SEG_OFF_SIN + V * K * 4;

// One run of the two-level scan: sequence n (batch row b), run j of its
// nseg runs, tokens [t0, t0 + len) of row b, global chunk index cs of its
// first chunk, and seg0 the global index of the sequence's first run.
struct SegInfo {
    int n, b, j, nseg, t0, len, cs, seg0, seq_t0, seq_len;
};

__device__ __forceinline__ int runs_of(int nch, int L) { return L > 0 ? (nch + L - 1) / L : 1; }

// Locates run s (global over every sequence).  In the packed layout all 64
// lanes of the wave must call it (wave-wide prefix sums over sequences).
// Returns false when s lies past the last run.
__device__ inline bool locate_segment(const PrefillParams& p, int s, SegInfo& g) {
    const int L = p.seg_len;
    if (!p.cu) {
        const int nch = ceil_div(p.T, C);
        const int per = runs_of(nch, L);
        g.n = s / per;
        if (g.n >= p.num_seqs) return false;
        g.b = g.n;
        g.j = s % per;
        g.nseg = per;
        g.seg0 = g.n * per;
        g.seq_t0 = 0;
        g.seq_len = p.T;
        const int c0 = L > 0 ? g.j * L : 0;
        g.cs = g.n * nch + c0;
        g.t0 = c0 * C;
        g.len = L > 0 ? min(L * C, p.T - g.t0) : p.T;
        return true;
    }
    const int lane = threadIdx.x & 63;
    int base_s = 0, base_c = 0;
    for (int n0 = 0; n0 < p.num_seqs; n0 += 64) {
        const int n = n0 + lane;
        int cs = 0, cc = 0;
        if (n < p.num_seqs) {
            cc = ceil_div(seq_len(p.cu, n, p.T), C);
            cs = L > 0 ? runs_of(cc, L) : 1;
        }
        int is = cs, ic = cc;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int ys = __shfl_up(is, off, 64);
            const int yc = __shfl_up(ic, off, 64);
            if (lane >= off) { is += ys; ic += yc; }
        }
        const int es = is - cs, ec = ic - cc;
        const bool hit = n < p.num_seqs && s >= base_s + es && s < base_s + is;
        const unsigned long long mask = __ballot(hit);
        if (mask) {
            const int l = __ffsll(mask) - 1;
            g.n = n0 + l;
            g.b = 0;
            g.seg0 = base_s + __shfl(es, l, 64);
            g.nseg = __shfl(cs, l, 64);
            const int cstart = base_c + __shfl(ec, l, 64);
            g.j = s - g.seg0;
            g.seq_t0 = cu_at(p.cu, g.n, p.T);
            g.seq_len = seq_len(p.cu, g.n, p.T);
            const int c0 = L > 0 ? g.j * L : 0;
            g.cs = cstart + c0;
            g.t0 = g.seq_t0 + c0 * C;
            g.len = L > 0 ? min(L * C, g.seq_len - c0 * C) : g.seq_len;
            return true;
        }
        base_s += __shfl(is, 63, 64);
        base_c += __shfl(ic, 63, 64);
    }
    return false;
}

// Byte offset of a 64-lane operand tile's fragment for this lane
// (fragment-major storage: 16 bytes per lane, 1 KiB per tile).
__device__ __forceinline__ uint32_t tile_frag(int tile, int lane) { return (tile * 64 + lane) * 16; }

}  // namespace

// Pass A and pass B launches (kda_prefill_seg.hip).
hipError_t launch_seg_state(const PrefillParams& p, hipStream_t s);
hipError_t launch_seg_chain(const PrefillParams& p, hipStream_t s);

}  // namespace kda
