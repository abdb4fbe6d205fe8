// Shared pieces of the two prefill paths: launch parameters and the chunk
// bookkeeping for fixed-length and packed (cu_seqlens) sequences.
#pragma once

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

struct PrefillParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    const void* g;
    const void* beta;
    int64_t qs[3], ks[3], vs[3], os[3], gs[3], bs[2];
    const float* A_log;
    const float* dt_bias;
    float lb;
    float scale;
    int gate, beta_is_raw, l2norm;      // gate: GateMode
    int T, HV, num_seqs;
    int group;               // HV / H: value heads per q/k head
    int num_slots;
    int max_chunks;          // chunks the workspace holds
    const int32_t* cu;       // nullable
    float* pool;
    const int32_t* idx;
    float* inter;            // nullable
    float* ws;
    int64_t chunk_floats;    // workspace floats per (chunk, head)
    // Two-level scan of the matrix-core path: runs of seg_len chunks of one
    // sequence are scanned in parallel (0: one run per sequence).
    int seg_len;
    int max_segs;            // runs the workspace holds (all sequences)
    int64_t seg_off;         // byte offset of the per-(run, head) area in ws
    // General path: the fp32 matrix-core prep flags
    // (1) the items it leaves to the exact prep, which then runs only those.
    int* flags;              // nullable; [max_chunks * HV]
    // General path: 256 floats that take the scan's output stores for rows
    // past a chunk's end (never read), so its stores need no branch.
    float* sink;
};

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Every row of a tensor starts on a 16-byte boundary: the base address and
// the first n strides (elements of `elem` bytes) are multiples of 16 bytes.
inline bool aligned_rows(const void* ptr, const int64_t* stride, int n, int elem) {
    if ((reinterpret_cast<uintptr_t>(ptr) & 15u) != 0) return false;
    for (int i = 0; i < n; ++i)
        if ((stride[i] * elem) % 16 != 0) return false;
    return true;
}

// cu_seqlens[n] clamped to [0, T], and the length of sequence n (>= 0), so a
// malformed cu_seqlens cannot move an access outside the T tokens.
__device__ __forceinline__ int cu_at(const int32_t* cu, int n, int T) { return min(max(cu[n], 0), T); }
__device__ __forceinline__ int seq_len(const int32_t* cu, int n, int T) {
    return max(cu_at(cu, n + 1, T) - cu_at(cu, n, T), 0);
}

// Sequence holding global chunk `ci` (packed layout), found with a wave-wide
// prefix sum over ceil(len_n / C).  All 64 lanes of the wave must call it.
// Returns false when ci lies past the last chunk.
__device__ inline bool locate_chunk(const int32_t* cu, int num_seqs, int T, int C, int ci, int& n_out, int& cstart_out) {
    const int lane = threadIdx.x & 63;
    int base = 0;
    for (int n0 = 0; n0 < num_seqs; n0 += 64) {
        const int n = n0 + lane;
        int cnt = 0;
        if (n < num_seqs) cnt = ceil_div(seq_len(cu, n, T), C);
        int incl = cnt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off, 64);
            if (lane >= off) incl += y;
        }
        const int excl = incl - cnt;
        const bool hit = n < num_seqs && ci >= base + excl && ci < base + incl;
        const unsigned long long mask = __ballot(hit);
        if (mask) {
            const int l = __ffsll(mask) - 1;
            n_out = n0 + l;
            cstart_out = base + __shfl(excl, l, 64);
            return true;
        }
        base += __shfl(incl, 63, 64);
    }
    return false;
}

// Number of chunks of sequences [0, n) (packed layout); wave-wide.
__device__ inline int chunks_before(const int32_t* cu, int n, int T, int C) {
    const int lane = threadIdx.x & 63;
    int total = 0;
    for (int m0 = 0; m0 < n; m0 += 64) {
        const int m = m0 + lane;
        int cnt = m < n ? ceil_div(seq_len(cu, m, T), C) : 0;
        total += group_sum_int(cnt);
    }
    return total;
}


// Layouts of the general path's per-(chunk, head) workspace, in the order
// the fp32-tile scan reads them, so that every 16-byte load of the scan is
// part of 1 KiB of consecutive memory across the wave (a row-major operand
// read as row runs touched a cache line per lane and load, and the loads,
// not the products, then set the scan's pace).
//
// Row runs of a [rows][L] operand (W and Qt with L = K, P and Kt^T with
// L = C): lane (r % 16) + 16 g of row block r / 16 reads columns
// g L/4 .. g L/4 + L/4 - 1 of row r as L/16 float4; float4 q of the 64
// lanes of a row block is 256 consecutive floats.
__host__ __device__ inline int64_t ws_run(int row, int col, int L) {
    const int per = L >> 2;                    // columns per lane group
    const int g = col / per, j = col - g * per;
    return ((int64_t)((row >> 4) * (per >> 2) + (j >> 2)) * 64 + (row & 15) + 16 * g) * 4 + (j & 3);
}
// Tiles of U' [C][V]: 16 x 16 tile (r / 16, v / 16) is 64 lanes of 4
// floats, lane (v % 16) + 16 ((r % 16) / 4) holding rows 4 ((r % 16) / 4)
// .. + 3 of column v (the fp32 tile product's accumulator layout).
__host__ __device__ inline int64_t ws_tile(int r, int v, int V) {
    return ((int64_t)((r >> 4) * (V >> 4) + (v >> 4)) * 64 + (v & 15) + 16 * ((r & 15) >> 2)) * 4 + (r & 3);
}

// Scan of the general path on fp32 matrix tiles; defined in kda_prefill_scan32.hip
// for C in {16, 64}, K and V in {32, 64, 128}.
template <typename TIn, int C, int K, int V>
hipError_t launch_scan32(const kda_prefill_args& a, const PrefillParams& p, hipStream_t s);

// Prep of the general path on fp32 matrix tiles (C = 64, K and V in {32,
// 64, 128}); defined in kda_prefill_prep32.hip.  Writes p.flags.
template <typename TIn, int K, int V>
hipError_t launch_prep32(const kda_prefill_args& a, const PrefillParams& p, hipStream_t s);
// The same at C = 16, one wave per chunk x head.
template <typename TIn, int K, int V>
hipError_t launch_prep16(const kda_prefill_args& a, const PrefillParams& p, hipStream_t s);

// Fast path (MFMA) entry points; defined in kda_prefill_mfma.hip.
bool prefill_mfma_eligible(const kda_prefill_args& a);
size_t prefill_mfma_workspace_bytes(const kda_prefill_args& a);
hipError_t launch_prefill_mfma(const kda_prefill_args& a, const PrefillParams& p, hipStream_t s);

}  // namespace kda
