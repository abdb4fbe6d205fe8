/*
 * libkda — Kimi Delta Attention (KDA) on AMD MI355X (gfx950), C ABI.
 *
 * Three phases of the KDA recurrence, per (sequence or request, head) with a
 * state S of K x V floats:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 *   kda_prefill  chunked prefill over fixed-length or packed (cu_seqlens)
 *                sequences; the final state of each sequence goes back to
 *                its pool slot.
 *   kda_decode   packed one-token decode; the pool slot is updated in place.
 *   kda_verify   speculative target verify of chain / tree drafts with the
 *                depthwise causal conv1d fused in; one state snapshot per
 *                draft node; the pool is only read.
 *   kda_commit   copies the accepted node's snapshot into the pool slot and
 *                rolls the conv state along the accepted path.
 *
 * The method and its three phases are those of "[KDA] Support Helion MTP
 * verification and harden prefill, decode" (sglang pull request 42857,
 * Motivation and Modifications).  The argument contract (q/k/v, raw gate
 * with A_log / dt_bias / lower_bound, raw beta, scale, in-kernel q/k L2
 * norm, cu_seqlens, initial_state + initial_state_indices, intermediate
 * states) and the error cases follow the report on sglang pull request
 * 35197, "Fix Helion small-token prefill bug", key code snippets of
 * kda_prefill.py (chunk_kda) and kda_decode.py
 * (validate_packed_decode_inputs).  The fused conv1d + recurrence verify
 * follows "[KDA] Default GLM-5-Next spec verify to the CuTe DSL KDA kernel"
 * (sglang pull request 42905), Summary.  The pages print no formula; the
 * recurrence above, the gate map and the conv details are the readings
 * documented at each struct below.
 *
 * Conventions shared by every call
 * --------------------------------
 *  * Every tensor pointer is a DEVICE pointer owned by the caller.  libkda
 *    never allocates, frees, synchronises, or reads device memory from the
 *    host, so each call only enqueues kernels on `stream` (a hipStream_t
 *    passed as void*; NULL = the null stream) and returns.  All calls can be
 *    captured into a HIP graph.
 *  * Errors come back as a kda_status_t and never launch anything; the text
 *    of the last error on the calling thread is kda_last_error().
 *  * Shapes, strides and flags are validated on the host.  Preconditions
 *    that would need device data (slot indices in range and distinct,
 *    cu_seqlens monotone, parents[b, i] in {-1} U [0, i)) are the caller's
 *    responsibility; violating them is undefined behaviour.
 *  * Activation tensors of one call share one dtype (`dtype`: KDA_BF16 or
 *    KDA_F32).  The state pool, snapshots, intermediate states, A_log and
 *    dt_bias are always float32.  Strides are in elements; the innermost
 *    dimension (K or V) of every activation tensor is contiguous; pools and
 *    snapshots are dense.
 *  * State layout: pool[slot, h, v, k] = S[k, v] (the state is stored
 *    transposed, [slots, HV, V, K]; in the 35197 report's decode snippet the
 *    last three dims of the initial state are the value heads, the value dim
 *    and the key dim, in that order).
 *  * Supported: HV a multiple of H, K and V in {32, 64, 128}.  K or V not a
 *    power of two is rejected with KDA_ERR_UNSUPPORTED (the 35197 report's
 *    decode input check refuses such head dims, whose padded lanes would go
 *    unmasked).
 *  * Grouped heads (reading; the pages name H and HV separately): value
 *    head h (of HV) reads q/k head h / (HV / H).
 *  * Gate (reading): with A_log != NULL the raw gate r is mapped to the
 *    log-decay g = lower_bound * sigmoid(exp(A_log[h]) * (r + dt_bias[h*K+k]))
 *    when has_lower_bound (the pages name A_log, dt_bias and lower_bound
 *    and a bounded gate of -5, without the formula), and to the unbounded
 *    g = -exp(A_log[h]) * softplus(r + dt_bias[h*K+k]) otherwise.  With
 *    A_log == NULL the gate tensor already holds g.  dt_bias may be NULL.
 *  * beta = sigmoid(raw) when beta_is_raw, else used as given (42857,
 *    Modifications: forward beta_is_raw).
 *  * use_qk_l2norm: q and k are scaled by (sum x^2 + 1e-6)^(-1/2) over the
 *    head dim before use.  `scale` multiplies every output.
 *  * Calls are reentrant.  Two calls that write the same pool slot or
 *    snapshot must not overlap on different streams.
 */
#ifndef LIBKDA_KDA_H_
#define LIBKDA_KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1

/* Size of the built-in scratch kda_prefill_noalloc uses as its workspace:
 * 128 MiB per device (a 4096-token, 16-head, K = V = 128 bf16 prefill at
 * chunk 64 fits). */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1,  /* a required pointer is NULL, a shape or
                                      stride is inconsistent, ...           */
    KDA_ERR_UNSUPPORTED = 2,       /* valid but not implemented (K, V, C,
                                      N, W, HV not a multiple of H)         */
    KDA_ERR_HIP = 3                /* a HIP launch failed                   */
} kda_status_t;

typedef enum kda_dtype {
    KDA_F32 = 0,
    KDA_BF16 = 1
} kda_dtype_t;

typedef enum kda_activation {
    KDA_ACT_NONE = 0,
    KDA_ACT_SILU = 1
} kda_activation_t;

/* Identifiers for kda_args_size(). */
enum { KDA_ARGS_PREFILL = 0, KDA_ARGS_DECODE = 1, KDA_ARGS_VERIFY = 2, KDA_ARGS_COMMIT = 3,
       KDA_ARGS_CONV_UPDATE = 4, KDA_ARGS_DECODE_CONV = 5 };

/* ------------------------------------------------------------------------
 * Prefill (chunk_kda entry of the 35197 report).
 *
 * Layout: q, k [B, T, H, K]; v, o [B, T, HV, V]; g [B, g_rows, HV, K];
 * beta [B, beta_rows, HV] (HV contiguous).  *_stride[0..2] are the strides
 * of the batch, token and head dims (beta_stride[0..1]: batch, token).
 *
 * Packed sequences: with cu_seqlens != NULL (int32 [num_seqs + 1], device,
 * rising from 0 to T) B must be 1 and sequence n is tokens
 * [cu_seqlens[n], cu_seqlens[n+1]).  Without it there are num_seqs == B
 * sequences of T tokens.
 *
 * Padded gate / beta: g_rows and beta_rows must be >= T (the 35197
 * report's prefill entry rejects shorter gate or beta tensors); rows >= T
 * are never read, whatever they hold.
 *
 * State: state_pool [num_slots, HV, V, K] float32 and state_indices
 * [num_seqs] int32 are REQUIRED (the same entry refuses a call without an
 * indexed pool).  Sequence n starts from pool[state_indices[n]] and its
 * final state is written back to the same slot.
 *
 * Intermediate states (optional, output_intermediate_states): with
 * intermediate_states != NULL, the state entering every chunk of chunk_size
 * tokens is written, [num_intermediate, HV, V, K] float32, at global chunk
 * index sum_{m<n} ceil(len_m / C) + c.  num_intermediate must be at least
 * B * ceil(T / C) (fixed) or floor(T / C) + num_seqs (packed).
 *
 * chunk_size is 16 or 64.  T == 0 or B == 0 is a successful no-op.
 * The call needs a device workspace of kda_prefill_workspace_size() bytes
 * (caller-owned, 256-byte aligned, contents irrelevant on entry).
 *
 * Two-level scan (matrix-core path only): with run_chunks = L > 0 each
 * sequence is cut into runs of L chunks whose state maps are composed in
 * parallel (per run, S_out = M S_in + B with M the product of the chunks'
 * K x K maps), the runs' entry states are chained over the runs, and every
 * run is then scanned from its entry state, all runs at once.  0 selects
 * the library default (currently one run per sequence: on the 16 x 128
 * workloads the single sequential scan measured faster), a negative value
 * forces one run per sequence.  The results equal the single-run scan
 * within rounding (not bit for bit, as the entry states are computed by
 * other products).  More runs need more workspace
 * (kda_prefill_workspace_size).
 *
 * Precision: float32 activations take an all-float32 path, as does a
 * bounded gate with lower_bound > 0 (whose log-decay is positive).  bf16
 * activations with chunk_size 64 and K = V = 128 run the chunk products on
 * bf16 / fp16 matrix tiles with float32 accumulation and a float32 state.
 * The state S and the corrected values U = U' - W S enter those tiles as
 * fp16; a scan block in which some |S| or |U| reaches 2^15 runs its chunks
 * again with per-wave power-of-two scaling of those operands, so the state
 * may take any float32 magnitude and U up to 2^29.  Exceptions: with
 * run_chunks > 0 the run maps keep the fp16 range (|S|, |U| < 65504); and a
 * log-decay g > 0 given directly (A_log == NULL) must keep every in-chunk
 * cumulative sum below ~11, as the decay factors e^G enter fp16 operands.
 * Outside these limits results may hold +-inf; nothing faults.
 * ---------------------------------------------------------------------- */
typedef struct kda_prefill_args {
    uint32_t struct_size;          /* sizeof(kda_prefill_args)              */
    int32_t dtype;                 /* kda_dtype_t of q, k, v, g, beta, o    */
    int64_t B, T, H, HV, K, V;
    int64_t chunk_size;            /* 16 or 64                              */
    const void* q;    int64_t q_stride[3];
    const void* k;    int64_t k_stride[3];
    const void* v;    int64_t v_stride[3];
    void* o;          int64_t o_stride[3];
    const void* g;    int64_t g_rows;    int64_t g_stride[3];
    const void* beta; int64_t beta_rows; int64_t beta_stride[2];
    const float* A_log;            /* [HV] or NULL (g is a log-decay)       */
    const float* dt_bias;          /* [HV*K] or NULL                        */
    float lower_bound;
    int32_t has_lower_bound;
    int32_t beta_is_raw;
    int32_t use_qk_l2norm;
    float scale;
    int32_t run_chunks;            /* two-level scan, see above; 0: default */
    const int32_t* cu_seqlens;     /* [num_seqs + 1] or NULL                */
    int64_t num_seqs;
    float* state_pool;             /* [num_slots, HV, V, K]                 */
    int64_t num_slots;
    const int32_t* state_indices;  /* [num_seqs]                            */
    float* intermediate_states;    /* [num_intermediate, HV, V, K] or NULL  */
    int64_t num_intermediate;
} kda_prefill_args;

/* ------------------------------------------------------------------------
 * Decode (validate_packed_decode_inputs of the 35197 report; bounded-gate
 * packed decode of 42857, Modifications).
 *
 * q, k [B, H, K] with strides (q_stride[0] batch, q_stride[1] head), e.g.
 * views of a packed mixed_qkv [B, 2*H*K + HV*V]; v [B, HV, V]; o [B, HV, V].
 * a [B, a_cols] raw gate (a_cols must equal HV*K, as the 35197 report's
 * decode input check requires); b [B, HV] raw beta.  state_indices [B]: request r updates
 * pool[state_indices[r]] in place; a negative index marks a padded request,
 * whose output is zero and whose state is not touched.
 * q, k and a are read four elements at a time: their base pointers must be
 * aligned to four elements (8 bytes for bf16, 16 for float32) and their
 * strides must be multiples of 4 (KDA_ERR_INVALID_ARGUMENT otherwise).
 * ---------------------------------------------------------------------- */
typedef struct kda_decode_args {
    uint32_t struct_size;          /* sizeof(kda_decode_args)               */
    int32_t dtype;                 /* kda_dtype_t of q, k, v, a, b, o       */
    int64_t B, H, HV, K, V;
    const void* q;    int64_t q_stride[2];
    const void* k;    int64_t k_stride[2];
    const void* v;    int64_t v_stride[2];
    void* o;          int64_t o_stride[2];
    const void* a;    int64_t a_stride;  int64_t a_cols;
    const void* b;    int64_t b_stride;
    const float* A_log;
    const float* dt_bias;
    float lower_bound;
    int32_t has_lower_bound;
    int32_t beta_is_raw;
    int32_t use_qk_l2norm;
    float scale;
    int32_t reserved0;
    float* state_pool;             /* [num_slots, HV, V, K]                 */
    int64_t num_slots;
    const int32_t* state_indices;  /* [B]                                   */
} kda_decode_args;

/* ------------------------------------------------------------------------
 * Target verify (42857, Modifications: chain / tree verification with
 * per-candidate state snapshots; 42905, Summary: conv1d + recurrence in one
 * launch).
 *
 * Draft tokens: request r owns rows r*N .. r*N+N-1 of mixed_qkv
 * [B*N, conv_dim] (pre-conv, channels q || k || v, conv_dim = 2*H*K + HV*V,
 * row stride mixed_stride), a [B*N, a_cols = HV*K] raw gate, b [B*N, HV]
 * raw beta, o [B*N, HV, V] (strides: row, head).
 *
 * Tree: parents [B, N] int32, parents[r, i] in {-1} U [0, i); -1 attaches
 * the node to the pool state.  parents == NULL is a chain (parent i-1).
 *
 * Conv (reading): width W = conv_width in [2, 4]; conv_weight [conv_dim, W]
 * and conv_bias [conv_dim] (nullable) contiguous, dtype `dtype`;
 * y_c = sum_j w[c, j] x_{c, t-W+1+j} (+ bias_c), then SiLU if
 * conv_activation == KDA_ACT_SILU.  The history of node i is the path from
 * the root to i, preceded by conv_state[cslot, c, 0 .. W-2] (oldest first),
 * conv_state [num_conv_slots, conv_dim, W-1] contiguous, cslot =
 * conv_state_indices[r] (NULL: state_indices[r]).  The L2 norm of q / k
 * follows the conv.
 *
 * State: the pool is read only.  Node i of request r leaves its state in
 * snapshots[sslot, i] with snapshots [num_snapshot_slots, N, HV, V, K]
 * float32 and sslot = snapshot_indices[r] (NULL: r).  snapshots == NULL
 * writes outputs only (then num_snapshot_slots and snapshot_indices are
 * ignored); the accepted state is then committed with kda_commit_replay.
 * That launch computes the draft as one small chunk on fp32 matrix tiles
 * (the state read once per request and head), so its outputs equal the
 * snapshot launch's within rounding, not bit for bit.  Requests with a
 * negative state index produce zero output and write no snapshot.  N is in
 * [1, 16].
 * ---------------------------------------------------------------------- */
typedef struct kda_verify_args {
    uint32_t struct_size;          /* sizeof(kda_verify_args)               */
    int32_t dtype;                 /* mixed_qkv, conv_*, a, b, o            */
    int64_t B, N, H, HV, K, V;
    const void* mixed_qkv; int64_t mixed_stride;
    const void* conv_weight;
    const void* conv_bias;
    int64_t conv_width;
    int32_t conv_activation;       /* kda_activation_t                      */
    int32_t reserved0;
    const void* conv_state;        /* [num_conv_slots, conv_dim, W-1]       */
    int64_t num_conv_slots;
    const int32_t* conv_state_indices;
    const int32_t* parents;        /* [B, N] or NULL (chain)                */
    void* o;          int64_t o_stride[2];
    const void* a;    int64_t a_stride;  int64_t a_cols;
    const void* b;    int64_t b_stride;
    const float* A_log;
    const float* dt_bias;
    float lower_bound;
    int32_t has_lower_bound;
    int32_t beta_is_raw;
    int32_t use_qk_l2norm;
    float scale;
    int32_t reserved1;
    const float* state_pool;       /* [num_slots, HV, V, K], read only      */
    int64_t num_slots;
    const int32_t* state_indices;  /* [B]                                   */
    float* snapshots;              /* [num_snapshot_slots, N, HV, V, K]     */
    int64_t num_snapshot_slots;
    const int32_t* snapshot_indices;  /* [B] or NULL (request r -> r)       */
} kda_verify_args;

/* ------------------------------------------------------------------------
 * Commit after verify (42857 review thread: commit a partially accepted
 * prefix, then verify again with new inputs and slots).
 *
 * accepted [B] int32: index of the last accepted node of request r, or -1
 * (nothing accepted: pool slot and conv state unchanged).  For r with
 * accepted[r] = i >= 0 and state_indices[r] >= 0:
 *   pool[state_indices[r]] <- snapshots[sslot, i]          (bit copy)
 *   conv_state[cslot]      <- the last W-1 inputs of conv_state[cslot]
 *                             followed by mixed_qkv rows of the path
 *                             root .. i                     (bit copy)
 * with sslot / cslot defaulting as in kda_verify.  conv_state == NULL
 * skips the conv roll.  mixed_qkv, parents and snapshots are those of the
 * preceding kda_verify call.
 * ---------------------------------------------------------------------- */
typedef struct kda_commit_args {
    uint32_t struct_size;          /* sizeof(kda_commit_args)               */
    int32_t dtype;                 /* mixed_qkv and conv_state              */
    int64_t B, N, HV, K, V;
    int64_t conv_dim, conv_width;
    const int32_t* accepted;       /* [B]                                   */
    const int32_t* parents;        /* [B, N] or NULL (chain)                */
    const float* snapshots;        /* [num_snapshot_slots, N, HV, V, K]     */
    int64_t num_snapshot_slots;
    const int32_t* snapshot_indices;
    float* state_pool;             /* [num_slots, HV, V, K]                 */
    int64_t num_slots;
    const int32_t* state_indices;  /* [B]                                   */
    void* conv_state;              /* [num_conv_slots, conv_dim, W-1] / NULL */
    int64_t num_conv_slots;
    const int32_t* conv_state_indices;
    const void* mixed_qkv;         /* [B*N, conv_dim]                       */
    int64_t mixed_stride;
} kda_commit_args;

/* ------------------------------------------------------------------------
 * Conv update before a packed decode: the depthwise causal conv of one new
 * token per request (the same conv as kda_verify's, 42905 Summary: conv1d
 * then the recurrence), whose output holds the q || k || v channels that
 * kda_decode reads as strided views.
 *
 * x [B, conv_dim] pre-conv (row stride x_stride), y [B, conv_dim] post-conv
 * (row stride y_stride; y == x is allowed), conv_weight [conv_dim, W] and
 * conv_bias [conv_dim] (nullable) contiguous, conv_state
 * [num_conv_slots, conv_dim, W-1] contiguous, oldest entry first; all of
 * dtype `dtype`.  W = conv_width in [2, 4].  For request r with
 * s = conv_state_indices[r] in [0, num_conv_slots):
 *   y[r, c] = sum_j w[c, j] * window[j] (+ bias[c]), then SiLU if
 *             conv_activation == KDA_ACT_SILU, window = conv_state[s, c, :]
 *             followed by x[r, c] (accumulated in fp32);
 *   conv_state[s, c, :] <- the window's last W-1 entries (bit copies).
 * Any other index marks a padded request: y[r] = 0, no state touched.
 * Requests must name distinct slots.
 * ---------------------------------------------------------------------- */
typedef struct kda_conv_update_args {
    uint32_t struct_size;          /* sizeof(kda_conv_update_args)          */
    int32_t dtype;
    int64_t B, conv_dim, conv_width;
    int32_t conv_activation;       /* kda_activation_t                      */
    int32_t reserved0;
    const void* x;    int64_t x_stride;
    void* y;          int64_t y_stride;
    const void* conv_weight;
    const void* conv_bias;
    void* conv_state;
    int64_t num_conv_slots;
    const int32_t* conv_state_indices;   /* [B]                             */
} kda_conv_update_args;

/* ------------------------------------------------------------------------
 * Decode with the conv update fused in (one launch): kda_conv_update on the
 * token's pre-conv channels followed by kda_decode on the q || k || v views
 * of its output ("[KDA] Default GLM-5-Next spec verify to the CuTe DSL KDA
 * kernel", Summary: conv1d and recurrence in one launch).
 *
 * mixed_qkv [B, conv_dim] pre-conv (channels q || k || v, conv_dim =
 * 2*H*K + HV*V, row stride mixed_stride);
 * conv_weight [conv_dim, W], conv_bias [conv_dim] (nullable), conv_state
 * [num_conv_slots, conv_dim, W-1] (oldest first), all contiguous and of
 * dtype `dtype`, W = conv_width in [2, 4].  The conv outputs stay in fp32
 * (as in kda_verify's fused conv), where the two-launch path stores them in
 * `dtype` first; the conv-state roll is the same bit copy.
 * a, b, gate, pool, o: as kda_decode.  Request r with a state index in
 * [0, num_slots) updates pool[state_indices[r]] and rolls
 * conv_state[cslot] in place (cslot = conv_state_indices[r], or
 * state_indices[r] when NULL; a cslot outside [0, num_conv_slots) gives
 * zero conv outputs and no roll); any other state index marks a padded
 * request: zero output, neither state touched.  Requests must name
 * distinct slots.  a and mixed_qkv must start on a 4-element boundary with
 * row strides that are multiples of 4, conv_weight and conv_state on an
 * 8-byte boundary (KDA_ERR_INVALID_ARGUMENT otherwise).  One kernel launch:
 * one block per (request, q/k head); nothing is allocated.
 * ---------------------------------------------------------------------- */
typedef struct kda_decode_conv_args {
    uint32_t struct_size;          /* sizeof(kda_decode_conv_args)          */
    int32_t dtype;                 /* mixed_qkv, conv_*, a, b, o            */
    int64_t B, H, HV, K, V;
    const void* mixed_qkv; int64_t mixed_stride;
    const void* conv_weight;
    const void* conv_bias;
    int64_t conv_width;
    int32_t conv_activation;       /* kda_activation_t                      */
    int32_t reserved0;
    void* conv_state;              /* [num_conv_slots, conv_dim, W-1]       */
    int64_t num_conv_slots;
    const int32_t* conv_state_indices;  /* [B] or NULL                      */
    void* o;          int64_t o_stride[2];
    const void* a;    int64_t a_stride;  int64_t a_cols;
    const void* b;    int64_t b_stride;
    const float* A_log;
    const float* dt_bias;
    float lower_bound;
    int32_t has_lower_bound;
    int32_t beta_is_raw;
    int32_t use_qk_l2norm;
    float scale;
    int32_t reserved1;
    float* state_pool;             /* [num_slots, HV, V, K]                 */
    int64_t num_slots;
    const int32_t* state_indices;  /* [B]                                   */
} kda_decode_conv_args;

/* ABI version of this header (KDA_ABI_VERSION). */
int kda_abi_version(void);

/* sizeof() of the argument struct named by KDA_ARGS_*; 0 if unknown.  The
 * struct_size field of every argument struct must equal this value. */
size_t kda_args_size(int which);

/* Text of the last error returned on the calling thread ("" if none). */
const char* kda_last_error(void);

/* Per-call timing.  The next compute call made on this thread (kda_prefill,
 * kda_decode, kda_verify, kda_commit, kda_commit_replay, kda_conv_update)
 * records start_event when its first kernel begins and stop_event when its
 * last kernel ends; the timestamps come from the kernel dispatches
 * themselves (hipExtLaunchKernel), so hipEventElapsedTime(start, stop) is
 * the call's time on the GPU without the launch gaps before and after it.
 * Both are hipEvent_t created by the caller with timing enabled; either may
 * be NULL.  The setting is used by exactly one call (launched, rejected or
 * empty) and then cleared.  Not for use under HIP graph capture. */
kda_status_t kda_set_call_events(void* start_event, void* stop_event);

/* Bytes of device workspace kda_prefill needs for these arguments.  Checks
 * the arguments like kda_prefill. */
kda_status_t kda_prefill_workspace_size(const kda_prefill_args* args, size_t* bytes);

/* Which implementation kda_prefill takes for these arguments; nothing is
 * launched and no device memory is read (only pointer values, strides and
 * sizes are looked at).  *path receives
 *   KDA_PREFILL_PATH_MATRIX (1) when all of these hold:
 *     - bf16 activations, chunk_size 64, K = V = 128;
 *     - no bounded gate with lower_bound > 0;
 *     - q, k, g and v have 16-byte aligned base addresses and batch, token
 *       and head strides that are multiples of 8 elements (16 bytes);
 *     - o's token stride is between 16 and 2^22 elements;
 *   KDA_PREFILL_PATH_GENERAL (0) otherwise: every product in float32
 *   (chunk_size 16 or 64, any K, V the arguments allow), on fp32 matrix
 *   tiles except chunks whose decay factors would leave the float32 range
 *   (a positive log-decay, or a decay span above 80 within 8 rows of a
 *   16-row block's reference row), which take exact per-element
 *   exponentials on the vector units.
 * A bf16 view that misses only an alignment condition runs correctly on the
 * general path, at that path's speed.  Checks the arguments like
 * kda_prefill and returns the same errors. */
typedef enum kda_prefill_path {
    KDA_PREFILL_PATH_GENERAL = 0,
    KDA_PREFILL_PATH_MATRIX = 1
} kda_prefill_path_t;
kda_status_t kda_prefill_path(const kda_prefill_args* args, int32_t* path);

/* Chunked prefill.  workspace: >= kda_prefill_workspace_size() bytes of
 * device memory owned by the caller (not used across calls). */
kda_status_t kda_prefill(const kda_prefill_args* args, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Chunked prefill that allocates nothing, for callers that cannot call
 * hipMalloc (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, kernels and results as
 * kda_prefill, with the workspace taken from a scratch array built into the
 * library: KDA_NOALLOC_SCRATCH_BYTES of device memory per device, reserved
 * when the library's code is loaded on that device and held until the
 * process ends.  The caller still passes every input and output.
 * A call whose kda_prefill_workspace_size() exceeds KDA_NOALLOC_SCRATCH_BYTES
 * returns KDA_ERR_INVALID_ARGUMENT and launches nothing.  Nothing in the
 * scratch has to hold any value on entry.  Every call on one device shares
 * that device's scratch and it keeps the last call's contents: two calls
 * that overlap on one device (different streams, or different threads
 * without ordering) race and corrupt each other's results; serialise them.
 * The first call on a device looks up the scratch's device address
 * (hipGetSymbolAddress); errors there are returned as KDA_ERR_HIP. */
kda_status_t kda_prefill_noalloc(const kda_prefill_args* args, void* stream);

/* Packed decode; updates the indexed pool slots in place. */
kda_status_t kda_decode(const kda_decode_args* args, void* stream);

/* Conv update and packed decode in one launch (kda_decode_conv_args). */
kda_status_t kda_decode_conv(const kda_decode_conv_args* args, void* stream);

/* Target verify with fused causal conv; writes snapshots and outputs. */
kda_status_t kda_verify(const kda_verify_args* args, void* stream);

/* Commit accepted snapshots to the pool and roll the conv state. */
kda_status_t kda_commit(const kda_commit_args* args, void* stream);

/* Conv update of one token per request; updates conv_state in place and
 * writes y.  One kernel launch on `stream`; nothing is allocated.  Errors:
 * KDA_ERR_INVALID_ARGUMENT for a NULL pointer, a stride below conv_dim or a
 * bad dtype / activation / slot count, KDA_ERR_UNSUPPORTED for W outside
 * [2, 4]. */
kda_status_t kda_conv_update(const kda_conv_update_args* args, void* stream);

/* Commit by replay: the alternative to per-candidate snapshots that
 * "[KDA] Default GLM-5-Next spec verify to the CuTe DSL KDA kernel" (42905,
 * Summary, target-verify table) times as "ReplaySSM rings"; the pages do not
 * describe its mechanism, so this is a design of its own.  Verify runs with snapshots == NULL
 * and writes outputs only; afterwards this call recomputes, from the pool
 * state and the same inputs, the recurrence over the path root ..
 * accepted[r] only, writes the result to pool[state_indices[r]] and rolls
 * the conv state as kda_commit does.
 *
 * args: the arguments of the preceding kda_verify call, unchanged (same
 * pool contents, inputs, parents and conv state); o, snapshots,
 * num_snapshot_slots and snapshot_indices are ignored.  The pool that
 * args->state_pool points to IS written (kda_verify only reads it).
 * accepted [B] int32 device: last accepted node of request r, or -1
 * (slot and conv state unchanged).  Requests with accepted[r] >= 0 must
 * name distinct pool slots and distinct conv slots.
 * The committed state equals the snapshot kda_verify would have written for
 * node accepted[r] bit for bit (same arithmetic in the same order).
 * Errors: as kda_verify, plus KDA_ERR_INVALID_ARGUMENT for accepted == NULL.
 * Two kernel launches on `stream`; nothing is allocated. */
kda_status_t kda_commit_replay(const kda_verify_args* args, const int32_t* accepted, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBKDA_KDA_H_ */
