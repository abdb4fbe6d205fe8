// Host entry points of libkda: argument validation, error reporting and
// dispatch to the kernel launchers.  Nothing here dereferences a device
// pointer, allocates, or synchronises; a rejected call launches nothing.
//
// The prefill and decode checks cover the cases the report on sglang pull
// request 35197 ("Fix Helion small-token prefill bug", key code snippets of
// the prefill entry and of the packed-decode input check) rejects: a missing
// state pool, gate or beta rows short of the token count, head dims that
// are not powers of two, and a raw gate of the wrong width.  The messages
// are this library's own.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "kda_internal.h"

namespace kda {

CallEvents& call_events() {
    thread_local CallEvents ev;
    return ev;
}

}  // namespace kda

namespace {

thread_local std::string g_last_error;

// The call events are one-shot: whatever a call does (launch, no-op or
// error), it leaves none set for the next call.
struct ClearCallEvents {
    ~ClearCallEvents() { kda::call_events() = kda::CallEvents{}; }
};

kda_status_t fail(kda_status_t st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

kda_status_t ok() {
    g_last_error.clear();
    return KDA_OK;
}

kda_status_t hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(KDA_ERR_HIP, "%s: HIP error %d (%s)", what, static_cast<int>(e), hipGetErrorString(e));
}

bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

bool supported_dim(int64_t x) { return x == 32 || x == 64 || x == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int32_t d) { return d == KDA_F32 || d == KDA_BF16; }

// Shared checks of head geometry; `who` names the call in messages.
kda_status_t check_heads(const char* who, int64_t H, int64_t HV, int64_t K, int64_t V) {
    if (H <= 0 || HV <= 0 || K <= 0 || V <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: H, HV, K and V must be positive", who);
    if (!pow2(K) || !pow2(V))
        return fail(KDA_ERR_UNSUPPORTED, "%s: head dims K=%lld and V=%lld must both be powers of two",
                    who, (long long)K, (long long)V);
    if (!supported_dim(K) || !supported_dim(V))
        return fail(KDA_ERR_UNSUPPORTED, "%s: K and V must be 32, 64 or 128 (got K=%lld, V=%lld)",
                    who, (long long)K, (long long)V);
    if (HV % H != 0)
        return fail(KDA_ERR_UNSUPPORTED, "%s: HV must be a multiple of H (got H=%lld, HV=%lld)",
                    who, (long long)H, (long long)HV);
    return KDA_OK;
}

kda_status_t check_gate(const char* who, const float* dt_bias,
                        float scale) {
    if (dt_bias != nullptr && !aligned16(dt_bias))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: dt_bias must be 16-byte aligned", who);
    if (!std::isfinite(scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: scale must be finite", who);
    return KDA_OK;
}

bool nonneg(const int64_t* s, int n) {
    for (int i = 0; i < n; ++i)
        if (s[i] < 0) return false;
    return true;
}

kda_status_t validate_prefill(const kda_prefill_args* a) {
    const char* who = "KDA prefill";
    if (a == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: args is NULL", who);
    if (a->struct_size != sizeof(kda_prefill_args))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: struct_size %u != %zu (ABI mismatch)", who,
                    a->struct_size, sizeof(kda_prefill_args));
    if (a->state_pool == nullptr || a->state_indices == nullptr)
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "%s: state_pool and state_indices are both required (each sequence starts from and "
                    "ends in an indexed pool slot)", who);
    if (a->B < 0 || a->T < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: B and T must be >= 0", who);
    if (a->g_rows < a->T || a->beta_rows < a->T)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: g has %lld rows and beta %lld; both need at least T=%lld",
                    who, (long long)a->g_rows, (long long)a->beta_rows, (long long)a->T);
    if (!valid_dtype(a->dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", who, a->dtype);
    kda_status_t st = check_heads(who, a->H, a->HV, a->K, a->V);
    if (st != KDA_OK) return st;
    if (a->chunk_size != 16 && a->chunk_size != 64)
        return fail(KDA_ERR_UNSUPPORTED, "%s: chunk_size must be 16 or 64 (got %lld)", who, (long long)a->chunk_size);
    if ((st = check_gate(who, a->dt_bias, a->scale)) != KDA_OK) return st;
    if (a->num_slots <= 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: num_slots must be positive", who);
    if (!aligned16(a->state_pool)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: state_pool must be 16-byte aligned", who);
    if (a->cu_seqlens != nullptr) {
        if (a->B != 1) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: cu_seqlens requires B == 1 (got B=%lld)", who, (long long)a->B);
        if (a->num_seqs < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: num_seqs must be >= 1 with cu_seqlens", who);
    } else if (a->num_seqs != a->B) {
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: num_seqs (%lld) must equal B (%lld) without cu_seqlens", who,
                    (long long)a->num_seqs, (long long)a->B);
    }
    if (a->B == 0 || a->T == 0) return KDA_OK;
    if (!a->q || !a->k || !a->v || !a->o || !a->g || !a->beta)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: q, k, v, o, g and beta are required", who);
    if (!nonneg(a->q_stride, 3) || !nonneg(a->k_stride, 3) || !nonneg(a->v_stride, 3) ||
        !nonneg(a->o_stride, 3) || !nonneg(a->g_stride, 3) || !nonneg(a->beta_stride, 2))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: strides must be non-negative", who);
    if (a->intermediate_states != nullptr) {
        if (!aligned16(a->intermediate_states))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: intermediate_states must be 16-byte aligned", who);
        const int64_t need = kda::prefill_max_chunks(*a);
        if (a->num_intermediate < need)
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: num_intermediate %lld < %lld chunks", who,
                        (long long)a->num_intermediate, (long long)need);
    }
    return KDA_OK;
}

kda_status_t validate_decode(const kda_decode_args* a) {
    const char* who = "KDA decode";
    if (a == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: args is NULL", who);
    if (a->struct_size != sizeof(kda_decode_args))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: struct_size %u != %zu (ABI mismatch)", who,
                    a->struct_size, sizeof(kda_decode_args));
    if (!valid_dtype(a->dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", who, a->dtype);
    kda_status_t st = check_heads(who, a->H, a->HV, a->K, a->V);
    if (st != KDA_OK) return st;
    if (a->a_cols != a->HV * a->K)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: raw gate a has %lld columns, HV*K = %lld*%lld expected", who,
                    (long long)a->a_cols, (long long)a->HV, (long long)a->K);
    if ((st = check_gate(who, a->dt_bias, a->scale)) != KDA_OK) return st;
    if (a->B < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: B must be >= 0", who);
    if (a->state_pool == nullptr || a->state_indices == nullptr)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s requires an indexed state pool", who);
    if (a->num_slots <= 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: num_slots must be positive", who);
    if (!aligned16(a->state_pool)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: state_pool must be 16-byte aligned", who);
    if (a->B == 0) return KDA_OK;
    if (!a->q || !a->k || !a->v || !a->o || !a->a || !a->b)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: q, k, v, o, a and b are required", who);
    if (!nonneg(a->q_stride, 2) || !nonneg(a->k_stride, 2) || !nonneg(a->v_stride, 2) || !nonneg(a->o_stride, 2) ||
        a->a_stride < 0 || a->b_stride < 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: strides must be non-negative", who);
    // q, k and a are read four elements at a time
    const uintptr_t vec = 4u * (a->dtype == KDA_BF16 ? 2u : 4u);
    auto rows4 = [&](const void* ptr, const int64_t* st, int n) {
        if (reinterpret_cast<uintptr_t>(ptr) % vec != 0) return false;
        for (int i = 0; i < n; ++i)
            if (st[i] % 4 != 0) return false;
        return true;
    };
    if (!rows4(a->q, a->q_stride, 2) || !rows4(a->k, a->k_stride, 2) || !rows4(a->a, &a->a_stride, 1))
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "%s: q, k and a must start on a 4-element boundary with strides that are multiples of 4", who);
    return KDA_OK;
}

kda_status_t validate_decode_conv(const kda_decode_conv_args* a) {
    const char* who = "KDA decode+conv";
    if (a == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: args is NULL", who);
    if (a->struct_size != sizeof(kda_decode_conv_args))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: struct_size %u != %zu (ABI mismatch)", who,
                    a->struct_size, sizeof(kda_decode_conv_args));
    if (!valid_dtype(a->dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", who, a->dtype);
    kda_status_t st = check_heads(who, a->H, a->HV, a->K, a->V);
    if (st != KDA_OK) return st;
    if (a->a_cols != a->HV * a->K)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: raw gate a has %lld columns, HV*K = %lld*%lld expected", who,
                    (long long)a->a_cols, (long long)a->HV, (long long)a->K);
    if (a->conv_width < 2 || a->conv_width > 4)
        return fail(KDA_ERR_UNSUPPORTED, "%s: conv_width must be in [2, 4] (got %lld)", who, (long long)a->conv_width);
    if (a->conv_activation != KDA_ACT_NONE && a->conv_activation != KDA_ACT_SILU)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown conv_activation %d", who, a->conv_activation);
    if ((st = check_gate(who, a->dt_bias, a->scale)) != KDA_OK) return st;
    if (a->B < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: B must be >= 0", who);
    if (a->state_pool == nullptr || a->state_indices == nullptr)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s requires an indexed state pool", who);
    if (a->num_slots <= 0 || a->num_conv_slots <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: slot counts must be positive", who);
    if (!aligned16(a->state_pool)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: state_pool must be 16-byte aligned", who);
    if (a->B == 0) return KDA_OK;
    if (!a->mixed_qkv || !a->conv_weight || !a->conv_state || !a->o || !a->a || !a->b)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: mixed_qkv, conv_weight, conv_state, o, a and b are required", who);
    const int64_t conv_dim = 2 * a->H * a->K + a->HV * a->V;
    if (a->mixed_stride < conv_dim)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: mixed_stride %lld < conv_dim %lld", who,
                    (long long)a->mixed_stride, (long long)conv_dim);
    if (!nonneg(a->o_stride, 2) || a->a_stride < 0 || a->b_stride < 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: strides must be non-negative", who);
    // the gate row and groups of four channels of mixed_qkv, the weights and
    // the conv state are read in vector loads
    const uintptr_t vec = 4u * (a->dtype == KDA_BF16 ? 2u : 4u);
    if (reinterpret_cast<uintptr_t>(a->a) % vec != 0 || a->a_stride % 4 != 0 ||
        reinterpret_cast<uintptr_t>(a->mixed_qkv) % vec != 0 || a->mixed_stride % 4 != 0 ||
        reinterpret_cast<uintptr_t>(a->conv_weight) % 8 != 0 || reinterpret_cast<uintptr_t>(a->conv_state) % 8 != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: a and mixed_qkv must start on a 4-element boundary with strides "
                                              "that are multiples of 4, conv_weight and conv_state on 8 bytes", who);
    return KDA_OK;
}

// replay: the arguments of kda_commit_replay (no output, no snapshots)
kda_status_t validate_verify(const kda_verify_args* a, bool replay) {
    const char* who = replay ? "KDA commit replay" : "KDA verify";
    if (a == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: args is NULL", who);
    if (a->struct_size != sizeof(kda_verify_args))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: struct_size %u != %zu (ABI mismatch)", who,
                    a->struct_size, sizeof(kda_verify_args));
    if (!valid_dtype(a->dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", who, a->dtype);
    kda_status_t st = check_heads(who, a->H, a->HV, a->K, a->V);
    if (st != KDA_OK) return st;
    if (a->N < 1 || a->N > 16)
        return fail(KDA_ERR_UNSUPPORTED, "%s: the number of draft tokens must be in [1, 16] (got %lld)", who, (long long)a->N);
    if (a->conv_width < 2 || a->conv_width > 4)
        return fail(KDA_ERR_UNSUPPORTED, "%s: conv_width must be in [2, 4] (got %lld)", who, (long long)a->conv_width);
    if (a->conv_activation != KDA_ACT_NONE && a->conv_activation != KDA_ACT_SILU)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown conv_activation %d", who, a->conv_activation);
    if (a->a_cols != a->HV * a->K)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: raw gate a has %lld columns, HV*K = %lld*%lld expected", who,
                    (long long)a->a_cols, (long long)a->HV, (long long)a->K);
    if ((st = check_gate(who, a->dt_bias, a->scale)) != KDA_OK) return st;
    if (a->B < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: B must be >= 0", who);
    if (a->state_pool == nullptr || a->state_indices == nullptr)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s requires an indexed state pool", who);
    if (a->num_slots <= 0 || a->num_conv_slots <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: slot counts must be positive", who);
    const bool snaps = !replay && a->snapshots != nullptr;   // ignored by the replay
    if (snaps && a->num_snapshot_slots <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: slot counts must be positive", who);
    if (snaps && a->snapshot_indices == nullptr && a->num_snapshot_slots < a->B)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: without snapshot_indices num_snapshot_slots must be >= B", who);
    if (!aligned16(a->state_pool) || (snaps && !aligned16(a->snapshots)))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: state_pool and snapshots must be 16-byte aligned", who);
    if (a->B == 0) return KDA_OK;
    if (!a->mixed_qkv || !a->conv_weight || !a->conv_state || !a->a || !a->b || (!replay && !a->o))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: mixed_qkv, conv_weight, conv_state, o, a and b are required", who);
    const int64_t conv_dim = 2 * a->H * a->K + a->HV * a->V;
    if (a->mixed_stride < conv_dim)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: mixed_stride %lld < conv_dim %lld", who,
                    (long long)a->mixed_stride, (long long)conv_dim);
    if ((!replay && !nonneg(a->o_stride, 2)) || a->a_stride < 0 || a->b_stride < 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: strides must be non-negative", who);
    return KDA_OK;
}

kda_status_t validate_conv_update(const kda_conv_update_args* a) {
    const char* who = "KDA conv update";
    if (a == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: args is NULL", who);
    if (a->struct_size != sizeof(kda_conv_update_args))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: struct_size %u != %zu (ABI mismatch)", who,
                    a->struct_size, sizeof(kda_conv_update_args));
    if (!valid_dtype(a->dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", who, a->dtype);
    if (a->B < 0 || a->B > 65535) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: B must be in [0, 65535]", who);
    if (a->conv_dim <= 0 || a->conv_dim > (int64_t(1) << 30))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: conv_dim must be in [1, 2^30]", who);
    if (a->conv_width < 2 || a->conv_width > 4)
        return fail(KDA_ERR_UNSUPPORTED, "%s: conv_width must be in [2, 4] (got %lld)", who, (long long)a->conv_width);
    if (a->conv_activation != KDA_ACT_NONE && a->conv_activation != KDA_ACT_SILU)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown conv_activation %d", who, a->conv_activation);
    if (a->num_conv_slots <= 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: num_conv_slots must be positive", who);
    if (a->B == 0) return KDA_OK;
    if (!a->x || !a->y || !a->conv_weight || !a->conv_state || !a->conv_state_indices)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: x, y, conv_weight, conv_state and conv_state_indices are required", who);
    if (a->x_stride < a->conv_dim || a->y_stride < a->conv_dim)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: x_stride and y_stride must be >= conv_dim", who);
    return KDA_OK;
}

kda_status_t validate_commit(const kda_commit_args* a) {
    const char* who = "KDA commit";
    if (a == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: args is NULL", who);
    if (a->struct_size != sizeof(kda_commit_args))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: struct_size %u != %zu (ABI mismatch)", who,
                    a->struct_size, sizeof(kda_commit_args));
    if (a->B < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: B must be >= 0", who);
    if (a->N < 1 || a->N > 16)
        return fail(KDA_ERR_UNSUPPORTED, "%s: the number of draft tokens must be in [1, 16] (got %lld)", who, (long long)a->N);
    if (a->HV <= 0 || a->K <= 0 || a->V <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: HV, K and V must be positive", who);
    if (a->state_pool == nullptr || a->state_indices == nullptr || a->snapshots == nullptr || a->accepted == nullptr)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: accepted, snapshots, state_pool and state_indices are required", who);
    if (a->num_slots <= 0 || a->num_snapshot_slots <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: slot counts must be positive", who);
    if (!aligned16(a->state_pool) || !aligned16(a->snapshots))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: state_pool and snapshots must be 16-byte aligned", who);
    if (((a->HV * a->V * a->K) & 3) != 0)
        return fail(KDA_ERR_UNSUPPORTED, "%s: HV*V*K must be a multiple of 4", who);
    if (a->conv_state != nullptr) {
        if (!valid_dtype(a->dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", who, a->dtype);
        if (a->conv_width < 2 || a->conv_width > 4)
            return fail(KDA_ERR_UNSUPPORTED, "%s: conv_width must be in [2, 4] (got %lld)", who, (long long)a->conv_width);
        if (a->mixed_qkv == nullptr || a->conv_dim <= 0 || a->mixed_stride < a->conv_dim)
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: the conv roll needs mixed_qkv with conv_dim > 0 and mixed_stride >= conv_dim", who);
        if (a->num_conv_slots <= 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: num_conv_slots must be positive", who);
    }
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

size_t kda_args_size(int which) {
    switch (which) {
        case KDA_ARGS_PREFILL: return sizeof(kda_prefill_args);
        case KDA_ARGS_DECODE: return sizeof(kda_decode_args);
        case KDA_ARGS_VERIFY: return sizeof(kda_verify_args);
        case KDA_ARGS_COMMIT: return sizeof(kda_commit_args);
        case KDA_ARGS_CONV_UPDATE: return sizeof(kda_conv_update_args);
        case KDA_ARGS_DECODE_CONV: return sizeof(kda_decode_conv_args);
        default: return 0;
    }
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

kda_status_t kda_set_call_events(void* start_event, void* stop_event) {
    kda::CallEvents& ev = kda::call_events();
    ev.start = static_cast<hipEvent_t>(start_event);
    ev.stop = static_cast<hipEvent_t>(stop_event);
    return ok();
}

kda_status_t kda_prefill_workspace_size(const kda_prefill_args* args, size_t* bytes) {
    if (bytes == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "KDA prefill: bytes is NULL");
    kda_status_t st = validate_prefill(args);
    if (st != KDA_OK) return st;
    *bytes = (args->B == 0 || args->T == 0) ? 0 : kda::prefill_workspace_bytes(*args);
    return ok();
}

kda_status_t kda_prefill_path(const kda_prefill_args* args, int32_t* path) {
    if (path == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "KDA prefill: path is NULL");
    kda_status_t st = validate_prefill(args);
    if (st != KDA_OK) return st;
    *path = kda::prefill_mfma_eligible(*args) ? KDA_PREFILL_PATH_MATRIX : KDA_PREFILL_PATH_GENERAL;
    return ok();
}

kda_status_t kda_prefill(const kda_prefill_args* args, void* workspace, size_t workspace_bytes, void* stream) {
    ClearCallEvents clear_events;
    kda_status_t st = validate_prefill(args);
    if (st != KDA_OK) return st;
    if (args->B == 0 || args->T == 0) return ok();
    const size_t need = kda::prefill_workspace_bytes(*args);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(KDA_ERR_INVALID_ARGUMENT, "KDA prefill: workspace of %zu bytes required (got %zu)", need,
                    workspace == nullptr ? size_t(0) : workspace_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "KDA prefill: workspace must be 256-byte aligned");
    return hip_status(kda::launch_prefill(*args, workspace, static_cast<hipStream_t>(stream)), "KDA prefill launch");
}

kda_status_t kda_prefill_noalloc(const kda_prefill_args* args, void* stream) {
    ClearCallEvents clear_events;
    kda_status_t st = validate_prefill(args);
    if (st != KDA_OK) return st;
    if (args->B == 0 || args->T == 0) return ok();
    const size_t need = kda::prefill_workspace_bytes(*args);
    if (need > KDA_NOALLOC_SCRATCH_BYTES)
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "KDA prefill (no allocation): needs %zu bytes of workspace, the built-in scratch holds %zu",
                    need, static_cast<size_t>(KDA_NOALLOC_SCRATCH_BYTES));
    void* ws = nullptr;
    hipError_t e = kda::noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "KDA prefill (no allocation): scratch address");
    return hip_status(kda::launch_prefill(*args, ws, static_cast<hipStream_t>(stream)),
                      "KDA prefill (no allocation) launch");
}

kda_status_t kda_decode(const kda_decode_args* args, void* stream) {
    ClearCallEvents clear_events;
    kda_status_t st = validate_decode(args);
    if (st != KDA_OK) return st;
    if (args->B == 0) return ok();
    return hip_status(kda::launch_decode(*args, static_cast<hipStream_t>(stream)), "KDA decode launch");
}

kda_status_t kda_decode_conv(const kda_decode_conv_args* args, void* stream) {
    ClearCallEvents clear_events;
    kda_status_t st = validate_decode_conv(args);
    if (st != KDA_OK) return st;
    if (args->B == 0) return ok();
    return hip_status(kda::launch_decode_conv(*args, static_cast<hipStream_t>(stream)), "KDA decode+conv launch");
}

kda_status_t kda_verify(const kda_verify_args* args, void* stream) {
    ClearCallEvents clear_events;
    kda_status_t st = validate_verify(args, false);
    if (st != KDA_OK) return st;
    if (args->B == 0) return ok();
    return hip_status(kda::launch_verify(*args, static_cast<hipStream_t>(stream)), "KDA verify launch");
}

kda_status_t kda_conv_update(const kda_conv_update_args* args, void* stream) {
    ClearCallEvents clear_events;
    kda_status_t st = validate_conv_update(args);
    if (st != KDA_OK) return st;
    if (args->B == 0) return ok();
    return hip_status(kda::launch_conv_update(*args, static_cast<hipStream_t>(stream)), "KDA conv update launch");
}

kda_status_t kda_commit_replay(const kda_verify_args* args, const int32_t* accepted, void* stream) {
    ClearCallEvents clear_events;
    kda_status_t st = validate_verify(args, true);
    if (st != KDA_OK) return st;
    if (accepted == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "KDA commit replay: accepted is required");
    if (args->B == 0) return ok();
    return hip_status(kda::launch_commit_replay(*args, accepted, static_cast<hipStream_t>(stream)),
                      "KDA commit replay launch");
}

kda_status_t kda_commit(const kda_commit_args* args, void* stream) {
    ClearCallEvents clear_events;
    kda_status_t st = validate_commit(args);
    if (st != KDA_OK) return st;
    if (args->B == 0) return ok();
    return hip_status(kda::launch_commit(*args, static_cast<hipStream_t>(stream)), "KDA commit launch");
}

}  // extern "C"
