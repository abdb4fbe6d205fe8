// Device helpers shared by the libkda kernels: bfloat16 conversion, typed
// element loads, wave64 lane reductions and the per-token preprocessing
// (gate map, beta, L2 norm).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr float kL2Eps = 1e-6f;

// bfloat16 stored as its 16 raw bits.
struct bf16 {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return __uint_as_float(uint32_t(x.bits) << 16); }

// float32 -> bfloat16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16 f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return bf16{uint16_t((u >> 16) | 0x40u)};
    u += 0x7fffu + ((u >> 16) & 1u);
    return bf16{uint16_t(u >> 16)};
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return f32_to_bf16(x); }

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i) { return to_f32(p[i]); }

// Four consecutive elements starting at p[i] (i a multiple of 4).
__device__ __forceinline__ float4 ld4(const float* p, int64_t i) {
    return *reinterpret_cast<const float4*>(p + i);
}
__device__ __forceinline__ float4 ld4(const bf16* p, int64_t i) {
    const uint2 u = *reinterpret_cast<const uint2*>(p + i);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

// Barrier for LDS hand-offs between the waves of a block.  The fences
// cover LDS only, so the barrier waits for this wave's LDS operations but
// leaves its global loads in flight (a plain __syncthreads() fences global
// memory as well and drains every outstanding load first).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum over aligned groups of W lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = W / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// Sum over aligned groups of W lanes (W in {4, 8, 16, 32}) in the VALU:
// quad permutes, then the half-row and row mirrors (each pairs a group with
// its neighbour), then a swizzle that exchanges the two 16-lane rows of a
// 32-lane half.  Every lane of a group ends with the same bits.
__device__ __forceinline__ float dpp_add(float x, int v) { return x + __int_as_float(v); }

template <int W>
__device__ __forceinline__ float lane_sum(float x) {
    static_assert(W == 4 || W == 8 || W == 16 || W == 32, "group width");
    constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;
    x = dpp_add(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), kXor1, 0xF, 0xF, false));
    x = dpp_add(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), kXor2, 0xF, 0xF, false));
    if constexpr (W >= 8) x = dpp_add(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), kHalfMirror, 0xF, 0xF, false));
    if constexpr (W >= 16) x = dpp_add(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), kMirror, 0xF, 0xF, false));
    if constexpr (W >= 32) x = dpp_add(x, __builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
    return x;
}

// Sum over the whole wave, returned in every lane.
__device__ __forceinline__ float wave_sum(float x) {
    x = lane_sum<32>(x);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
}

__device__ __forceinline__ float uniform_f(float x) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

__device__ __forceinline__ int group_sum_int(int x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// 1 / (1 + e^-x) with the hardware reciprocal (1 ulp) instead of a
// correctly rounded division (a ten-instruction sequence).
__device__ __forceinline__ float sigmoidf(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// Gate map (reading of the A_log / dt_bias / lower_bound arguments), by
// mode: kGateRaw (A_log == NULL): the raw value already is the log-decay;
// kGateBounded: g = lower_bound * sigmoid(exp(A_log) (raw + dt_bias));
// kGateUnbounded (A_log without lower_bound):
// g = -exp(A_log) softplus(raw + dt_bias), with softplus(x) =
// max(x, 0) + log(1 + e^-|x|).
enum GateMode { kGateRaw = 0, kGateBounded = 1, kGateUnbounded = 2 };

__device__ __forceinline__ float softplusf(float x) {
    return fmaxf(x, 0.0f) + __logf(1.0f + __expf(-fabsf(x)));
}

__device__ __forceinline__ float log_gate(float raw, int mode, float expA, float dt, float lb) {
    if (mode == kGateBounded) return lb * sigmoidf(expA * (raw + dt));
    if (mode == kGateUnbounded) return -expA * softplusf(raw + dt);
    return raw;
}

// exp(g)
__device__ __forceinline__ float gate_decay(float raw, int mode, float expA, float dt, float lb) {
    return __expf(log_gate(raw, mode, expA, dt, lb));
}

// Host side: the mode of a call's gate arguments.
inline int gate_mode(const float* A_log, int32_t has_lower_bound) {
    return A_log == nullptr ? kGateRaw : has_lower_bound ? kGateBounded : kGateUnbounded;
}

__device__ __forceinline__ float fdot4(float4 a, float4 b) {
    return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

__device__ __forceinline__ float4 f4scale(float4 a, float s) { return make_float4(a.x * s, a.y * s, a.z * s, a.w * s); }

__device__ __forceinline__ float4 f4mul(float4 a, float4 b) {
    return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}

__device__ __forceinline__ float4 f4fma(float4 a, float s, float4 c) {
    return make_float4(fmaf(a.x, s, c.x), fmaf(a.y, s, c.y), fmaf(a.z, s, c.z), fmaf(a.w, s, c.w));
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming store (non-temporal: the line is not kept in cache).
__device__ __forceinline__ void st4_nt(float* p, float4 v) {
    f32x4 t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(p));
}

__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }

}  // namespace kda
