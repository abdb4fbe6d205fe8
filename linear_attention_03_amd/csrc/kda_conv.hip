// Conv update before a packed decode: the depthwise causal conv (width W)
// of one new token per request, with the conv state rolled in place.  The
// conv is the one fused into the verify kernel ("[KDA] Default GLM-5-Next
// spec verify to the CuTe DSL KDA kernel", Summary: conv1d, then the
// recurrence); here it stands alone so that a decode step can consume its
// q || k || v output as strided views.
//
// One thread per (request, channel): the thread reads its W-1 state
// entries, the new input and the channel's weights, writes the output and
// the shifted state.  Every element has one owner, so y may alias x.  The
// grid's x dimension covers the channels in blocks of 256, y the requests;
// a block reads 256 (W-1) contiguous state entries.

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

struct ConvParams {
    const void* x;
    int64_t xs;
    void* y;
    int64_t ys;
    const void* w;
    const void* bias;
    void* cs;
    const int32_t* cidx;
    int64_t C;
    int W, num_slots, act;
};

template <typename T, int W>
__global__ __launch_bounds__(256) void conv_update_kernel(const ConvParams p) {
    const int r = blockIdx.y;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= p.C) return;
    T* y = static_cast<T*>(p.y) + (int64_t)r * p.ys + c;
    const int s = p.cidx[r];
    if (s < 0 || s >= p.num_slots) {            // padded request
        *y = from_f32<T>(0.0f);
        return;
    }
    const T xin = static_cast<const T*>(p.x)[(int64_t)r * p.xs + c];
    T* st = static_cast<T*>(p.cs) + ((int64_t)s * p.C + c) * (W - 1);
    const T* wc = static_cast<const T*>(p.w) + c * W;
    T old[W - 1];
    float wv[W];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) old[j] = st[j];
#pragma unroll
    for (int j = 0; j < W; ++j) wv[j] = to_f32(wc[j]);
    const float b = p.bias ? ld(static_cast<const T*>(p.bias), c) : 0.0f;
    // newest first, as in the verify kernel's conv
    float acc = fmaf(wv[W - 1], to_f32(xin), b);
#pragma unroll
    for (int j = W - 2; j >= 0; --j) acc = fmaf(wv[j], to_f32(old[j]), acc);
    if (p.act == KDA_ACT_SILU) acc = acc * sigmoidf(acc);
    *y = from_f32<T>(acc);
#pragma unroll
    for (int j = 0; j < W - 2; ++j) st[j] = old[j + 1];
    st[W - 2] = xin;
}

template <typename T>
hipError_t launch_t(const ConvParams& p, int64_t B, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>((p.C + 255) / 256), static_cast<unsigned>(B));
    switch (p.W) {
        case 2: klaunch(conv_update_kernel<T, 2>, grid, dim3(256), 0, s, p); break;
        case 3: klaunch(conv_update_kernel<T, 3>, grid, dim3(256), 0, s, p); break;
        default: klaunch(conv_update_kernel<T, 4>, grid, dim3(256), 0, s, p); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_update(const kda_conv_update_args& a, hipStream_t s) {
    ConvParams p;
    p.x = a.x; p.xs = a.x_stride; p.y = a.y; p.ys = a.y_stride;
    p.w = a.conv_weight; p.bias = a.conv_bias; p.cs = a.conv_state; p.cidx = a.conv_state_indices;
    p.C = a.conv_dim;
    p.W = static_cast<int>(a.conv_width);
    p.num_slots = static_cast<int>(a.num_conv_slots);
    p.act = a.conv_activation;
    return a.dtype == KDA_BF16 ? launch_t<bf16>(p, a.B, s) : launch_t<float>(p, a.B, s);
}

}  // namespace kda
