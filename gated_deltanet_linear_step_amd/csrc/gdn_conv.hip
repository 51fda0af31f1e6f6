// gdn_conv.hip -- depthwise causal conv1d + SiLU with carried raw inputs (gfx950).
//
// For sequence i and channel c, output token t of the sequence is
//     y = silu( sum_{m<K} w[c][m] * xhat(t + m - (K-1)) )
// with xhat(j) = x[start_i + j][c] for j >= 0, else the carried state
// state[i][c][(K-1) + j]; the new state is the last K-1 entries of
// [state || x_i] (ferrum-kernels 0.8.0 tests page, `cpu_segment` conv section;
// libmir-metal 0.1.0 decode page, `convolve`).
//
// One thread per (token, channel); threads of a block share one token row, so
// x and y accesses are coalesced along channels. Tokens t < K-1 are the only
// ones that read the old state, so the thread of token 0 computes all of them
// AND writes the new window: no other thread reads or writes that channel's
// state, which removes the read-before-overwrite hazard without a second pass.
// Every thread issues all of its loads before its first store (the pointers
// are restrict-qualified), so each thread costs one memory round trip.

#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {
namespace {

constexpr int kConvThreads = 256;

__device__ __forceinline__ int find_seq(const int32_t *__restrict__ cu, int N, int r)
{
    // largest i with cu[i] <= r (cu non-decreasing, cu[0] = 0, r < cu[N])
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= r)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

template <int K>
__global__ __launch_bounds__(kConvThreads) void conv_kernel(ConvParams p)
{
    constexpr int W = K - 1;
    const void *__restrict__ xg = p.x;
    const void *__restrict__ wg = p.w;
    void *__restrict__ sg = p.state;
    void *__restrict__ yg = p.y;

    const int cblocks = (p.C + kConvThreads - 1) / kConvThreads;
    const int r = blockIdx.x / cblocks;
    const int c = (blockIdx.x % cblocks) * kConvThreads + threadIdx.x;
    if (r >= p.total || c >= p.C)
        return;
    int seq, start, len;
    if (p.cu) {
        seq = find_seq(p.cu, p.N, r);
        start = p.cu[seq];
        len = p.cu[seq + 1] - start;
    } else {
        seq = r / p.uniform_len;
        start = seq * p.uniform_len;
        len = p.uniform_len;
    }
    const int t = r - start;
    if (t != 0 && t < W)
        return;  // computed by the token-0 thread of this (sequence, channel)

    float w[K];
#pragma unroll
    for (int m = 0; m < K; ++m)
        w[m] = load_act(wg, (int64_t)c * K + m, p.x_dt);

    if (t >= W) {
        float xv[K];
#pragma unroll
        for (int m = 0; m < K; ++m)
            xv[m] = load_act(xg, (int64_t)(start + t + m - W) * p.x_stride + c, p.x_dt);
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < K; ++m)
            acc += w[m] * xv[m];
        store_act(yg, (int64_t)r * p.y_stride + c, p.y_dt, silu_f(acc));
        return;
    }

    // t == 0: win[W + j] = xhat(j) for j in [-W, W) covers every output token
    // that touches the old state; the new window is xhat(len - W .. len - 1).
    const int64_t sbase = ((int64_t)seq * p.C + c) * W;
    float win[2 * W];
#pragma unroll
    for (int m = 0; m < W; ++m)
        win[m] = load_act(sg, sbase + m, p.x_dt);
#pragma unroll
    for (int j = 0; j < W; ++j)
        win[W + j] = j < len ? load_act(xg, (int64_t)(start + j) * p.x_stride + c, p.x_dt) : 0.f;
    float tail[W];
#pragma unroll
    for (int pos = 0; pos < W; ++pos) {
        const int j = len + pos - W;  // >= 1 - W since len >= 1
        if (j >= W) {
            tail[pos] = load_act(xg, (int64_t)(start + j) * p.x_stride + c, p.x_dt);
        } else {
            float v = 0.f;  // win[W + j] by a select chain (keeps win in registers)
#pragma unroll
            for (int e = 0; e < 2 * W; ++e)
                v = (e == W + j) ? win[e] : v;
            tail[pos] = v;
        }
    }
    const int tend = len < W ? len : W;
#pragma unroll
    for (int tt = 0; tt < W; ++tt) {
        if (tt < tend) {
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < K; ++m)
                acc += w[m] * win[tt + m];
            store_act(yg, (int64_t)(start + tt) * p.y_stride + c, p.y_dt, silu_f(acc));
        }
    }
    // the window holds raw inputs, so each value is exactly representable in x_dt
#pragma unroll
    for (int pos = 0; pos < W; ++pos)
        store_act(sg, sbase + pos, p.x_dt, tail[pos]);
}

// Decode shape: one token per sequence, K = 4, C % 4 == 0. Thread per
// (sequence, 4 consecutive channels): the taps, the 3-entry windows and the
// inputs of the 4 channels are contiguous, so each is one vector load.
template <int XT, int YT>
__global__ __launch_bounds__(kConvThreads) void conv_step4_kernel(ConvParams p)
{
    const int groups = p.C / 4;
    const int64_t idx = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
    if (idx >= (int64_t)p.N * groups)
        return;
    const int seq = (int)(idx / groups);
    const int c = (int)(idx % groups) * 4;
    float w[4][4], win[4][3], x[4];
    if constexpr (XT == DT_F32) {
        const float4 *wp = reinterpret_cast<const float4 *>(static_cast<const float *>(p.w) + (int64_t)c * 4);
        const float4 *sp = reinterpret_cast<const float4 *>(static_cast<const float *>(p.state) + ((int64_t)seq * p.C + c) * 3);
        const float4 xv = *reinterpret_cast<const float4 *>(static_cast<const float *>(p.x) + (int64_t)seq * p.x_stride + c);
        float wf[16], sf[12];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 v = wp[j];
            wf[4 * j] = v.x; wf[4 * j + 1] = v.y; wf[4 * j + 2] = v.z; wf[4 * j + 3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const float4 v = sp[j];
            sf[4 * j] = v.x; sf[4 * j + 1] = v.y; sf[4 * j + 2] = v.z; sf[4 * j + 3] = v.w;
        }
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
            for (int m = 0; m < 4; ++m) w[ch][m] = wf[ch * 4 + m];
#pragma unroll
            for (int m = 0; m < 3; ++m) win[ch][m] = sf[ch * 3 + m];
        }
        x[0] = xv.x; x[1] = xv.y; x[2] = xv.z; x[3] = xv.w;
    } else {
        const uint4 *wp = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.w) + (int64_t)c * 4);
        const uint2 *sp = reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.state) + ((int64_t)seq * p.C + c) * 3);
        const uint2 xv = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.x) + (int64_t)seq * p.x_stride + c);
        uint32_t wb[8], sb[6];
        const uint4 w0 = wp[0], w1 = wp[1];
        wb[0] = w0.x; wb[1] = w0.y; wb[2] = w0.z; wb[3] = w0.w;
        wb[4] = w1.x; wb[5] = w1.y; wb[6] = w1.z; wb[7] = w1.w;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const uint2 v = sp[j];
            sb[2 * j] = v.x; sb[2 * j + 1] = v.y;
        }
        auto cvt = [](uint32_t word, int half) {
            const uint32_t h = half ? (word >> 16) : (word & 0xffffu);
            return XT == DT_BF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
        };
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int e = ch * 4 + m;
                w[ch][m] = cvt(wb[e >> 1], e & 1);
            }
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                const int e = ch * 3 + m;
                win[ch][m] = cvt(sb[e >> 1], e & 1);
            }
        }
        x[0] = cvt(xv.x, 0); x[1] = cvt(xv.x, 1); x[2] = cvt(xv.y, 0); x[3] = cvt(xv.y, 1);
    }
    float y[4];
#pragma unroll
    for (int ch = 0; ch < 4; ++ch)
        y[ch] = silu_f(w[ch][0] * win[ch][0] + w[ch][1] * win[ch][1] + w[ch][2] * win[ch][2] +
                       w[ch][3] * x[ch]);
    // outputs
    if constexpr (YT == DT_F32) {
        *reinterpret_cast<float4 *>(static_cast<float *>(p.y) + (int64_t)seq * p.y_stride + c) =
            make_float4(y[0], y[1], y[2], y[3]);
    } else {
        auto pack = [](float v) {
            return (uint32_t)(YT == DT_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v));
        };
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.y) + (int64_t)seq * p.y_stride + c) =
            make_uint2(pack(y[0]) | (pack(y[1]) << 16), pack(y[2]) | (pack(y[3]) << 16));
    }
    // new windows: (win1, win2, x) per channel, raw values in x's dtype
    if constexpr (XT == DT_F32) {
        float4 *sp = reinterpret_cast<float4 *>(static_cast<float *>(p.state) + ((int64_t)seq * p.C + c) * 3);
        sp[0] = make_float4(win[0][1], win[0][2], x[0], win[1][1]);
        sp[1] = make_float4(win[1][2], x[1], win[2][1], win[2][2]);
        sp[2] = make_float4(x[2], win[3][1], win[3][2], x[3]);
    } else {
        // re-pack the raw 16-bit bits (exact: they came from the same dtype)
        auto bits = [](float v) {
            return (uint32_t)(XT == DT_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v));
        };
        uint32_t nb[12];
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
            nb[ch * 3] = bits(win[ch][1]);
            nb[ch * 3 + 1] = bits(win[ch][2]);
            nb[ch * 3 + 2] = bits(x[ch]);
        }
        uint2 *sp = reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.state) + ((int64_t)seq * p.C + c) * 3);
#pragma unroll
        for (int j = 0; j < 3; ++j)
            sp[j] = make_uint2(nb[4 * j] | (nb[4 * j + 1] << 16), nb[4 * j + 2] | (nb[4 * j + 3] << 16));
    }
}

template <int XT>
hipError_t launch_step4_x(const ConvParams &p, hipStream_t s)
{
    const int64_t threads = (int64_t)p.N * (p.C / 4);
    const dim3 grid((unsigned)((threads + kConvThreads - 1) / kConvThreads)), block(kConvThreads);
    switch (p.y_dt) {
    case DT_F32: hipLaunchKernelGGL((conv_step4_kernel<XT, DT_F32>), grid, block, 0, s, p); break;
    case DT_F16: hipLaunchKernelGGL((conv_step4_kernel<XT, DT_F16>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((conv_step4_kernel<XT, DT_BF16>), grid, block, 0, s, p); break;
    }
    return hipGetLastError();
}

template <int K>
hipError_t launch_conv_t(const ConvParams &p, hipStream_t s)
{
    const int64_t cblocks = (p.C + kConvThreads - 1) / kConvThreads;
    hipLaunchKernelGGL(conv_kernel<K>, dim3((unsigned)(cblocks * p.total)), dim3(kConvThreads), 0,
                       s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv(const ConvParams &p, hipStream_t s)
{
    if (p.total == 0 || p.C == 0)
        return hipSuccess;
    // one token per sequence with vector-friendly layouts: the vectorised path
    const int xs = p.x_dt == DT_F32 ? 4 : 2, ys = p.y_dt == DT_F32 ? 4 : 2;
    const bool vec_ok = p.K == 4 && !p.cu && p.uniform_len == 1 && p.C % 4 == 0 &&
                        p.x_stride % 4 == 0 && p.y_stride % 4 == 0 &&
                        reinterpret_cast<uintptr_t>(p.x) % (4 * xs) == 0 &&
                        reinterpret_cast<uintptr_t>(p.y) % (4 * ys) == 0 &&
                        reinterpret_cast<uintptr_t>(p.w) % (16 * xs) == 0 &&
                        reinterpret_cast<uintptr_t>(p.state) % (4 * xs) == 0;
    if (vec_ok) {
        switch (p.x_dt) {
        case DT_F32: return launch_step4_x<DT_F32>(p, s);
        case DT_F16: return launch_step4_x<DT_F16>(p, s);
        default: return launch_step4_x<DT_BF16>(p, s);
        }
    }
    switch (p.K) {
    case 2: return launch_conv_t<2>(p, s);
    case 3: return launch_conv_t<3>(p, s);
    case 4: return launch_conv_t<4>(p, s);
    case 5: return launch_conv_t<5>(p, s);
    case 6: return launch_conv_t<6>(p, s);
    case 7: return launch_conv_t<7>(p, s);
    case 8: return launch_conv_t<8>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
