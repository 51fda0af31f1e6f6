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

#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {
namespace {

constexpr int kConvThreads = 256;
constexpr int kMaxK = 8;

__device__ __forceinline__ int find_seq(const int32_t *cu, int N, int r)
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

__global__ __launch_bounds__(kConvThreads) void conv_kernel(ConvParams p)
{
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
    const int W = p.K - 1;
    if (t != 0 && t < W)
        return;  // computed by the token-0 thread of this (sequence, channel)

    float w[kMaxK];
    for (int m = 0; m < p.K; ++m)
        w[m] = load_act(p.w, (int64_t)c * p.K + m, p.x_dt);
    const int64_t sbase = ((int64_t)seq * p.C + c) * W;

    if (t >= W) {
        float acc = 0.f;
        for (int m = 0; m < p.K; ++m)
            acc += w[m] * load_act(p.x, (int64_t)(start + t + m - W) * p.x_stride + c, p.x_dt);
        store_act(p.y, (int64_t)r * p.y_stride + c, p.y_dt, silu_f(acc));
        return;
    }

    // t == 0: tokens [0, min(W, len)) and the state window
    float old[kMaxK];
    for (int m = 0; m < W; ++m)
        old[m] = load_act(p.state, sbase + m, p.x_dt);
    const int tend = min(W, len);
    for (int tt = 0; tt < tend; ++tt) {
        float acc = 0.f;
        for (int m = 0; m < p.K; ++m) {
            const int j = tt + m - W;
            const float xv = j >= 0 ? load_act(p.x, (int64_t)(start + j) * p.x_stride + c, p.x_dt)
                                    : old[W + j];
            acc += w[m] * xv;
        }
        store_act(p.y, (int64_t)(start + tt) * p.y_stride + c, p.y_dt, silu_f(acc));
    }
    for (int pos = 0; pos < W; ++pos) {
        const int j = len + pos - W;
        const float xv = j >= 0 ? load_act(p.x, (int64_t)(start + j) * p.x_stride + c, p.x_dt)
                                : old[W + j];
        // the window holds raw inputs, so the value is exactly representable in x_dt
        store_act(p.state, sbase + pos, p.x_dt, xv);
    }
}

}  // namespace

hipError_t launch_conv(const ConvParams &p, hipStream_t s)
{
    if (p.total == 0 || p.C == 0)
        return hipSuccess;
    const int64_t cblocks = (p.C + kConvThreads - 1) / kConvThreads;
    const int64_t blocks = cblocks * p.total;
    hipLaunchKernelGGL(conv_kernel, dim3((unsigned)blocks), dim3(kConvThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace gdn
