// gdn_decode.hip -- batched decode step of the gated delta rule on gfx950.
//
// Per token t and v-head h (k-head kh by the head map), every value row j of the
// fp32 state S[dv][dk] (key index innermost) goes through
//     S_j <- a S_j,  p_j = S_j . k,  d_j = beta (v_j - p_j),  S_j <- S_j + d_j k,
//     o_j = scale (S_j . q)
// (docs.rs ferrox-core 0.24.0 src/gdn.rs, module doc and `delta_step`; the
// ferrum-kernels 0.8.0 tests page, `cpu_segment`). Around it, fused in the same
// kernel: the q/k L2 norm, the gates from raw a/b, and the gated RMS norm of the
// output (same `cpu_segment`).
//
// Design (HBM bound: 0.5 flop per state byte):
//  * one workgroup per (sequence, v-head), NW waves; wave w owns value rows
//    [w*DV/NW, (w+1)*DV/NW). A row's DK floats are spread over DK/4 lanes as one
//    float4 each, so one dwordx4 wave load moves 64/(DK/4) whole rows (1 KiB).
//  * every state row is loaded into VGPRs once per call, carried through all of
//    the call's tokens (rows are independent), and stored once.
//  * the two row dot products use the old state: S_j.k and S_j.q are reduced
//    together (DPP butterflies over the row's lanes), then
//        p_j = a (S_j.k),  o_j = scale (a (S_j.q) + d_j (k.q)),
//    which is S_new.q expanded -- the same value in another rounding order (the
//    ferrox-core page notes this expansion next to its throughput probe).
//  * v for the token is staged in LDS; outputs are gathered in LDS and the gated
//    RMS norm runs over them after the token group.

#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {
namespace {

constexpr int kTokGroup = 8;  // tokens whose outputs are buffered in LDS at once

template <int DK, int DV, int NW>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeParams p)
{
    constexpr int LPR = DK / 4;       // lanes holding one row
    constexpr int RPI = 64 / LPR;     // rows per wave-wide load
    constexpr int RPW = DV / NW;      // rows per wave
    constexpr int NI = RPW / RPI;     // float4 row pieces per lane
    static_assert(DK % 4 == 0 && 64 % LPR == 0 && RPW % RPI == 0 && NI >= 1, "shape");

    __shared__ float v_s[kTokGroup][DV];
    __shared__ float o_s[kTokGroup][DV];

    const HeadCfg &hc = p.hc;
    const ActInputs &in = p.in;
    const int Hv = hc.Hv;
    const int h = blockIdx.x % Hv;
    const int b = blockIdx.x / Hv;
    const int slot = p.slots ? p.slots[b] : b;
    if (slot < 0 || slot >= p.num_slots)
        return;  // whole workgroup leaves before any barrier
    const int kh = k_head_of(hc.head_map, h, hc.Hk, Hv);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane / LPR;
    const int col = (lane % LPR) * 4;
    const uint32_t flags = hc.flags;

    float *Sg = p.state + ((int64_t)slot * Hv + h) * (int64_t)(DV * DK);
    const int row0 = wave * RPW + sub;

    float4 S[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i)
        S[i] = *reinterpret_cast<const float4 *>(Sg + (row0 + i * RPI) * DK + col);

    float dec_rate = 0.f, dtb = 0.f;
    if (flags & F_RAW_GATES) {
        float dp = in.decay_param[h];
        dec_rate = hc.decay_kind == 0 ? -expf(dp) : dp;
        dtb = in.dt_bias[h];
    }

    for (int t0 = 0; t0 < p.T; t0 += kTokGroup) {
        const int tn = min(kTokGroup, p.T - t0);
        for (int idx = threadIdx.x; idx < tn * DV; idx += NW * 64) {
            const int tt = idx / DV, j = idx % DV;
            const int64_t r = (int64_t)b * p.T + t0 + tt;
            v_s[tt][j] = load_act(in.v, r * in.v_stride + (int64_t)h * DV + j, in.qkv_dt);
        }
        __syncthreads();

        for (int tt = 0; tt < tn; ++tt) {
            const int64_t r = (int64_t)b * p.T + t0 + tt;
            float4 kk = load_act4(in.k, r * in.k_stride + (int64_t)kh * DK + col, in.qkv_dt);
            float4 qq = load_act4(in.q, r * in.q_stride + (int64_t)kh * DK + col, in.qkv_dt);
            if (flags & F_L2NORM) {
                const float sk = group_sum<LPR>(dot4(kk, kk));
                const float sq = group_sum<LPR>(dot4(qq, qq));
                const float ik = rsqrtf(sk + hc.l2_eps), iq = rsqrtf(sq + hc.l2_eps);
                kk.x *= ik; kk.y *= ik; kk.z *= ik; kk.w *= ik;
                qq.x *= iq; qq.y *= iq; qq.z *= iq; qq.w *= iq;
            }
            float g, beta;
            if (flags & F_RAW_GATES) {
                const float av = load_act(in.a, r * Hv + h, in.ab_dt);
                const float bv = load_act(in.b, r * Hv + h, in.ab_dt);
                g = dec_rate * softplus_f(av + dtb);
                beta = sigmoid_f(bv);
            } else {
                g = in.g[r * Hv + h];
                beta = in.beta[r * Hv + h];
            }
            const float alpha = expf(g);
            const float kq = group_sum<LPR>(dot4(kk, qq));

            float pk[NI], pq[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                pk[i] = dot4(S[i], kk);
                pq[i] = dot4(S[i], qq);
            }
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                pk[i] = group_sum<LPR>(pk[i]);
                pq[i] = group_sum<LPR>(pq[i]);
            }
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int row = row0 + i * RPI;
                const float d = beta * (v_s[tt][row] - alpha * pk[i]);
                const float o = hc.scale * (alpha * pq[i] + d * kq);
                S[i].x = fmaf(alpha, S[i].x, d * kk.x);
                S[i].y = fmaf(alpha, S[i].y, d * kk.y);
                S[i].z = fmaf(alpha, S[i].z, d * kk.z);
                S[i].w = fmaf(alpha, S[i].w, d * kk.w);
                if (col == 0)
                    o_s[tt][row] = o;
            }
        }
        __syncthreads();

        // epilogue: one wave per token of the group
        for (int tt = wave; tt < tn; tt += NW) {
            const int64_t r = (int64_t)b * p.T + t0 + tt;
            const int64_t obase = (r * Hv + h) * DV;
            if (flags & F_GATED_NORM) {
                float ss = 0.f;
                for (int j = lane; j < DV; j += 64)
                    ss += o_s[tt][j] * o_s[tt][j];
                ss = group_sum<64>(ss);
                const float inv = rsqrtf(ss / (float)DV + hc.norm_eps);
                for (int j = lane; j < DV; j += 64) {
                    const float zv = load_act(in.z, obase + j, in.z_dt);
                    store_act(p.out, obase + j, p.out_dt, o_s[tt][j] * inv * in.norm_w[j] * silu_f(zv));
                }
            } else {
                for (int j = lane; j < DV; j += 64)
                    store_act(p.out, obase + j, p.out_dt, o_s[tt][j]);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < NI; ++i)
        *reinterpret_cast<float4 *>(Sg + (row0 + i * RPI) * DK + col) = S[i];
}

template <int DK, int DV, int NW>
hipError_t launch_decode_t(const DecodeParams &p, hipStream_t s)
{
    const int64_t blocks = (int64_t)p.B * p.hc.Hv;
    hipLaunchKernelGGL((decode_kernel<DK, DV, NW>), dim3((unsigned)blocks), dim3(NW * 64), 0, s, p);
    return hipGetLastError();
}

}  // namespace

bool decode_supported(int dk, int dv)
{
    return (dk == 128 && dv == 128) || (dk == 64 && dv == 64) || (dk == 32 && dv == 32);
}

hipError_t launch_decode(const DecodeParams &p, hipStream_t s)
{
    if (p.B == 0)
        return hipSuccess;
    if (p.hc.dk == 128 && p.hc.dv == 128)
        return launch_decode_t<128, 128, 4>(p, s);
    if (p.hc.dk == 64 && p.hc.dv == 64)
        return launch_decode_t<64, 64, 4>(p, s);
    if (p.hc.dk == 32 && p.hc.dv == 32)
        return launch_decode_t<32, 32, 4>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace gdn
