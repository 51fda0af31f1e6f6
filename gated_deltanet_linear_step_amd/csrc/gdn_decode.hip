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
//    [w*DV/NW, (w+1)*DV/NW). A row's DK floats are spread over LPR lanes, each
//    holding DK/(4 LPR) float4 pieces of it: lane r of a row holds the columns
//    4r + 4 LPR m. One dwordx4 wave load moves piece m of 64/LPR rows, each as
//    a contiguous 16 LPR-byte run. The row dot products then reduce over LPR
//    lanes only (DPP within a row of 16 lanes when LPR <= 16, no LDS step).
//  * every state row is loaded into VGPRs once per call, carried through all of
//    the call's tokens (rows are independent), and stored once.
//  * the two row dot products use the old state: S_j.k and S_j.q are reduced
//    together (DPP butterflies over the row's lanes), then
//        p_j = a (S_j.k),  o_j = scale (a (S_j.q) + d_j (k.q)),
//    which is S_new.q expanded -- the same value in another rounding order (the
//    ferrox-core page notes this expansion next to its throughput probe).
//  * a token's activations are loaded before anything that waits on them, and
//    nothing waits on memory before the state loads are issued (kernel
//    arguments fetched in one round trip, gate words as vector loads, the conv
//    taps and window kept as raw words until after the state loads). In the
//    unfused step v arrives one element per lane and is spread to the rows by
//    shuffles; in the fused layer each lane reads its rows' v from the conv
//    output in LDS. The outputs are gathered in LDS and the gated RMS norm runs
//    over them after each group of tokens.
//  * CK > 0 (gdn_decode_layer): q, k, v arrive before the causal conv. Thread c
//    of the workgroup owns one of the 2 dk + dv channels it reads (its weights
//    and the window of the last CK-1 raw inputs in registers), convolves a group
//    of tokens into LDS, and the waves take q, k, v from there. The window after
//    the call goes to the output conv state; q/k channels are written by one
//    workgroup per k-head.
//  * Several tokens per sequence (fused layer): each token's norms, k.q and gates
//    are computed once per conv group, by one wave per token, and shared through
//    LDS instead of by every lane for every token. The operations are the
//    single-token path's, so a call and any split of it agree bit for bit.
//  * One token per sequence (the serving step): a kernel of its own, with no
//    token loop, so its registers fit easily; each wave forms the gated norm's
//    sum of squares over all rows (in the order the multi-token epilogue uses,
//    so results agree bit for bit) and stores its own rows' outputs.

#include "gdn_device.h"
#include "gdn_kernels.h"

#ifndef GDN_DECODE_NW
#define GDN_DECODE_NW 8  // waves per workgroup for the 128 x 128 state
#endif

namespace gdn {
namespace {

constexpr int kTokGroup = 8;  // tokens whose outputs are buffered in LDS at once

typedef float f32x4 __attribute__((ext_vector_type(4)));

// State pieces, plain or with non-temporal hints (GDN_STREAM_STATE: states that do
// not stay in the last-level cache between calls). At B=64 x 32 heads the plain
// form is 10 % faster while the 128 MiB state stays in the Infinity Cache; on
// streams past it (four rotating state sets, 48 layers at B=32) the hinted form is
// 11 % faster. Hinting only the stores, or only the loads, changes neither.
template <bool NT>
__device__ __forceinline__ float4 load_state4(const float *p)
{
    f32x4 v;
    if constexpr (NT)
        v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    else
        v = *reinterpret_cast<const f32x4 *>(p);
    return make_float4(v.x, v.y, v.z, v.w);
}

template <bool NT>
__device__ __forceinline__ void store_state4(float *p, float4 s)
{
    f32x4 v = {s.x, s.y, s.z, s.w};
    if constexpr (NT)
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
    else
        *reinterpret_cast<f32x4 *>(p) = v;
}

// Activations of one token for one wave, as raw bits: the k and q pieces, the
// two gate words (raw a/b or given g/beta) and one v element per lane. Loading
// and converting are separate so the state loads can be issued in between.
template <int QT, int PPR>
struct TokenRaw {
    Raw4<QT> k[PPR], q[PPR];
    GateWord ga, gb;
    uint32_t v;
};

// piece m of a lane that holds columns col + 4 LPR m of a row
template <int DK, int DV, int QT, int PPR, int LPR, bool QKV = true>
__device__ __forceinline__ void load_token(TokenRaw<QT, PPR> &t, const DecodeParams &p, int64_t r,
                                           int h, int kh, int col, int vrow)
{
    const ActInputs &in = p.in;
    const int Hv = p.hc.Hv;
    if constexpr (QKV) {
#pragma unroll
        for (int m = 0; m < PPR; ++m) {
            t.k[m] = load_raw4<QT>(in.k, r * in.k_stride + (int64_t)kh * DK + col + 4 * LPR * m);
            t.q[m] = load_raw4<QT>(in.q, r * in.q_stride + (int64_t)kh * DK + col + 4 * LPR * m);
        }
    }
    const bool raw = p.hc.flags & F_RAW_GATES;
    const int gdt = raw ? in.ab_dt : DT_F32;
    const int64_t gi = r * Hv + h + vgpr_zero();  // a vector load (see vgpr_zero)
    t.ga = load_gate(raw ? in.a : (const void *)in.g, gi, gdt);
    t.gb = load_gate(raw ? in.b : (const void *)in.beta, gi, gdt);
    if constexpr (QKV)
        t.v = load_raw1<QT>(in.v, r * in.v_stride + (int64_t)h * DV + vrow);
}

// The causal conv of one channel for the fused layer: weights and the window of
// the last CK-1 raw inputs (oldest first) in registers. w[0] pairs with the
// oldest input.
template <int QT, int CK>
struct ConvLane {
    static constexpr int ES = QT == DT_F32 ? 4 : 2;  // bytes per element
    float w[CK], win[CK - 1];
    // The channel's taps and window as loaded: one copy each of their contiguous
    // bytes, kept as whole words. Element loads would be merged into wider ones
    // and split again as they land, which makes the code wait for them right
    // there; convert() splits the words after the state loads are issued.
    uint32_t wr[(CK * ES + 3) / 4], winr[((CK - 1) * ES + 3) / 4];

    __device__ __forceinline__ void load(const DecodeParams &p, int64_t ch, int64_t sbase)
    {
        __builtin_memcpy(wr, static_cast<const char *>(p.conv_w) + ch * CK * ES, CK * ES);
        __builtin_memcpy(winr, static_cast<const char *>(p.conv_in) + sbase * ES, (CK - 1) * ES);
    }
    __device__ __forceinline__ void convert()
    {
        // the words enter here as opaque registers, so no part of the splitting
        // can be moved up next to the loads
#pragma unroll
        for (int i = 0; i < (int)(sizeof(wr) / 4); ++i)
            asm volatile("" : "+v"(wr[i]));
#pragma unroll
        for (int i = 0; i < (int)(sizeof(winr) / 4); ++i)
            asm volatile("" : "+v"(winr[i]));
#pragma unroll
        for (int m = 0; m < CK; ++m)
            w[m] = raw1_to_f32<QT>(element(wr, m));
#pragma unroll
        for (int m = 0; m < CK - 1; ++m)
            win[m] = raw1_to_f32<QT>(element(winr, m));
    }
    __device__ __forceinline__ static uint32_t element(const uint32_t *words, int m)
    {
        if constexpr (ES == 4)
            return words[m];
        else
            return (words[m / 2] >> (16 * (m % 2))) & 0xffffu;
    }
    __device__ __forceinline__ float tap(float x)
    {
        float acc = w[CK - 1] * x;
#pragma unroll
        for (int m = 0; m < CK - 1; ++m)
            acc = fmaf(w[m], win[m], acc);
#pragma unroll
        for (int m = 0; m < CK - 2; ++m)
            win[m] = win[m + 1];
        win[CK - 2] = x;
        return silu_f(acc);
    }
    __device__ __forceinline__ void store(const DecodeParams &p, int64_t sbase) const
    {
#pragma unroll
        for (int m = 0; m < CK - 1; ++m)
            store_act(p.conv_out, sbase + m, QT, win[m]);
    }
};

// A lane's share of a row dot product over its PPR pieces, as one explicit fused
// chain (for PPR = 1 it is dot4 itself)
template <int PPR>
__device__ __forceinline__ float dotn(const float4 *a, const float4 *b)
{
    float acc = dot4(a[0], b[0]);
#pragma unroll
    for (int m = 1; m < PPR; ++m) {
        acc = fmaf(a[m].x, b[m].x, acc);
        acc = fmaf(a[m].y, b[m].y, acc);
        acc = fmaf(a[m].z, b[m].z, acc);
        acc = fmaf(a[m].w, b[m].w, acc);
    }
    return acc;
}

// Lanes per state row: 16 for the 128-wide rows (two float4 pieces per lane, the
// row sums stay within a 16-lane DPP row), dk/4 (one piece per lane) otherwise.
// At 128 x 128, 16 lanes per row take 40 % of the reduction steps of 32 (4 rows
// per lane with 2 x 4 DPP steps each, against 8 rows with 2 x 5 steps, one of
// them through LDS) for 8 more VGPRs of k and q; 32 and 8 lanes spill.
#ifndef GDN_DECODE_LPR128
#define GDN_DECODE_LPR128 16
#endif
// 256-wide rows: 32 lanes (two pieces each); 64 lanes spill at 16 waves.
// 96-wide rows: 8 lanes (three pieces each), since 24 does not divide a wave.
#ifndef GDN_DECODE_LPR256
#define GDN_DECODE_LPR256 32
#endif
template <int DK, int DV>
constexpr int decode_lpr()
{
    return DK == 128 ? GDN_DECODE_LPR128 : DK == 256 ? GDN_DECODE_LPR256 : DK == 96 ? 8 : DK / 4;
}

// Token modes: MODE_ANY (one or more tokens, per-lane scalars), MODE_GROUP (fused
// layer, several tokens: the per-token scalars -- q/k norms, k.q, gates -- once per
// token of a conv group, shared through LDS), MODE_ONE (one token per sequence: no
// token loop, and each wave stores its own rows' outputs). The arithmetic is the
// same operation for operation in every mode, so a call and any split of it agree
// bit for bit.
enum { MODE_ANY = 0, MODE_GROUP = 1, MODE_ONE = 2 };

// Two 8-wave workgroups per CU (4 waves per SIMD, at most 128 VGPRs) for the shapes
// whose state share fits; the larger shapes take the registers they need. The
// one-token kernel needs about 85 VGPRs; held to 80 for a third workgroup per CU
// it spills 16-28 bytes per lane and runs 6-13 % slower.
template <int DK, int DV, int NW>
constexpr int decode_min_waves()
{
    return NW == 8 && DK * DV <= 128 * 128    ? 4
           : NW == 16 && DK * DV <= 128 * 128 ? 8  // the streamed one-token kernel, 63 VGPRs
           : NW == 6                          ? 3
                                              : 1;
}

template <int DK, int DV, int NW, int QT, int CK, int MODE, bool NT>
__global__ __launch_bounds__(NW * 64, (decode_min_waves<DK, DV, NW>())) void decode_kernel(DecodeParams p)
{
    constexpr bool GS = MODE == MODE_GROUP;
    constexpr int LPR = decode_lpr<DK, DV>();  // lanes holding one row
    constexpr int PPR = DK / (4 * LPR);        // float4 pieces of a row per lane
    constexpr int RPI = 64 / LPR;              // rows per wave-wide load
    constexpr int RPW = DV / NW;               // rows per wave
    constexpr int RPL = RPW / RPI;             // rows per lane
    constexpr int NI = RPL * PPR;              // float4 state pieces per lane
    static_assert(DK % (4 * LPR) == 0 && 64 % LPR == 0 && RPW % RPI == 0 && RPL >= 1, "shape");
    static_assert(RPW <= 64, "one v value per lane covers the wave's rows");

    __shared__ float o_s[kTokGroup][DV];
    constexpr int NCH = 2 * DK + DV;  // conv channels one workgroup reads
    static_assert(CK == 0 || NCH <= NW * 64, "one conv channel per thread");
    __shared__ float y_s[CK > 0 ? kTokGroup : 1][CK > 0 ? NCH : 1];  // conv outputs
    // per token of a conv group: 1/|k|, 1/|q|, k.q of the normalised pair, alpha, beta
    __shared__ float sc_s[GS ? kTokGroup : 1][5];
    constexpr int GT = (kTokGroup + NW - 1) / NW;  // group tokens per wave

    // One field from each 64-byte line of the kernel arguments, consumed together:
    // the four lines are fetched at once behind one wait, instead of line by line
    // as each field is first used, a memory round trip each.
    asm volatile("" ::"s"(p.in.q), "s"(p.in.decay_param), "s"(p.hc.Hv), "s"(p.T));
    const HeadCfg &hc = p.hc;
    const int Hv = hc.Hv;
    const int h = blockIdx.x % Hv;
    const int b = blockIdx.x / Hv;
    // A sentinel or out-of-range slot: the workgroup issues its loads from slot 0
    // (in bounds: the host launches nothing when there are no slots) and leaves
    // once they are issued, before any barrier or store. Leaving here instead
    // would put a wait for the slot and the kernel arguments behind the branch
    // in front of every load.
    const int slot_arg = p.slots ? p.slots[b] : b;
    const bool live = slot_arg >= 0 && slot_arg < p.num_slots;
    const int slot = live ? slot_arg : 0;
    const int kh = k_head_of(hc.head_map, h, hc.Hk, Hv);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane / LPR;
    const int col = (lane % LPR) * 4;
    const uint32_t flags = hc.flags;
    const int row0 = wave * RPW + sub;
    const int vrow = wave * RPW + (lane % RPW);  // the v element this lane fetches

    // per-head gate parameters: vector loads issued with the token's inputs (ahead
    // of the state in the in-order return queue); exp is taken where they are used
    float dparam = 0.f, dtb = 0.f;
    if (flags & F_RAW_GATES) {
        const int hz = h + vgpr_zero();
        dparam = p.in.decay_param[hz];
        dtb = p.in.dt_bias[hz];
    }

    // Token 0's activations are issued before the state: vector-memory returns
    // are counted in order, so the prologue math can run while the state is in
    // flight, and each row piece is processed as soon as it lands.
    TokenRaw<QT, PPR> tr;
    // fused layer: each wave fetches the gate words of its tokens of a conv group
    // (tokens wave, wave + NW, ...) with the group's inputs; otherwise every lane
    // fetches its token's activations
    const bool raw_g = flags & F_RAW_GATES;
    const void *gsa = raw_g ? p.in.a : static_cast<const void *>(p.in.g);
    const void *gsb = raw_g ? p.in.b : static_cast<const void *>(p.in.beta);
    const int gdt0 = raw_g ? p.in.ab_dt : DT_F32;
    GateWord gwa[GT], gwb[GT];
    auto load_group_gates = [&](int t0, int tn) {
#pragma unroll
        for (int i = 0; i < GT; ++i) {
            const int64_t r = (int64_t)b * p.T + t0 + min(wave + i * NW, tn - 1);
            const int64_t gi = r * Hv + h + vgpr_zero();
            gwa[i] = load_gate(gsa, gi, gdt0);
            gwb[i] = load_gate(gsb, gi, gdt0);
        }
    };
    if constexpr (GS)
        load_group_gates(0, min(p.T, kTokGroup));
    else
        load_token<DK, DV, QT, PPR, LPR, CK == 0>(tr, p, (int64_t)b * p.T, h, kh, col, vrow);
    // fused conv: this thread's channel (q, k or v) and its raw inputs of the first
    // token group, issued before the state loads, and its taps and window: before
    // the state too for one token per sequence (the conv then runs while the state
    // is in flight), right after it for several (the multi-token kernel has no
    // registers to spare across the state loads, nor has a 16-wave workgroup)
    constexpr bool kTapsFirst = !GS && NW <= 8;
    const int64_t nch = 2 * (int64_t)hc.Hk * DK + (int64_t)Hv * DV;
    const int cl = threadIdx.x;  // channel within the workgroup's 2 dk + dv
    int64_t cch = 0;             // its index in the conv channel order
    const void *xsrc = nullptr;
    int64_t xoff = 0, xstride = 0;
    ConvLane<QT, (CK > 0 ? CK : 2)> cvl;
    uint32_t xr[kTokGroup];
    if constexpr (CK > 0) {
        if (cl < DK) {
            cch = (int64_t)kh * DK + cl;
            xsrc = p.in.q; xoff = (int64_t)kh * DK + cl; xstride = p.in.q_stride;
        } else if (cl < 2 * DK) {
            cch = (int64_t)hc.Hk * DK + (int64_t)kh * DK + (cl - DK);
            xsrc = p.in.k; xoff = (int64_t)kh * DK + (cl - DK); xstride = p.in.k_stride;
        } else {
            cch = 2 * (int64_t)hc.Hk * DK + (int64_t)h * DV + (cl - 2 * DK);
            xsrc = p.in.v; xoff = (int64_t)h * DV + (cl - 2 * DK); xstride = p.in.v_stride;
        }
        if (cl < NCH) {
            const int tn = min(p.T, kTokGroup);
#pragma unroll
            for (int tt = 0; tt < kTokGroup; ++tt)
                if (tt < tn)
                    xr[tt] = load_raw1<QT>(xsrc, ((int64_t)b * p.T + tt) * xstride + xoff);
            if constexpr (kTapsFirst)
                cvl.load(p, cch, ((int64_t)slot * nch + cch) * (CK - 1));
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the token loads ahead of the state loads

    float *Sg = p.state + ((int64_t)slot * Hv + h) * (int64_t)(DV * DK);
    float4 S[NI];  // S[r * PPR + m]: piece m of the lane's row r
#pragma unroll
    for (int i = 0; i < NI; ++i)
        S[i] = load_state4<NT>(Sg + (row0 + (i / PPR) * RPI) * DK + col + 4 * LPR * (i % PPR));
    if constexpr (CK > 0 && !kTapsFirst) {
        if (cl < NCH)
            cvl.load(p, cch, ((int64_t)slot * nch + cch) * (CK - 1));
    }
    // the gated norm's z and weights for the first token group, behind the state:
    // the epilogue then waits on nothing (branch-free: without the norm the loads
    // read the state's first word and are not used)
    constexpr int ZT = (kTokGroup + NW - 1) / NW, ZJ = (DV + 63) / 64;
    const bool gated = flags & F_GATED_NORM;
    // One token per sequence: every wave stores the outputs of its own rows (lane
    // < RPW holds row wave RPW + lane), instead of one wave storing them all.
    constexpr bool solo = MODE == MODE_ONE;
    const int jsolo = wave * RPW + (lane % RPW);
    uint32_t zw[ZT][ZJ];
    float nw[ZJ];
    auto prefetch_z = [&](int t0, int tn) {
        const void *zsrc = gated ? p.in.z : static_cast<const void *>(p.state);
        if constexpr (solo) {
            const int64_t obase = ((int64_t)b * Hv + h) * DV;
            zw[0][0] = load_word_nb(zsrc, gated ? obase + jsolo : 0, p.in.z_dt);
            return;
        }
#pragma unroll
        for (int i = 0; i < ZT; ++i) {
            const int tt = wave + i * NW;
            const int64_t obase = (((int64_t)b * p.T + t0 + tt) * Hv + h) * DV;
#pragma unroll
            for (int m = 0; m < ZJ; ++m) {
                const int j = lane + 64 * m;
                const bool use = gated && tt < tn && j < DV;
                zw[i][m] = load_word_nb(zsrc, use ? obase + j : 0, p.in.z_dt);
            }
        }
    };
    prefetch_z(0, min(p.T, kTokGroup));
#pragma unroll
    for (int m = 0; m < ZJ; ++m) {
        const int j = solo ? jsolo : lane + 64 * m;
        nw[m] = (gated ? p.in.norm_w : p.state)[gated && j < DV ? j : 0];
    }
    __builtin_amdgcn_sched_barrier(0);  // ... and their use behind the state loads
    if (!live)
        return;  // whole workgroup, before any barrier or store
    const bool raw_gates = flags & F_RAW_GATES;

    // fused conv of tokens [t0, t0 + tn) into y_s (xr holds their raw inputs)
    auto conv_group = [&](int tn) {
        if constexpr (CK > 0) {
            if (cl < NCH) {
                for (int tt = 0; tt < tn; ++tt)
                    y_s[tt][cl] = cvl.tap(raw1_to_f32<QT>(xr[tt]));
            }
        }
    };
    auto load_group = [&](int t0, int tn) {
        if constexpr (CK > 0) {
            if (cl < NCH) {
#pragma unroll
                for (int tt = 0; tt < kTokGroup; ++tt)
                    if (tt < tn)
                        xr[tt] = load_raw1<QT>(xsrc, ((int64_t)b * p.T + t0 + tt) * xstride + xoff);
            }
            if constexpr (GS)
                load_group_gates(t0, tn);
        }
    };
    const int gdt = raw_gates ? p.in.ab_dt : DT_F32;
    // the gates of one token from its raw words
    // the gates of one token from its a and b (or g and beta) inputs; both token
    // paths decode the same element to the same float first
    auto gates = [&](float ga, float gb, float &alpha, float &beta) {
        float g;
        if (raw_gates) {
            const float dec_rate = hc.decay_kind == 0 ? -expf(dparam) : dparam;
            g = dec_rate * softplus_f(ga + dtb);
            beta = sigmoid_f(gb);
        } else {
            g = ga;
            beta = gb;
        }
        alpha = expf(g);
    };
    // The per-token scalars of one token from its convolved q and k (kk, qq: this
    // lane's four elements) and gate words: the norms scale kk and qq in place.
    auto scale_vec = [&](float4 *x, float f) {
#pragma unroll
        for (int m = 0; m < PPR; ++m) {
            x[m].x *= f; x[m].y *= f; x[m].z *= f; x[m].w *= f;
        }
    };
    auto token_scalars = [&](float4 *kk, float4 *qq, float ga, float gb, float &ik, float &iq,
                             float &kq, float &alpha, float &beta) {
        ik = 1.f;
        iq = 1.f;
        if (flags & F_L2NORM) {
            const float sk = group_sum<LPR>(dotn<PPR>(kk, kk));
            const float sq = group_sum<LPR>(dotn<PPR>(qq, qq));
            ik = rsqrtf(sk + hc.l2_eps);
            iq = rsqrtf(sq + hc.l2_eps);
            scale_vec(kk, ik);
            scale_vec(qq, iq);
        }
        gates(ga, gb, alpha, beta);
        kq = group_sum<LPR>(dotn<PPR>(kk, qq));
    };
    // GS: the scalars of a conv group's tokens, wave w taking tokens w, w + NW, ...
    // (every lane computes, lane 0 writes sc_s)
    auto group_scalars = [&](int tn) {
        if constexpr (GS) {
#pragma unroll
            for (int i = 0; i < GT; ++i) {
                const int tt = wave + i * NW;
                if (tt < tn) {
                    float4 qq[PPR], kk[PPR];
#pragma unroll
                    for (int m = 0; m < PPR; ++m) {
                        qq[m] = *reinterpret_cast<const float4 *>(&y_s[tt][col + 4 * LPR * m]);
                        kk[m] = *reinterpret_cast<const float4 *>(&y_s[tt][DK + col + 4 * LPR * m]);
                    }
                    float ik, iq, kq, alpha, beta;
                    token_scalars(kk, qq, gate_value(gwa[i], gdt), gate_value(gwb[i], gdt), ik, iq, kq,
                                  alpha, beta);
                    if (lane == 0) {
                        sc_s[tt][0] = ik;
                        sc_s[tt][1] = iq;
                        sc_s[tt][2] = kq;
                        sc_s[tt][3] = alpha;
                        sc_s[tt][4] = beta;
                    }
                }
            }
        }
    };
    if constexpr (CK > 0) {
        if (cl < NCH)
            cvl.convert();
        conv_group(min(p.T, kTokGroup));
        __syncthreads();
        if constexpr (GS) {
            group_scalars(min(p.T, kTokGroup));
            __syncthreads();
        }
    }

    // One token through this wave's rows: prologue (norms, gates), then the two
    // reductions, the update and the read-out per row piece; outputs go to
    // o_s[tt] for the group epilogue.
    auto process_token = [&](int tt, int64_t r) {
        float4 kk[PPR], qq[PPR];
        float vr[RPL];  // v of each of the lane's rows
        float alpha, beta, kq;
        if constexpr (CK > 0) {
#pragma unroll
            for (int m = 0; m < PPR; ++m) {
                qq[m] = *reinterpret_cast<const float4 *>(&y_s[tt][col + 4 * LPR * m]);
                kk[m] = *reinterpret_cast<const float4 *>(&y_s[tt][DK + col + 4 * LPR * m]);
            }
#pragma unroll
            for (int rr = 0; rr < RPL; ++rr)
                vr[rr] = y_s[tt][2 * DK + row0 + rr * RPI];
        } else {
#pragma unroll
            for (int m = 0; m < PPR; ++m) {
                kk[m] = raw4_to_f32<QT>(tr.k[m]);
                qq[m] = raw4_to_f32<QT>(tr.q[m]);
            }
            const float vv = raw1_to_f32<QT>(tr.v);  // row vrow's v, spread to the rows
#pragma unroll
            for (int rr = 0; rr < RPL; ++rr)
                vr[rr] = __shfl(vv, sub + rr * RPI, 64);
        }
        if constexpr (GS) {
            const float ik = sc_s[tt][0], iq = sc_s[tt][1];
            if (flags & F_L2NORM) {
                scale_vec(kk, ik);
                scale_vec(qq, iq);
            }
            kq = sc_s[tt][2];
            alpha = sc_s[tt][3];
            beta = sc_s[tt][4];
        } else {
            float ik, iq;
            token_scalars(kk, qq, gate_value(tr.ga, gdt), gate_value(tr.gb, gdt), ik, iq, kq, alpha, beta);
        }
#pragma unroll
        for (int rr = 0; rr < RPL; ++rr) {
            float4 *Sr = &S[rr * PPR];
            const float pk = group_sum<LPR>(dotn<PPR>(Sr, kk));
            const float pq = group_sum<LPR>(dotn<PPR>(Sr, qq));
            const float d = beta * fmaf(-alpha, pk, vr[rr]);
            const float o = hc.scale * fmaf(alpha, pq, d * kq);
#pragma unroll
            for (int m = 0; m < PPR; ++m) {
                Sr[m].x = fmaf(alpha, Sr[m].x, d * kk[m].x);
                Sr[m].y = fmaf(alpha, Sr[m].y, d * kk[m].y);
                Sr[m].z = fmaf(alpha, Sr[m].z, d * kk[m].z);
                Sr[m].w = fmaf(alpha, Sr[m].w, d * kk[m].w);
            }
            if (col == 0)
                o_s[tt][row0 + rr * RPI] = o;
        }
    };

    float zsilu = 0.f;  // solo: SiLU(z) of this lane's row, formed before the last barrier
    // Gated RMS norm (or plain copy) of the tokens [t0, t0 + tn): one wave per token.
    // (z and the norm weights come from the registers prefetch_z filled)
    auto epilogue = [&](int t0, int tn) {
        if constexpr (solo) {
            // every wave forms the same sum of squares, in the order the
            // one-wave-per-token epilogue below uses, so both agree bit for bit
            const int64_t obase = ((int64_t)b * Hv + h) * DV;
            if (gated) {
                float ss = 0.f;
                for (int j = lane; j < DV; j += 64)
                    ss = fmaf(o_s[0][j], o_s[0][j], ss);
                ss = group_sum<64>(ss);
                const float inv = rsqrtf(ss / (float)DV + hc.norm_eps);
                if (lane < RPW)
                    store_act(p.out, obase + jsolo, p.out_dt, o_s[0][jsolo] * inv * nw[0] * zsilu);
            } else if (lane < RPW) {
                store_act(p.out, obase + jsolo, p.out_dt, o_s[0][jsolo]);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < ZT; ++i) {
            const int tt = wave + i * NW;
            if (tt >= tn)
                break;
            const int64_t r = (int64_t)b * p.T + t0 + tt;
            const int64_t obase = (r * Hv + h) * DV;
            if (gated) {
                float ss = 0.f;
                for (int j = lane; j < DV; j += 64)
                    ss = fmaf(o_s[tt][j], o_s[tt][j], ss);
                ss = group_sum<64>(ss);
                const float inv = rsqrtf(ss / (float)DV + hc.norm_eps);
#pragma unroll
                for (int m = 0; m < ZJ; ++m) {
                    const int j = lane + 64 * m;
                    if (j < DV) {
                        const float zv = word_to_f32(zw[i][m], obase + j, p.in.z_dt);
                        store_act(p.out, obase + j, p.out_dt, o_s[tt][j] * inv * nw[m] * silu_f(zv));
                    }
                }
            } else {
                for (int j = lane; j < DV; j += 64)
                    store_act(p.out, obase + j, p.out_dt, o_s[tt][j]);
            }
        }
    };

    // token 0 in straight-line code, so each row piece is used as soon as it lands
    process_token(0, (int64_t)b * p.T);
    for (int t = 1; t < (solo ? 1 : p.T); ++t) {
        const int tt = t % kTokGroup;
        if (tt == 0) {  // o_s (and y_s) hold a full group: drain it, convolve the next
            load_group(t, min(p.T - t, kTokGroup));
            __syncthreads();
            epilogue(t - kTokGroup, kTokGroup);
            prefetch_z(t, min(p.T - t, kTokGroup));
            conv_group(min(p.T - t, kTokGroup));
            __syncthreads();
            if constexpr (GS) {
                group_scalars(min(p.T - t, kTokGroup));
                __syncthreads();
            }
        }
        const int64_t r = (int64_t)b * p.T + t;
        if constexpr (!GS)
            load_token<DK, DV, QT, PPR, LPR, CK == 0>(tr, p, r, h, kh, col, vrow);
        process_token(tt, r);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i)
        store_state4<NT>(Sg + (row0 + (i / PPR) * RPI) * DK + col + 4 * LPR * (i % PPR), S[i]);
    if constexpr (CK > 0) {
        // the window after this call's tokens; q/k channels from one v-head per k-head
        const bool qk_writer = hc.head_map == 0 ? (h % (Hv / hc.Hk) == 0) : (h < hc.Hk);
        if (cl < NCH && (cl >= 2 * DK || qk_writer))
            cvl.store(p, ((int64_t)slot * nch + cch) * (CK - 1));
    }
    if (solo && gated)
        zsilu = silu_f(word_to_f32(zw[0][0], ((int64_t)b * Hv + h) * DV + jsolo, p.in.z_dt));
    __syncthreads();
    const int tlast0 = ((p.T - 1) / kTokGroup) * kTokGroup;
    epilogue(tlast0, p.T - tlast0);
}

template <int DK, int DV, int NW, int CK, int MODE, bool NT>
void launch_decode_nt(const DecodeParams &p, hipStream_t s)
{
    const dim3 grid((unsigned)((int64_t)p.B * p.hc.Hv)), block(NW * 64);
    switch (p.in.qkv_dt) {
    case DT_F32: hipLaunchKernelGGL((decode_kernel<DK, DV, NW, DT_F32, CK, MODE, NT>), grid, block, 0, s, p); break;
    case DT_F16: hipLaunchKernelGGL((decode_kernel<DK, DV, NW, DT_F16, CK, MODE, NT>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((decode_kernel<DK, DV, NW, DT_BF16, CK, MODE, NT>), grid, block, 0, s, p); break;
    }
}

template <int DK, int DV, int NW, int CK>
void launch_decode_ck(const DecodeParams &p, const DecodePlan &pl, hipStream_t s)
{
    // the mode and the hint come from the plan; both are compile-time in the kernel
    if (pl.mode == MODE_ONE) {
        if (pl.nontemporal)
            launch_decode_nt<DK, DV, NW, CK, MODE_ONE, true>(p, s);
        else
            launch_decode_nt<DK, DV, NW, CK, MODE_ONE, false>(p, s);
    } else if constexpr (CK > 0) {
        if (pl.nontemporal)
            launch_decode_nt<DK, DV, NW, CK, MODE_GROUP, true>(p, s);
        else
            launch_decode_nt<DK, DV, NW, CK, MODE_GROUP, false>(p, s);
    } else {
        if (pl.nontemporal)
            launch_decode_nt<DK, DV, NW, CK, MODE_ANY, true>(p, s);
        else
            launch_decode_nt<DK, DV, NW, CK, MODE_ANY, false>(p, s);
    }
}

template <int DK, int DV, int NW>
void launch_decode_t(const DecodeParams &p, const DecodePlan &pl, hipStream_t s)
{
    if (p.conv_k == 4)
        launch_decode_ck<DK, DV, NW, 4>(p, pl, s);
    else
        launch_decode_ck<DK, DV, NW, 0>(p, pl, s);
}

}  // namespace

// Built head shapes (dk, dv) and their waves per workgroup. A row's dk floats sit
// in decode_lpr lanes (16 for dk = 128, 32 for 256, 8 for 96, dk/4 otherwise; the
// count divides 64), each wave holds at most 64 rows, and the fused layer gives
// every one of its 2 dk + dv conv channels a thread. A lane's share of the state
// must fit its registers: 16 float4 pieces at 8 waves (256 VGPRs per lane), 8 at
// 16 waves (128). dk = dv = 256 takes 16 pieces at 16 waves (768 conv channels):
// the one-token kernels fit (the fused layer spills 20 bytes per lane), the
// multi-token ones spill 200-280 bytes per lane and run slower, still correct.
bool decode_supported(int dk, int dv) { return decode_plan(dk, dv, 1, 1, 1, false, 0).waves > 0; }

// Waves per workgroup for each built shape. The 128 x 128 state takes 8 waves of 16
// rows, except streamed one-token calls (GDN_STREAM_STATE): 16 waves of 8 rows, two
// workgroups per CU at 63 VGPRs. On states past the Infinity Cache that is 4 %
// faster than 8 waves (rotating sets 49.9 -> 47.7 us, 48 layers at B=32 1.83 ->
// 1.79 ms); on cached states and at B=1 it is slower, so unhinted calls keep 8
// waves. Same arithmetic, same bits.
DecodePlan decode_plan(int dk, int dv, int B, int T, int Hv, bool fused_conv, uint32_t flags)
{
    DecodePlan pl{};
    const bool nt = (flags & F_STREAM_STATE) != 0;
    if (dk == 128 && dv == 128)
        pl.waves = nt && T == 1 ? 16 : GDN_DECODE_NW;
    else if ((dk == 64 && dv == 64) || (dk == 32 && dv == 32))
        pl.waves = 4;
    else if (dk == 96 && dv == 96)
        pl.waves = 6;
    else if ((dk == 64 && dv == 128) || (dk == 128 && dv == 64) || (dk == 128 && dv == 256))
        pl.waves = 8;
    else if ((dk == 256 && dv == 128) || (dk == 256 && dv == 256))
        pl.waves = 16;
    else
        return DecodePlan{};  // not built: waves == 0
    pl.lanes_per_row = dk == 128 ? GDN_DECODE_LPR128 : dk == 256 ? GDN_DECODE_LPR256 : dk == 96 ? 8 : dk / 4;
    pl.mode = T == 1 ? MODE_ONE : fused_conv ? MODE_GROUP : MODE_ANY;
    pl.nontemporal = nt ? 1 : 0;
    pl.workgroups = B * Hv;
    pl.threads = 64 * pl.waves;
    return pl;
}

hipError_t launch_decode(const DecodeParams &p, hipStream_t s)
{
    if (p.B == 0 || p.num_slots == 0)  // no slots: every sequence is a sentinel
        return hipSuccess;
    const int dk = p.hc.dk, dv = p.hc.dv;
    const DecodePlan pl = decode_plan(dk, dv, p.B, p.T, p.hc.Hv, p.conv_k == 4, p.hc.flags);
    if (dk == 128 && dv == 128) {
        if (pl.waves == 16) {
            // only instantiated for streamed one-token calls
            if (p.conv_k == 4)
                launch_decode_nt<128, 128, 16, 4, MODE_ONE, true>(p, s);
            else
                launch_decode_nt<128, 128, 16, 0, MODE_ONE, true>(p, s);
        } else {
            launch_decode_t<128, 128, GDN_DECODE_NW>(p, pl, s);
        }
    } else if (dk == 64 && dv == 64) {
        launch_decode_t<64, 64, 4>(p, pl, s);
    } else if (dk == 32 && dv == 32) {
        launch_decode_t<32, 32, 4>(p, pl, s);
    } else if (dk == 64 && dv == 128) {
        launch_decode_t<64, 128, 8>(p, pl, s);
    } else if (dk == 128 && dv == 64) {
        launch_decode_t<128, 64, 8>(p, pl, s);
    } else if (dk == 128 && dv == 256) {
        launch_decode_t<128, 256, 8>(p, pl, s);
    } else if (dk == 256 && dv == 128) {
        launch_decode_t<256, 128, 16>(p, pl, s);
    } else if (dk == 96 && dv == 96) {
        launch_decode_t<96, 96, 6>(p, pl, s);
    } else if (dk == 256 && dv == 256) {
        launch_decode_t<256, 256, 16>(p, pl, s);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace gdn
