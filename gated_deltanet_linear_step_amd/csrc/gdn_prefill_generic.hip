// gdn_prefill_generic.hip -- chunked prefill for the head shapes other than
// dk = dv = 128 (whose MFMA kernels are in gdn_prefill.hip).
//
// The same chunk algebra (derived from the recurrence; the ferrox-core 0.24.0
// gdn.rs page states that the chunked prefill is the recurrence summed in
// another order, and the ferrum-kernels 0.8.0 tests page checks a 64-token
// chunked core against the token-by-token reference at (Hk, Hv, dk, dv) =
// (2, 4, 32, 32), `chunked_c64_matches_recurrent_oracle_and_non_aligned_state_
// continuity`). Per chunk of n tokens of one v-head with entering state S:
//     A   = strictly-lower(beta_t exp(G_t - G_s) k_t . k_s),  T = (I + A)^-1
//     W   = T diag(beta gamma) K,   U = T diag(beta) V,   D = U - W S^T
//     O   = scale (diag(gamma) Q S^T + Aqk D),  Aqk = lower-incl(exp(G_t - G_s) q_t . k_s)
//     S  <- gamma_last S + D^T diag(exp(G_last - G_t)) K
//
// Design: one workgroup of 256 threads per (sequence, v-head, 32-row slice of
// dv), sequential over the sequence's chunks, with the slice's f32 state resident
// in LDS for the whole call. Every product runs on f32 MFMA (16 x 16 x 4), its
// operands read from LDS rows padded to an odd length; the next chunk's inputs
// are loaded into registers while the current one is computed. No workspace except the f32 core
// output the gated norm reads. Chunks are 64 tokens, 32 when dk = 256 (the LDS
// holds the chunk's K and Q/W rows and the state slice: 125-159 KB).

#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kSlice = 32;  // dv rows per workgroup

template <int DK>
constexpr int gen_chunk()
{
    return DK >= 256 ? 32 : 64;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// C[m][n] = sum_k a(m, k) b(k, n) for m < M, n < N on v_mfma_f32_16x16x4_f32 (f32
// operands, f32 accumulation). The 16 x 16 output tiles are dealt to the 4 waves,
// two at a time so that consecutive products go to different accumulators; lane
// (li, lg) = (lane % 16, lane / 16) feeds a(m0 + li, k0 + lg) and b(k0 + lg,
// n0 + li) and receives C[m0 + 4 lg + r][n0 + li] in acc[r], handed to
// c(m, n, value).
template <int M, int N, int K, class FA, class FB, class FC>
__device__ __forceinline__ void mfma_product(FA a, FB b, FC c)
{
    constexpr int TN = N / 16, NT = (M / 16) * TN;
    static_assert(M % 16 == 0 && N % 16 == 0 && K % 4 == 0, "16 x 16 x 4 tiles");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    for (int t = wave; t < NT; t += 8) {
        const int t2 = t + 4 < NT ? t + 4 : t;  // a second tile, or the first again
        const int m0 = (t / TN) * 16, n0 = (t % TN) * 16, m1 = (t2 / TN) * 16, n1 = (t2 % TN) * 16;
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int k0 = 0; k0 < K; k0 += 4) {
            acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a(m0 + li, k0 + lg), b(k0 + lg, n0 + li), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a(m1 + li, k0 + lg), b(k0 + lg, n1 + li), acc1, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            c(m0 + 4 * lg + r, n0 + li, acc0[r]);
        if (t2 != t) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                c(m1 + 4 * lg + r, n1 + li, acc1[r]);
        }
    }
}

template <int DK, int DV>
__global__ __launch_bounds__(kThreads, 1) void prefill_generic_kernel(PrefillParams p)
{
    constexpr int CC = gen_chunk<DK>();
    constexpr int KP = DK + 1, CP = CC + 1, VP = kSlice + 1;
    constexpr int NSL = DV / kSlice;
    static_assert(DV % kSlice == 0 && CC <= 64 && CC % 16 == 0 && DK % 16 == 0, "shape");

    __shared__ float Kc[CC][KP];      // the chunk's (normalised) keys
    __shared__ float Qc[CC][KP];      // its queries, then W
    __shared__ float Ss[kSlice][KP];  // the state slice S[dv0 + j][i]
    __shared__ float Am[CC][CP];      // A (strictly lower)
    __shared__ float Tm[CC][CP];      // T = (I + A)^-1
    __shared__ float Aq[CC][CP];      // Aqk (lower, diagonal included)
    __shared__ float Vs[CC][VP];      // v rows of the slice
    __shared__ float Us[CC][VP];      // U, then D
    __shared__ float Qs[CC][VP];      // Q S^T
    __shared__ float G_s[CC], beta_s[CC], gam_s[CC], bg_s[CC], ev_s[CC];

    const HeadCfg &hc = p.hc;
    const ActInputs &in = p.in;
    const int Hv = hc.Hv;
    const int slice = blockIdx.x % NSL;
    const int h = (blockIdx.x / NSL) % Hv;
    const int seq = blockIdx.x / (NSL * Hv);
    const int kh = k_head_of(hc.head_map, h, hc.Hk, Hv);
    const int dv0 = slice * kSlice;
    const int start = p.cu[seq], len = p.cu[seq + 1] - start;
    if (len <= 0)
        return;  // empty sequence: state untouched
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t flags = hc.flags;
    const bool raw = flags & F_RAW_GATES;
    float *Sg = p.state + (((int64_t)seq * Hv + h) * DV + dv0) * DK;

    for (int e = tid; e < kSlice * DK; e += kThreads)
        Ss[e / DK][e % DK] = Sg[e];

    // -- a chunk's inputs as raw words, every load issued before any is used and
    // no branch around a load: addresses are clamped into the chunk (rows past its
    // end re-read row n-1, columns past dk re-read column dk-1) and the values
    // masked where they are used; each element comes as the 32-bit word holding it
    // (a q/k/v row has an even length from a 4-element aligned start, so the word
    // stays in the row) and the dtype is a select. Wave w takes rows w, w + 4, ...;
    // lane l holds columns l, l + 64, ...; wave 0's lane t holds token t's gates.
    // The next chunk's words are requested as soon as the current ones are in LDS,
    // so their round trip overlaps the current chunk's products.
    constexpr int RW = CC / 4, EPL = (DK + 63) / 64, VPT = CC * kSlice / kThreads;
    const int qdt = in.qkv_dt;
    uint32_t kw[RW][EPL], qw[RW][EPL], vw[VPT];
    const void *gsa = raw ? in.a : static_cast<const void *>(in.g);
    const void *gsb = raw ? in.b : static_cast<const void *>(in.beta);
    const int gdt = raw ? in.ab_dt : DT_F32;
    GateWord ga, gb;
    const float dparam = raw ? in.decay_param[h] : 0.f, dtb = raw ? in.dt_bias[h] : 0.f;
    auto issue = [&](int c0) {
        const int n = min(CC, len - c0);
        const int64_t tok0 = start + c0;
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            const int64_t row = tok0 + min(wave + 4 * i, n - 1);
#pragma unroll
            for (int m = 0; m < EPL; ++m) {
                const int c = min(lane + 64 * m, DK - 1);
                kw[i][m] = load_word_nb(in.k, row * in.k_stride + (int64_t)kh * DK + c, qdt);
                qw[i][m] = load_word_nb(in.q, row * in.q_stride + (int64_t)kh * DK + c, qdt);
            }
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int e = tid + kThreads * i;
            const int64_t row = tok0 + min(e / kSlice, n - 1);
            vw[i] = load_word_nb(in.v, row * in.v_stride + (int64_t)h * DV + dv0 + e % kSlice, qdt);
        }
        const int64_t gi = (tok0 + min(lane, n - 1)) * Hv + h;
        ga = load_gate(gsa, gi, gdt);
        gb = load_gate(gsb, gi, gdt);
    };
    issue(0);

    for (int c0 = 0; c0 < len; c0 += CC) {
        const int n = min(CC, len - c0);
        const int64_t tok0 = start + c0;
        __syncthreads();  // the previous chunk is done with every buffer

#pragma unroll
        for (int i = 0; i < RW; ++i) {
            const int r = wave + 4 * i;
            float kv[EPL], qv[EPL];
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int m = 0; m < EPL; ++m) {
                const int c = lane + 64 * m;
                const bool ok = r < n && c < DK;
                const int64_t idx = (int64_t)min(c, DK - 1);  // parity of the element in its word
                kv[m] = ok ? word_to_f32(kw[i][m], idx, qdt) : 0.f;
                qv[m] = ok ? word_to_f32(qw[i][m], idx, qdt) : 0.f;
                sk = fmaf(kv[m], kv[m], sk);
                sq = fmaf(qv[m], qv[m], sq);
            }
            float ik = 1.f, iq = 1.f;
            if (flags & F_L2NORM) {
                ik = rsqrtf(group_sum<64>(sk) + hc.l2_eps);
                iq = rsqrtf(group_sum<64>(sq) + hc.l2_eps);
            }
#pragma unroll
            for (int m = 0; m < EPL; ++m) {
                const int c = lane + 64 * m;
                if (c < DK) {
                    Kc[r][c] = kv[m] * ik;
                    Qc[r][c] = qv[m] * iq;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int e = tid + kThreads * i, r = e / kSlice, j = e % kSlice;
            Vs[r][j] = r < n ? word_to_f32(vw[i], j, qdt) : 0.f;
        }
        // -- gates and their in-chunk prefix sums (wave 0, lane = token); tokens
        // past the chunk's end get g = beta = 0, so they carry G_{n-1}
        float g = gate_value(ga, gdt), beta = gate_value(gb, gdt);
        if (c0 + CC < len)
            issue(c0 + CC);  // the next chunk's words, in flight from here
        if (wave == 0) {
            if (raw) {
                const float rate = hc.decay_kind == 0 ? -expf(dparam) : dparam;
                g = rate * softplus_f(g + dtb);
                beta = sigmoid_f(beta);
            }
            if (lane >= n)
                g = beta = 0.f;
            float Gc = g;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_up(Gc, off, 64);
                if (lane >= off)
                    Gc += o;
            }
            const float Glast = __shfl(Gc, CC - 1, 64);
            if (lane < CC) {
                G_s[lane] = Gc;
                beta_s[lane] = beta;
                gam_s[lane] = expf(Gc);
                bg_s[lane] = beta * expf(Gc);
                ev_s[lane] = expf(Glast - Gc);
            }
        }
        __syncthreads();

        // -- A, Aqk and Q S^T (the entering state)
        mfma_product<CC, CC, DK>([&](int t, int i) { return Kc[t][i]; }, [&](int i, int s) { return Kc[s][i]; },
                                 [&](int t, int s, float v) {
                                     Am[t][s] = s < t ? beta_s[t] * expf(G_s[t] - G_s[s]) * v : 0.f;
                                 });
        mfma_product<CC, CC, DK>([&](int t, int i) { return Qc[t][i]; }, [&](int i, int s) { return Kc[s][i]; },
                                 [&](int t, int s, float v) { Aq[t][s] = s <= t ? expf(G_s[t] - G_s[s]) * v : 0.f; });
        mfma_product<CC, kSlice, DK>([&](int t, int i) { return Qc[t][i]; },
                                     [&](int i, int j) { return Ss[j][i]; },
                                     [&](int t, int j, float v) { Qs[t][j] = v; });
        __syncthreads();

        // -- T = (I + A)^-1 (unit lower triangular), in 16 x 16 blocks. (a) Each
        // diagonal block by forward substitution in registers, one column per
        // thread; the thread also zeroes its column above the block.
        constexpr int NB = CC / 16;
        if (tid < CC) {
            const int b0 = (tid >> 4) * 16, c = tid & 15;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int s2 = 0; s2 < r; ++s2)
                    acc = fmaf(Am[b0 + r][b0 + s2], x[s2], acc);
                x[r] = r < c ? 0.f : (r == c ? 1.f : -acc);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r)
                Tm[b0 + r][b0 + c] = x[r];
            for (int r = 0; r < b0; ++r)
                Tm[r][b0 + c] = 0.f;
        }
        __syncthreads();
        // (b) the blocks below the diagonal, one sub-diagonal after another:
        // T_ij = -T_ii (sum_{k=j}^{i-1} A_ik T_kj); the sums go through Us, which
        // is free until U is formed
        float(*Mb)[16][16] = reinterpret_cast<float(*)[16][16]>(&Us[0][0]);
        static_assert(sizeof(Us) >= sizeof(float) * 256 * (NB > 1 ? NB - 1 : 1), "block sums fit in Us");
        for (int L = 1; L < NB; ++L) {
            for (int e = tid; e < (NB - L) * 256; e += kThreads) {
                const int j = e >> 8, i = j + L, r = (e >> 4) & 15, c = e & 15;
                float acc = 0.f;
                for (int kb = j; kb < i; ++kb) {
                    float part = 0.f;  // one 16-long block: loads issued together
#pragma unroll
                    for (int s2 = 0; s2 < 16; ++s2)
                        part = fmaf(Am[16 * i + r][16 * kb + s2], Tm[16 * kb + s2][16 * j + c], part);
                    acc += part;
                }
                Mb[j][r][c] = acc;
            }
            __syncthreads();
            for (int e = tid; e < (NB - L) * 256; e += kThreads) {
                const int j = e >> 8, i = j + L, r = (e >> 4) & 15, c = e & 15;
                float acc = 0.f;
#pragma unroll
                for (int s2 = 0; s2 < 16; ++s2)
                    acc = fmaf(Tm[16 * i + r][16 * i + s2], Mb[j][s2][c], acc);
                Tm[16 * i + r][16 * j + c] = -acc;
            }
            __syncthreads();
        }

        // -- W = T diag(beta gamma) K (into Qc) and U = T diag(beta) V
        mfma_product<CC, DK, CC>([&](int t, int s) { return Tm[t][s] * bg_s[s]; },
                                 [&](int s, int i) { return Kc[s][i]; },
                                 [&](int t, int i, float v) { Qc[t][i] = v; });
        mfma_product<CC, kSlice, CC>([&](int t, int s) { return Tm[t][s] * beta_s[s]; },
                                     [&](int s, int j) { return Vs[s][j]; },
                                     [&](int t, int j, float v) { Us[t][j] = v; });
        __syncthreads();

        // -- D = U - W S^T (in place)
        mfma_product<CC, kSlice, DK>([&](int t, int i) { return Qc[t][i]; },
                                     [&](int i, int j) { return Ss[j][i]; },
                                     [&](int t, int j, float v) { Us[t][j] -= v; });
        __syncthreads();

        // -- O = scale (gamma Q S^T + Aqk D) to the output, and the state update
        // S <- gamma_last S + D^T diag(e) K (different buffers: no barrier between)
        {
            void *obase = (flags & F_GATED_NORM) ? static_cast<void *>(p.onorm) : p.out;
            const int odt = (flags & F_GATED_NORM) ? DT_F32 : p.out_dt;
            mfma_product<CC, kSlice, CC>([&](int t, int s) { return Aq[t][s]; },
                                         [&](int s, int j) { return Us[s][j]; },
                                         [&](int t, int j, float v) {
                                             if (t < n)
                                                 store_act(obase, ((tok0 + t) * Hv + h) * DV + dv0 + j, odt,
                                                           hc.scale * fmaf(gam_s[t], Qs[t][j], v));
                                         });
            const float gl = gam_s[CC - 1];
            mfma_product<kSlice, DK, CC>([&](int j, int t) { return Us[t][j] * ev_s[t]; },
                                         [&](int t, int i) { return Kc[t][i]; },
                                         [&](int j, int i, float v) { Ss[j][i] = fmaf(gl, Ss[j][i], v); });
        }
    }
    __syncthreads();
    for (int e = tid; e < kSlice * DK; e += kThreads)
        Sg[e] = Ss[e / DK][e % DK];
}

// Gated RMS norm of the f32 core output, one wave per (token, v-head) row.
template <int DV>
__global__ __launch_bounds__(256) void norm_generic_kernel(PrefillParams p)
{
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (int64_t)p.total * p.hc.Hv)
        return;
    const int lane = threadIdx.x & 63;
    constexpr int NJ = (DV + 63) / 64;
    const float *o = p.onorm + row * DV;
    float ov[NJ];
    float ss = 0.f;
#pragma unroll
    for (int m = 0; m < NJ; ++m) {
        const int j = lane + 64 * m;
        ov[m] = j < DV ? o[j] : 0.f;
        ss = fmaf(ov[m], ov[m], ss);
    }
    const float inv = rsqrtf(group_sum<64>(ss) / (float)DV + p.hc.norm_eps);
#pragma unroll
    for (int m = 0; m < NJ; ++m) {
        const int j = lane + 64 * m;
        if (j < DV)
            store_act(p.out, row * DV + j, p.out_dt,
                      ov[m] * inv * p.in.norm_w[j] * silu_f(load_act(p.in.z, row * DV + j, p.in.z_dt)));
    }
}

template <int DK, int DV>
hipError_t launch_generic(const PrefillParams &p, hipStream_t s)
{
    const dim3 grid((unsigned)((int64_t)p.N * p.hc.Hv * (DV / kSlice)));
    hipLaunchKernelGGL((prefill_generic_kernel<DK, DV>), grid, dim3(kThreads), 0, s, p);
    if (p.hc.flags & F_GATED_NORM) {
        const int64_t rows = (int64_t)p.total * p.hc.Hv;
        hipLaunchKernelGGL((norm_generic_kernel<DV>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace

// The head shapes of the one-kernel path: those the decode is built for, except
// 128 x 128, which has the MFMA kernels.
bool prefill_generic_supported(int dk, int dv)
{
    return (dk == 32 && dv == 32) || (dk == 64 && dv == 64) || (dk == 96 && dv == 96) ||
           (dk == 64 && dv == 128) || (dk == 128 && dv == 64) || (dk == 128 && dv == 256) ||
           (dk == 256 && dv == 128) || (dk == 256 && dv == 256);
}

int prefill_generic_chunk(int dk) { return dk >= 256 ? 32 : 64; }

hipError_t launch_prefill_generic(const PrefillParams &p, hipStream_t s)
{
    const int dk = p.hc.dk, dv = p.hc.dv;
    if (dk == 32 && dv == 32)
        return launch_generic<32, 32>(p, s);
    if (dk == 64 && dv == 64)
        return launch_generic<64, 64>(p, s);
    if (dk == 96 && dv == 96)
        return launch_generic<96, 96>(p, s);
    if (dk == 64 && dv == 128)
        return launch_generic<64, 128>(p, s);
    if (dk == 128 && dv == 64)
        return launch_generic<128, 64>(p, s);
    if (dk == 128 && dv == 256)
        return launch_generic<128, 256>(p, s);
    if (dk == 256 && dv == 128)
        return launch_generic<256, 128>(p, s);
    if (dk == 256 && dv == 256)
        return launch_generic<256, 256>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace gdn
