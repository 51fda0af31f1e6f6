// gdn_prefill_generic.hip -- chunked prefill for the head shapes other than
// dk = dv = 128 (whose f16-operand MFMA kernels are in gdn_prefill.hip).
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
// Kernels (all arithmetic f32; every product on v_mfma_f32_16x16x4_f32):
//  1. plan_generic_kernel -- the chunk table (several sequences only; one
//     sequence's chunk bounds are closed-form).
//  2. prep_generic_kernel -- per (chunk, k-head), all chunks in parallel: the
//     normalised q and k rows, K K^T and Q K^T once, then for each v-head reading
//     the k-head: gates and their prefix sums, A, T = (I + A)^-1 in 16 x 16
//     blocks, W, U and scale * Aqk and the decay rows, all to the workspace.
//  3. carry_generic_kernel -- per (sequence, v-head, 32 rows of dv), sequential
//     over the sequence's chunks with the slice's f32 state resident in LDS: only
//     the state-dependent products (Q S^T, W S^T, Aqk D, D^T diag(e) K). The next
//     chunk's operands are loaded into registers while the current one runs.
//  4. norm_generic_kernel -- the gated RMS norm of the f32 core output.
// Chunks are 64 tokens, 32 when dk = 256 (the LDS then holds the 256-wide tiles).

#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kSlice = 32;  // dv rows per carry workgroup

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

// ---------------------------------------------------------------- workspace

struct GenWs {
    size_t chunk_seq, chunk_start, chunk_len, seq_chunk0, q, k, w, u, aq, dec, onorm, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// MC = the chunk count bound (total / chunk + N); per (chunk, k-head) the
// normalised q and k rows, per (chunk, v-head) W, U, scale * Aqk and three decay
// rows, all f32; with the gated norm an f32 core output.
GenWs gen_layout(int Hk, int Hv, int dk, int dv, int64_t MC, int N, int64_t total, bool norm)
{
    const int C = dk >= 256 ? 32 : 64;
    GenWs L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    L.chunk_seq = take(sizeof(int32_t) * MC);
    L.chunk_start = take(sizeof(int32_t) * MC);
    L.chunk_len = take(sizeof(int32_t) * MC);
    L.seq_chunk0 = take(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
    L.q = take(sizeof(float) * MC * Hk * C * dk);
    L.k = take(sizeof(float) * MC * Hk * C * dk);
    L.w = take(sizeof(float) * MC * Hv * C * dk);
    L.u = take(sizeof(float) * MC * Hv * C * dv);
    L.aq = take(sizeof(float) * MC * Hv * C * C);
    L.dec = take(sizeof(float) * MC * Hv * 3 * C);
    L.onorm = norm ? take(sizeof(float) * (size_t)total * Hv * dv) : off;
    L.total = off;
    return L;
}

// ---------------------------------------------------------------- 1. plan

// Chunk table: chunk g of the packed call is chunk k of sequence s, starting at
// token cu[s] + CC k with min(CC, len - CC k) tokens; seq_chunk0[s] = s's first.
template <int CC>
__global__ __launch_bounds__(256) void plan_generic_kernel(PrefillParams p)
{
    __shared__ int scan[256];
    __shared__ int base_s;
    if (threadIdx.x == 0)
        base_s = 0;
    __syncthreads();
    for (int i0 = 0; i0 < p.N; i0 += 256) {
        const int i = i0 + threadIdx.x;
        const int len = i < p.N ? p.cu[i + 1] - p.cu[i] : 0;
        const int nc = (len + CC - 1) / CC;
        scan[threadIdx.x] = nc;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {  // inclusive scan
            const int v = threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
            __syncthreads();
            scan[threadIdx.x] += v;
            __syncthreads();
        }
        if (i < p.N)
            p.seq_chunk0[i] = base_s + scan[threadIdx.x] - nc;
        const int tot = scan[255];
        for (int c = threadIdx.x; c < tot; c += 256) {
            int lo = 0, hi = 255;  // the first sequence whose inclusive count exceeds c
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (scan[mid] > c)
                    hi = mid;
                else
                    lo = mid + 1;
            }
            const int k = c - (lo ? scan[lo - 1] : 0);
            const int seq = i0 + lo;
            const int s0 = p.cu[seq], sl = p.cu[seq + 1] - s0;
            const int g = base_s + c;
            p.chunk_seq[g] = seq;
            p.chunk_start[g] = s0 + k * CC;
            p.chunk_len[g] = min(CC, sl - k * CC);
        }
        __syncthreads();
        if (threadIdx.x == 255)
            base_s += scan[255];
        __syncthreads();
    }
}

// ---------------------------------------------------------------- 2. prep

template <int DK, int DV>
__global__ __launch_bounds__(kThreads, 1) void prep_generic_kernel(PrefillParams p)
{
    constexpr int CC = gen_chunk<DK>();
    constexpr int KP = DK + 1, CP = CC + 1, VP = kSlice + 1;
    constexpr int NB = CC / 16;
    static_assert(DV % kSlice == 0 && CC <= 64 && CC % 16 == 0 && DK % 16 == 0, "shape");

    __shared__ float Kc[CC][KP];  // the chunk's (normalised) keys
    __shared__ float Qc[CC][KP];  // its queries
    __shared__ float Gm[CC][CP];  // K K^T
    __shared__ float Qk[CC][CP];  // Q K^T
    __shared__ float Am[CC][CP];  // A (strictly lower), per v-head
    __shared__ float Tm[CC][CP];  // T = (I + A)^-1
    __shared__ float Vs[CC][VP];  // one 32-wide slice of v
    __shared__ float Mb[NB > 1 ? NB - 1 : 1][16][16];  // block sums of the inverse
    __shared__ float G_s[CC], beta_s[CC], bg_s[CC];

    const HeadCfg &hc = p.hc;
    const ActInputs &in = p.in;
    const int Hv = hc.Hv, Hk = hc.Hk, G = Hv / Hk;
    const int chunk = blockIdx.x / Hk, kh = blockIdx.x % Hk;
    const bool one_seq = p.N == 1;  // tokens [0, total): no table
    const int64_t tok0 = one_seq ? (int64_t)CC * chunk : p.chunk_start[chunk];
    const int n = one_seq ? min(CC, p.total - CC * chunk) : p.chunk_len[chunk];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t flags = hc.flags;
    const bool raw = flags & F_RAW_GATES;
    const int qdt = in.qkv_dt;
    auto vhead = [&](int j) { return hc.head_map == 0 ? kh * G + j : kh + j * Hk; };

    // -- keys and queries: every load issued before any use, no branch around a
    // load (rows past the chunk's end re-read row n-1, columns past dk re-read
    // column dk-1, both masked after; the 32-bit word holding each element -- a
    // q/k row has an even length from a 4-element aligned start, so the word stays
    // in the row -- and the dtype by a select). Wave w takes rows w, w + 4, ...;
    // lane l columns l, l + 64, ...
    {
        constexpr int RW = CC / 4, EPL = (DK + 63) / 64;
        uint32_t kw[RW][EPL], qw[RW][EPL];
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
        float *gq = p.gq + ((int64_t)chunk * Hk + kh) * CC * DK;
        float *gk = p.gk + ((int64_t)chunk * Hk + kh) * CC * DK;
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            const int r = wave + 4 * i;
            float kv[EPL], qv[EPL];
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int m = 0; m < EPL; ++m) {
                const int c = lane + 64 * m;
                const bool ok = r < n && c < DK;
                const int64_t idx = (int64_t)min(c, DK - 1);  // the element's parity in its word
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
                    gk[r * DK + c] = kv[m] * ik;
                    gq[r * DK + c] = qv[m] * iq;
                }
            }
        }
    }
    __syncthreads();

    // -- K K^T and Q K^T, shared by the v-heads reading this k-head
    mfma_product<CC, CC, DK>([&](int t, int i) { return Kc[t][i]; }, [&](int i, int s) { return Kc[s][i]; },
                             [&](int t, int s, float v) { Gm[t][s] = v; });
    mfma_product<CC, CC, DK>([&](int t, int i) { return Qc[t][i]; }, [&](int i, int s) { return Kc[s][i]; },
                             [&](int t, int s, float v) { Qk[t][s] = v; });

    const void *gsa = raw ? in.a : static_cast<const void *>(in.g);
    const void *gsb = raw ? in.b : static_cast<const void *>(in.beta);
    const int gdt = raw ? in.ab_dt : DT_F32;
    for (int j = 0; j < G; ++j) {
        const int h = vhead(j);
        __syncthreads();  // the products are in LDS; the previous v-head is done with its buffers
        // -- gates and their in-chunk prefix sums (wave 0, lane = token); tokens
        // past the chunk's end get g = beta = 0, so they carry G_{n-1}
        float *dec = p.gdec + ((int64_t)chunk * Hv + h) * 3 * CC;
        if (wave == 0) {
            const int64_t gi = (tok0 + min(lane, n - 1)) * Hv + h;
            const GateWord ga = load_gate(gsa, gi, gdt), gb = load_gate(gsb, gi, gdt);
            float g = gate_value(ga, gdt), beta = gate_value(gb, gdt);
            if (raw) {
                const float rate = hc.decay_kind == 0 ? -expf(in.decay_param[h]) : in.decay_param[h];
                g = rate * softplus_f(g + in.dt_bias[h]);
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
                const float gam = expf(Gc);
                G_s[lane] = Gc;
                beta_s[lane] = beta;
                bg_s[lane] = beta * gam;
                dec[lane] = hc.scale * gam;         // the output's decay (scale folded in)
                dec[CC + lane] = expf(Glast - Gc);  // the state update's decay
                dec[2 * CC + lane] = gam;           // gamma_t (gamma_last at CC - 1)
            }
        }
        __syncthreads();
        // -- A and scale * Aqk (to the workspace)
        float *aq = p.gaq + ((int64_t)chunk * Hv + h) * CC * CC;
        for (int e = tid; e < CC * CC; e += kThreads) {
            const int t = e / CC, s = e % CC;
            const float dg = s <= t ? expf(G_s[t] - G_s[s]) : 0.f;
            Am[t][s] = s < t ? beta_s[t] * dg * Gm[t][s] : 0.f;
            aq[e] = hc.scale * dg * Qk[t][s];
        }
        __syncthreads();
        // -- T = (I + A)^-1 (unit lower triangular), in 16 x 16 blocks. (a) Each
        // diagonal block by forward substitution in registers, one column per
        // thread, which also zeroes its column above the block.
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
        // T_ij = -T_ii (sum_{k=j}^{i-1} A_ik T_kj)
        for (int L = 1; L < NB; ++L) {
            for (int e = tid; e < (NB - L) * 256; e += kThreads) {
                const int jb = e >> 8, i = jb + L, r = (e >> 4) & 15, c = e & 15;
                float acc = 0.f;
                for (int kb = jb; kb < i; ++kb) {
                    float part = 0.f;  // one 16-long block: loads issued together
#pragma unroll
                    for (int s2 = 0; s2 < 16; ++s2)
                        part = fmaf(Am[16 * i + r][16 * kb + s2], Tm[16 * kb + s2][16 * jb + c], part);
                    acc += part;
                }
                Mb[jb][r][c] = acc;
            }
            __syncthreads();
            for (int e = tid; e < (NB - L) * 256; e += kThreads) {
                const int jb = e >> 8, i = jb + L, r = (e >> 4) & 15, c = e & 15;
                float acc = 0.f;
#pragma unroll
                for (int s2 = 0; s2 < 16; ++s2)
                    acc = fmaf(Tm[16 * i + r][16 * i + s2], Mb[jb][s2][c], acc);
                Tm[16 * i + r][16 * jb + c] = -acc;
            }
            __syncthreads();
        }
        // -- W = T diag(beta gamma) K (to the workspace)
        float *wg = p.gw + ((int64_t)chunk * Hv + h) * CC * DK;
        mfma_product<CC, DK, CC>([&](int t, int s) { return Tm[t][s] * bg_s[s]; },
                                 [&](int s, int i) { return Kc[s][i]; },
                                 [&](int t, int i, float v) { wg[t * DK + i] = v; });
        // -- U = T diag(beta) V (to the workspace), 32 columns of v at a time
        float *ug = p.gu + ((int64_t)chunk * Hv + h) * CC * DV;
        for (int d0 = 0; d0 < DV; d0 += kSlice) {
            constexpr int VPT = CC * kSlice / kThreads;
            uint32_t vw[VPT];
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int e = tid + kThreads * i;
                const int64_t row = tok0 + min(e / kSlice, n - 1);
                vw[i] = load_word_nb(in.v, row * in.v_stride + (int64_t)h * DV + d0 + e % kSlice, qdt);
            }
            __syncthreads();  // the previous slice's product is done with Vs
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int e = tid + kThreads * i, r = e / kSlice, jj = e % kSlice;
                Vs[r][jj] = r < n ? word_to_f32(vw[i], jj, qdt) : 0.f;
            }
            __syncthreads();
            mfma_product<CC, kSlice, CC>([&](int t, int s) { return Tm[t][s] * beta_s[s]; },
                                         [&](int s, int jj) { return Vs[s][jj]; },
                                         [&](int t, int jj, float v) { ug[t * DV + d0 + jj] = v; });
        }
    }
}

// ---------------------------------------------------------------- 3. carry

template <int DK, int DV>
__global__ __launch_bounds__(kThreads, 1) void carry_generic_kernel(PrefillParams p)
{
    constexpr int CC = gen_chunk<DK>();
    constexpr int KP = DK + 1, CP = CC + 1, VP = kSlice + 1;
    constexpr int NSL = DV / kSlice;
    // per thread: the words of one chunk's operands it moves into LDS
    constexpr int WQK = CC * DK / kThreads, WU = CC * kSlice / kThreads, WA = CC * CC / kThreads;
    static_assert(CC * DK % kThreads == 0 && CC * kSlice % kThreads == 0 && CC * CC % kThreads == 0 &&
                      3 * CC <= kThreads, "operand split");

    __shared__ float Ss[kSlice][KP];  // the state slice S[dv0 + j][i]
    __shared__ float Qn[CC][KP];      // normalised q rows
    __shared__ float Kn[CC][KP];      // normalised k rows
    __shared__ float Wm[CC][KP];      // W
    __shared__ float Us[CC][VP];      // U of the slice, then D
    __shared__ float Aq[CC][CP];      // scale * Aqk
    __shared__ float Qs[CC][VP];      // Q S^T
    __shared__ float Dc[3][CC];       // scale gamma_t, exp(G_last - G_t), gamma_t

    const HeadCfg &hc = p.hc;
    const int Hv = hc.Hv, Hk = hc.Hk;
    const int slice = blockIdx.x % NSL;
    const int h = (blockIdx.x / NSL) % Hv;
    const int seq = blockIdx.x / (NSL * Hv);
    const int kh = k_head_of(hc.head_map, h, Hk, Hv);
    const int dv0 = slice * kSlice;
    const bool one_seq = p.N == 1;
    const int start = one_seq ? 0 : p.cu[seq];
    const int len = one_seq ? p.total : p.cu[seq + 1] - start;
    if (len <= 0)
        return;  // empty sequence: state untouched
    const int nch = (len + CC - 1) / CC;
    const int cfirst = one_seq ? 0 : p.seq_chunk0[seq];
    const int tid = threadIdx.x;
    const uint32_t flags = hc.flags;
    float *Sg = p.state + (((int64_t)seq * Hv + h) * DV + dv0) * DK;

    for (int e = tid; e < kSlice * DK; e += kThreads)
        Ss[e / DK][e % DK] = Sg[e];

    // the operands of one chunk, as registers: element tid + 256 i of each array
    float rq[WQK], rk[WQK], rw[WQK], ru[WU], ra[WA], rd;
    auto fetch = [&](int ci) {
        const int64_t c = cfirst + ci;
        const float *gq = p.gq + (c * Hk + kh) * CC * DK, *gk = p.gk + (c * Hk + kh) * CC * DK;
        const float *gw = p.gw + (c * Hv + h) * CC * DK;
        const float *gu = p.gu + (c * Hv + h) * CC * DV + dv0;
        const float *ga = p.gaq + (c * Hv + h) * CC * CC, *gd = p.gdec + (c * Hv + h) * 3 * CC;
#pragma unroll
        for (int i = 0; i < WQK; ++i) {
            rq[i] = gq[tid + kThreads * i];
            rk[i] = gk[tid + kThreads * i];
            rw[i] = gw[tid + kThreads * i];
        }
#pragma unroll
        for (int i = 0; i < WU; ++i) {
            const int e = tid + kThreads * i;
            ru[i] = gu[(e / kSlice) * DV + e % kSlice];
        }
#pragma unroll
        for (int i = 0; i < WA; ++i)
            ra[i] = ga[tid + kThreads * i];
        rd = gd[min(tid, 3 * CC - 1)];
    };
    fetch(0);

    for (int ci = 0; ci < nch; ++ci) {
        const int n = min(CC, len - ci * CC);
        const int64_t tok0 = start + (int64_t)ci * CC;
        __syncthreads();  // the previous chunk is done with every buffer
#pragma unroll
        for (int i = 0; i < WQK; ++i) {
            const int e = tid + kThreads * i;
            Qn[e / DK][e % DK] = rq[i];
            Kn[e / DK][e % DK] = rk[i];
            Wm[e / DK][e % DK] = rw[i];
        }
#pragma unroll
        for (int i = 0; i < WU; ++i) {
            const int e = tid + kThreads * i;
            Us[e / kSlice][e % kSlice] = ru[i];
        }
#pragma unroll
        for (int i = 0; i < WA; ++i) {
            const int e = tid + kThreads * i;
            Aq[e / CC][e % CC] = ra[i];
        }
        if (tid < 3 * CC)
            Dc[tid / CC][tid % CC] = rd;
        if (ci + 1 < nch)
            fetch(ci + 1);  // the next chunk's operands, in flight from here
        __syncthreads();

        // -- Q S^T and D = U - W S^T, both on the entering state
        mfma_product<CC, kSlice, DK>([&](int t, int i) { return Qn[t][i]; }, [&](int i, int j) { return Ss[j][i]; },
                                     [&](int t, int j, float v) { Qs[t][j] = v; });
        mfma_product<CC, kSlice, DK>([&](int t, int i) { return Wm[t][i]; }, [&](int i, int j) { return Ss[j][i]; },
                                     [&](int t, int j, float v) { Us[t][j] -= v; });
        __syncthreads();

        // -- O = scale gamma Q S^T + (scale Aqk) D to the output, and the state
        // update S <- gamma_last S + D^T diag(e) K (separate buffers: no barrier)
        {
            void *obase = (flags & F_GATED_NORM) ? static_cast<void *>(p.onorm) : p.out;
            const int odt = (flags & F_GATED_NORM) ? DT_F32 : p.out_dt;
            mfma_product<CC, kSlice, CC>([&](int t, int s) { return Aq[t][s]; },
                                         [&](int s, int j) { return Us[s][j]; },
                                         [&](int t, int j, float v) {
                                             if (t < n)
                                                 store_act(obase, ((tok0 + t) * Hv + h) * DV + dv0 + j, odt,
                                                           fmaf(Dc[0][t], Qs[t][j], v));
                                         });
            const float gl = Dc[2][CC - 1];
            mfma_product<kSlice, DK, CC>([&](int j, int t) { return Us[t][j] * Dc[1][t]; },
                                         [&](int t, int i) { return Kn[t][i]; },
                                         [&](int j, int i, float v) { Ss[j][i] = fmaf(gl, Ss[j][i], v); });
        }
    }
    __syncthreads();
    for (int e = tid; e < kSlice * DK; e += kThreads)
        Sg[e] = Ss[e / DK][e % DK];
}

// ---------------------------------------------------------------- 4. gated norm

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
    if (p.N > 1)
        hipLaunchKernelGGL((plan_generic_kernel<gen_chunk<DK>()>), dim3(1), dim3(256), 0, s, p);
    hipLaunchKernelGGL((prep_generic_kernel<DK, DV>), dim3((unsigned)((int64_t)p.num_chunks * p.hc.Hk)),
                       dim3(kThreads), 0, s, p);
    hipLaunchKernelGGL((carry_generic_kernel<DK, DV>), dim3((unsigned)((int64_t)p.N * p.hc.Hv * (DV / kSlice))),
                       dim3(kThreads), 0, s, p);
    if (p.hc.flags & F_GATED_NORM) {
        const int64_t rows = (int64_t)p.total * p.hc.Hv;
        hipLaunchKernelGGL((norm_generic_kernel<DV>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace

// The head shapes of the f32 path: those the decode is built for, except 128 x
// 128, which has the f16-operand MFMA kernels.
bool prefill_generic_supported(int dk, int dv)
{
    return (dk == 32 && dv == 32) || (dk == 64 && dv == 64) || (dk == 96 && dv == 96) ||
           (dk == 64 && dv == 128) || (dk == 128 && dv == 64) || (dk == 128 && dv == 256) ||
           (dk == 256 && dv == 128) || (dk == 256 && dv == 256);
}

int prefill_generic_chunk(int dk) { return dk >= 256 ? 32 : 64; }

size_t prefill_generic_workspace_bytes(int Hk, int Hv, int dk, int dv, int64_t max_chunks, int N,
                                       int64_t total_tokens, bool norm)
{
    return gen_layout(Hk, Hv, dk, dv, max_chunks, N, total_tokens, norm).total;
}

void prefill_generic_carve(PrefillParams &p, void *ws, int64_t max_chunks)
{
    const GenWs L = gen_layout(p.hc.Hk, p.hc.Hv, p.hc.dk, p.hc.dv, max_chunks, p.N, p.total,
                               (p.hc.flags & F_GATED_NORM) != 0);
    unsigned char *b = static_cast<unsigned char *>(ws);
    p.chunk_seq = reinterpret_cast<int32_t *>(b + L.chunk_seq);
    p.chunk_start = reinterpret_cast<int32_t *>(b + L.chunk_start);
    p.chunk_len = reinterpret_cast<int32_t *>(b + L.chunk_len);
    p.seq_chunk0 = reinterpret_cast<int32_t *>(b + L.seq_chunk0);
    p.gq = reinterpret_cast<float *>(b + L.q);
    p.gk = reinterpret_cast<float *>(b + L.k);
    p.gw = reinterpret_cast<float *>(b + L.w);
    p.gu = reinterpret_cast<float *>(b + L.u);
    p.gaq = reinterpret_cast<float *>(b + L.aq);
    p.gdec = reinterpret_cast<float *>(b + L.dec);
    p.onorm = reinterpret_cast<float *>(b + L.onorm);
}

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
