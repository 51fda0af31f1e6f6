// gdn_prefill.hip -- chunked prefill of the gated delta rule on gfx950 (MFMA).
//
// The recurrence of the decode step, summed chunk by chunk: the ferrox-core
// 0.24.0 gdn.rs page states that the chunked prefill is the same recurrence in
// another summation order, and the ferrum-kernels 0.8.0 tests page checks a
// 64-token chunked core against the token-by-token reference
// (`chunked_c64_matches_recurrent_oracle_and_non_aligned_state_continuity`).
// The chunk algebra below is derived from the recurrence itself.
//
// Within one chunk of n <= 64 tokens of one v-head, with entering state S0
// (dv x dk), G_t = g_0 + ... + g_t, gamma_t = exp(G_t):
//     S_t = gamma_t S0 + sum_{s<=t} exp(G_t - G_s) d_s k_s^T             (unrolled rule)
//     d_t + sum_{s<t} A_ts d_s = beta_t v_t - beta_t gamma_t S0 k_t,
//         A_ts = beta_t exp(G_t - G_s) (k_t . k_s)   for s < t
// so with T = (I + A)^-1, U = T diag(beta) V, W = T diag(beta gamma) K:
//     D   = U - W S0^T                                (rows d_t)
//     O   = scale (diag(gamma) Q S0^T + Aqk D),  Aqk_ts = exp(G_t - G_s)(q_t . k_s), s <= t
//     S_n = gamma_{n-1} S0 + D^T diag(exp(G_{n-1} - G_t)) K
//
// Kernels:
//  1. plan_kernel   -- chunk table: 64-token chunks from each sequence's first
//                      token (the last may be short; none straddles sequences).
//  2. prep_kernel   -- per (chunk, v-head), all chunks in parallel: q/k L2 norm,
//                      gates and their in-chunk prefix sums, the gram K K^T and
//                      Q K^T (f16 MFMA), T = (I + A)^-1 in f32 (16x16 diagonal
//                      blocks by substitution, off-diagonal blocks by f32 MFMA
//                      block products), then U and W (f16 MFMA). Writes U (f32),
//                      W, Aqk, the normalised Q and K^T (f16) and G to the workspace.
//  3. carry_kernel  -- per (sequence, v-head, 16-row slice of dv), sequential
//                      over the sequence's chunks: the state slice stays in MFMA
//                      accumulators (f32) with an f16 copy in LDS as an operand;
//                      D, O and the next state per chunk on f16 MFMA with f32
//                      accumulation. D enters the state update as an f16 hi+lo
//                      pair. The next chunk's operands are prefetched into VGPRs
//                      while the current chunk is computed.
//  4. norm_kernel   -- gated RMS norm of the f32 core output (optional).

#include "gdn_device.h"
#include "gdn_kernels.h"

namespace gdn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;     // 64 tokens per chunk
constexpr int DH = 128;       // head dim (dk = dv) of the built prefill
constexpr int KP = DH + 8;    // padded f16 row (272 B): conflict-free 16-B MFMA operand reads
constexpr int TP = C + 8;     // padded f16 row of a transposed [dim][token] tile (144 B)
constexpr int AP = C + 4;     // padded f32 row of the 64x64 A / T matrix
constexpr int DT = 16;        // dv rows per carry workgroup

__device__ __forceinline__ f32x4 mfma16(half8 a, half8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 lds_half8(const _Float16 *p)
{
    return *reinterpret_cast<const half8 *>(p);
}

// The carry feeds MFMA outputs straight back in as MFMA operands. A 16x16
// output tile leaves lane l holding rows 4(l/16) .. 4(l/16)+3 of column l%16;
// two such tiles (rows r and r+16) make up the 8 k-values one lane supplies to
// a 16x16x32 product. Every matrix contracted against them is therefore stored
// with each 32-wide block of the contracted index reordered so that slot
// 8g + i holds index 4g + i (i < 4) or 16 + 4g + (i - 4) (i >= 4).
__host__ __device__ constexpr int perm_pos(int c)  // slot of index c within its 32-block
{
    return (c & ~31) | (8 * ((c & 15) >> 2) + (c & 3) + 4 * ((c >> 4) & 1));
}
__host__ __device__ constexpr int perm_idx(int p)  // index held by slot p
{
    return (p & ~31) | (4 * ((p >> 3) & 3) + (p & 3) + 16 * ((p >> 2) & 1));
}
static_assert(perm_idx(perm_pos(21)) == 21 && perm_pos(perm_idx(13)) == 13, "permutation");

// ---------------------------------------------------------------- workspace

struct WsLayout {
    size_t chunk_seq, chunk_start, chunk_len, seq_chunk0, qn, knT, wmat, umat, aqk, gcum, onorm, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(int Hk, int Hv, int64_t MC, int N, int64_t total_tokens, bool norm)
{
    WsLayout L{};
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
    L.qn = take(sizeof(uint16_t) * MC * Hk * C * DH);
    L.knT = take(sizeof(uint16_t) * MC * Hk * DH * C);
    L.wmat = take(sizeof(uint16_t) * MC * Hv * C * DH);
    L.umat = take(sizeof(float) * MC * Hv * C * DH);
    L.aqk = take(sizeof(uint16_t) * MC * Hv * C * C);
    L.gcum = take(sizeof(float) * MC * Hv * 2 * C);
    L.onorm = norm ? take(sizeof(float) * (size_t)total_tokens * Hv * DH) : off;
    L.total = off;
    return L;
}

// ---------------------------------------------------------------- 1. plan

__global__ __launch_bounds__(256) void plan_kernel(PrefillParams p)
{
    __shared__ int scan[256];
    __shared__ int base_s;
    if (threadIdx.x == 0)
        base_s = 0;
    __syncthreads();
    for (int i0 = 0; i0 < p.N; i0 += 256) {
        const int i = i0 + threadIdx.x;
        int start = 0, len = 0;
        if (i < p.N) {
            start = p.cu[i];
            len = p.cu[i + 1] - start;
        }
        const int nc = (len + C - 1) / C;
        scan[threadIdx.x] = nc;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {  // inclusive Hillis-Steele scan
            const int v = threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
            __syncthreads();
            scan[threadIdx.x] += v;
            __syncthreads();
        }
        const int first = base_s + scan[threadIdx.x] - nc;
        if (i < p.N) {
            p.seq_chunk0[i] = first;
            for (int c = 0; c < nc; ++c) {
                p.chunk_seq[first + c] = i;
                p.chunk_start[first + c] = start + c * C;
                p.chunk_len[first + c] = min(C, len - c * C);
            }
        }
        __syncthreads();
        if (threadIdx.x == 255)
            base_s += scan[255];
        __syncthreads();
    }
}

// ---------------------------------------------------------------- 2. prep

template <int QT>
__global__ __launch_bounds__(256, 2) void prep_kernel(PrefillParams p)
{
    // LDS: X1 = normalised K rows (f16) then A / T (f32, in place);
    //      X2 = normalised Q rows (f16) then the block-product scratch (f32).
    __shared__ __attribute__((aligned(16))) unsigned char X1[C * AP * 4];
    __shared__ __attribute__((aligned(16))) unsigned char X2[C * KP * 2];
    __shared__ __attribute__((aligned(16))) _Float16 VbT[DH][TP];  // beta_t v_t, transposed
    __shared__ __attribute__((aligned(16))) _Float16 KbT[DH][TP];  // beta_t gamma_t k_t, transposed
    __shared__ float G_s[C], beta_s[C];
    static_assert(C * AP * 4 >= C * KP * 2, "X1 holds both the K rows and A / T");
    static_assert(C * KP * 2 >= 32 * 36 * 4, "X2 holds the Q rows and the 32x32 scratch");

    _Float16(*Kh)[KP] = reinterpret_cast<_Float16(*)[KP]>(X1);
    _Float16(*Qh)[KP] = reinterpret_cast<_Float16(*)[KP]>(X2);
    float(*Am)[AP] = reinterpret_cast<float(*)[AP]>(X1);
    float(*Pm)[36] = reinterpret_cast<float(*)[36]>(X2);

    const HeadCfg &hc = p.hc;
    const ActInputs &in = p.in;
    const int Hv = hc.Hv, Hk = hc.Hk;
    const int chunk = blockIdx.x / Hv;
    const int h = blockIdx.x % Hv;
    const int kh = k_head_of(hc.head_map, h, Hk, Hv);
    const int tok0 = p.chunk_start[chunk];
    const int n = p.chunk_len[chunk];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t flags = hc.flags;
    // one of the v-heads reading kh writes the normalised Q and K^T for the carry
    const bool qk_writer = hc.head_map == 0 ? (h % (Hv / Hk) == 0) : (h < Hk);

    // -- gates and their prefix sums (wave 0, lane = token)
    if (wave == 0) {
        float g = 0.f, beta = 0.f;
        if (lane < n) {
            const int64_t gi = (int64_t)(tok0 + lane) * Hv + h;
            if (flags & F_RAW_GATES) {
                const float dp = in.decay_param[h];
                const float rate = hc.decay_kind == 0 ? -expf(dp) : dp;
                g = rate * softplus_f(load_act(in.a, gi, in.ab_dt) + in.dt_bias[h]);
                beta = sigmoid_f(load_act(in.b, gi, in.ab_dt));
            } else {
                g = in.g[gi];
                beta = in.beta[gi];
            }
        }
        float G = g;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_up(G, off, 64);
            if (lane >= off)
                G += o;
        }
        G_s[lane] = G;  // tokens >= n carry G_{n-1} (their g is 0)
        beta_s[lane] = beta;
    }
    __syncthreads();

    // -- rows of k and q: wave w loads tokens 16w .. 16w+15, 32 lanes per row;
    // rows past the chunk's end re-read its last row and are zeroed after.
    {
        const int sub = lane >> 5, c4 = (lane & 31) * 4;
        Raw4<QT> kr[8], qr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = wave * 16 + 2 * i + sub;
            const int64_t r = tok0 + min(t, n - 1);
            kr[i] = load_raw4<QT>(in.k, r * in.k_stride + (int64_t)kh * DH + c4);
            qr[i] = load_raw4<QT>(in.q, r * in.q_stride + (int64_t)kh * DH + c4);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = wave * 16 + 2 * i + sub;
            float4 kk = raw4_to_f32<QT>(kr[i]), qq = raw4_to_f32<QT>(qr[i]);
            if (flags & F_L2NORM) {
                const float ik = rsqrtf(group_sum<32>(dot4(kk, kk)) + hc.l2_eps);
                const float iq = rsqrtf(group_sum<32>(dot4(qq, qq)) + hc.l2_eps);
                kk.x *= ik; kk.y *= ik; kk.z *= ik; kk.w *= ik;
                qq.x *= iq; qq.y *= iq; qq.z *= iq; qq.w *= iq;
            }
            const float keep = t < n ? 1.f : 0.f;
            typedef _Float16 half4 __attribute__((ext_vector_type(4)));
            const half4 kh4 = {(_Float16)(keep * kk.x), (_Float16)(keep * kk.y),
                               (_Float16)(keep * kk.z), (_Float16)(keep * kk.w)};
            const half4 qh4 = {(_Float16)(keep * qq.x), (_Float16)(keep * qq.y),
                               (_Float16)(keep * qq.z), (_Float16)(keep * qq.w)};
            *reinterpret_cast<half4 *>(&Kh[t][c4]) = kh4;
            *reinterpret_cast<half4 *>(&Qh[t][c4]) = qh4;
        }
    }
    __syncthreads();

    // -- transposed tiles, one (dim, 8-token octet) item per 16-byte LDS write:
    // beta v from the input (lanes along dim: coalesced), beta gamma k from the
    // f16 rows just written (the same rounded K the gram and the carry use).
#pragma unroll
    for (int it = 0; it < (DH * C / 8) / 256; ++it) {
        const int e = it * 256 + threadIdx.x;
        const int j = e % DH, o = e / DH;
        half8 vb, kb;
        uint32_t vr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t r = tok0 + min(o * 8 + i, n - 1);
            vr[i] = load_raw1<QT>(in.v, r * in.v_stride + (int64_t)h * DH + j);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = o * 8 + i;
            const float bt = beta_s[t];  // 0 for tokens past the chunk's end
            vb[i] = (_Float16)(bt * raw1_to_f32<QT>(vr[i]));
            kb[i] = (_Float16)(bt * __expf(G_s[t]) * (float)Kh[t][j]);
        }
        *reinterpret_cast<half8 *>(&VbT[j][o * 8]) = vb;
        *reinterpret_cast<half8 *>(&KbT[j][o * 8]) = kb;
    }
    __syncthreads();

    // -- K K^T and Q K^T on the lower block triangle: wave w owns token rows 16w..
    const int li = lane & 15, lg = lane >> 4;
    f32x4 gram[4], qk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        gram[j] = {0.f, 0.f, 0.f, 0.f};
        qk[j] = {0.f, 0.f, 0.f, 0.f};
        if (j <= wave) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const half8 ka = lds_half8(&Kh[wave * 16 + li][ks * 32 + lg * 8]);
                const half8 qa = lds_half8(&Qh[wave * 16 + li][ks * 32 + lg * 8]);
                const half8 kb = lds_half8(&Kh[j * 16 + li][ks * 32 + lg * 8]);
                gram[j] = mfma16(ka, kb, gram[j]);
                qk[j] = mfma16(qa, kb, qk[j]);
            }
        }
    }

    // normalised Q rows and K^T go to the workspace for the carry
    if (qk_writer) {
        uint16_t *qdst = p.qn + ((int64_t)chunk * Hk + kh) * C * DH;
        uint16_t *kdst = p.knT + ((int64_t)chunk * Hk + kh) * DH * C;
        for (int e = threadIdx.x; e < C * DH / 8; e += 256) {
            const int t = e / (DH / 8), c8 = (e % (DH / 8)) * 8;
            half8 v;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = Qh[t][perm_idx(c8 + i)];
            *reinterpret_cast<half8 *>(qdst + t * DH + c8) = v;
        }
        for (int e = threadIdx.x; e < DH * C / 8; e += 256) {
            const int dk = e % DH, t8 = (e / DH) * 8;
            half8 v;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = Kh[perm_idx(t8 + i)][dk];
            *reinterpret_cast<half8 *>(kdst + dk * C + t8) = v;
        }
    }
    __syncthreads();  // Kh / Qh are dead from here: X1 becomes A / T, X2 scratch

    // -- A (strictly lower, f32) into X1; decayed, masked Q K^T to the workspace
    {
        uint16_t *aq = p.aqk + ((int64_t)chunk * Hv + h) * C * C;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = wave * 16 + lg * 4 + r, s = j * 16 + li;
                const float dg = s <= t ? __expf(G_s[t] - G_s[s]) : 0.f;
                Am[t][s] = s < t ? beta_s[t] * dg * gram[j][r] : 0.f;
                aq[t * C + perm_pos(s)] = f32_to_f16_bits(dg * qk[j][r]);
            }
        }
    }
    __syncthreads();

    // -- T = (I + A)^-1 in place. (a) the four 16x16 diagonal blocks by forward
    // substitution: wave 0, lane = (block, column).
    if (wave == 0) {
        const int b0 = (lane >> 4) * 16, c = lane & 15;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int s = 0; s < r; ++s)
                acc += Am[b0 + r][b0 + s] * x[s];
            x[r] = r < c ? 0.f : (r == c ? 1.f : -acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
            Am[b0 + r][b0 + c] = x[r];
    }
    __syncthreads();
    // (b) 32x32 diagonal halves: T10 = -T11 (A10 T00), waves 0 and 1 (blocks 1,0 and 3,2)
    if (wave < 2) {
        const int bi = (2 * wave + 1) * 16, bj = 2 * wave * 16;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            acc = mfma4(Am[bi + li][bj + ks * 4 + lg], Am[bj + ks * 4 + lg][bj + li], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Pm[wave * 16 + lg * 4 + r][li] = acc[r];
    }
    __syncthreads();
    if (wave < 2) {
        const int bi = (2 * wave + 1) * 16, bj = 2 * wave * 16;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            acc = mfma4(Am[bi + li][bi + ks * 4 + lg], Pm[wave * 16 + ks * 4 + lg][li], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Am[bi + lg * 4 + r][bj + li] = -acc[r];
    }
    __syncthreads();
    // (c) lower-left 32x32: T_LL = -T_11 (A_LL T_00); wave = one 16x16 output tile
    {
        const int ti = wave >> 1, tj = wave & 1;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            acc = mfma4(Am[32 + ti * 16 + li][ks * 4 + lg], Am[ks * 4 + lg][tj * 16 + li], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Pm[ti * 16 + lg * 4 + r][tj * 16 + li] = acc[r];
    }
    __syncthreads();
    {
        const int ti = wave >> 1, tj = wave & 1;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            acc = mfma4(Am[32 + ti * 16 + li][32 + ks * 4 + lg], Pm[ks * 4 + lg][tj * 16 + li], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Am[32 + ti * 16 + lg * 4 + r][tj * 16 + li] = -acc[r];
    }
    __syncthreads();

    // -- U = T (beta V) and W = T (beta gamma K): wave w owns token rows 16w..
    {
        half8 ta[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                ta[ks][i] = (_Float16)Am[wave * 16 + li][ks * 32 + lg * 8 + i];
        float *ud = p.umat + ((int64_t)chunk * Hv + h) * C * DH;
        uint16_t *wd = p.wmat + ((int64_t)chunk * Hv + h) * C * DH;
#pragma unroll
        for (int nt = 0; nt < DH / 16; ++nt) {
            f32x4 u = {0.f, 0.f, 0.f, 0.f}, w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                u = mfma16(ta[ks], lds_half8(&VbT[nt * 16 + li][ks * 32 + lg * 8]), u);
                w = mfma16(ta[ks], lds_half8(&KbT[nt * 16 + li][ks * 32 + lg * 8]), w);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = wave * 16 + lg * 4 + r;
                ud[t * DH + nt * 16 + li] = u[r];
                wd[t * DH + perm_pos(nt * 16 + li)] = f32_to_f16_bits(w[r]);
            }
        }
    }
    if (threadIdx.x < C) {
        // decay factors the carry multiplies by: gamma_t = exp(G_t) and
        // exp(G_last - G_t) (G_last = G at the chunk's last token = G_s[C-1])
        float *gd = p.gcum + ((int64_t)chunk * Hv + h) * 2 * C;
        gd[threadIdx.x] = __expf(G_s[threadIdx.x]);
        gd[C + threadIdx.x] = __expf(G_s[C - 1] - G_s[threadIdx.x]);
    }
}

// ---------------------------------------------------------------- 3. carry

// OUT: the output's dtype, or kOutNorm for the f32 buffer the gated norm reads
constexpr int kOutNorm = 3;

template <int OUT>
__device__ __forceinline__ void store_out(const PrefillParams &p, int64_t idx, float v)
{
    if constexpr (OUT == kOutNorm)
        p.onorm[idx] = v;
    else if constexpr (OUT == DT_F32)
        static_cast<float *>(p.out)[idx] = v;
    else if constexpr (OUT == DT_BF16)
        static_cast<uint16_t *>(p.out)[idx] = f32_to_bf16_bits(v);
    else
        static_cast<uint16_t *>(p.out)[idx] = f32_to_f16_bits(v);
}

// LDS image of one chunk's operands for a workgroup covering NU dv slices. Rows are
// stored with their 16-byte blocks XOR-swizzled so the rows one MFMA operand
// read touches fall in distinct banks: 256-byte rows (W, Q) use
// block ^ (row & 15), 128-byte rows (K^T, Aqk) use block ^ ((row >> 1) & 7).
// u holds the workgroup's 16*NU columns of U, gd the two decay factors per token.
template <int NU>
struct ChunkImage {
    unsigned char w[C * DH * 2];   // W  [t][dk (permuted)]
    unsigned char q[C * DH * 2];   // Q  [t][dk (permuted)]
    unsigned char kt[DH * C * 2];  // K^T [dk][t (permuted)]
    unsigned char aq[C * C * 2];   // Aqk [t][s (permuted)]
    float u[C][16 * NU];           // U  [t][dv0 .. dv0 + 16 NU), blocks swizzled (NU > 1)
    float gd[4 * C];               // [t] = gamma_t, [C + t] = exp(G_last - G_t); [2C, 4C) repeats
};

__device__ __forceinline__ int swz256(int row, int blk) { return row * 256 + 16 * (blk ^ (row & 15)); }
__device__ __forceinline__ int swz128(int row, int blk) { return row * 128 + 16 * (blk ^ ((row >> 1) & 7)); }

typedef __attribute__((address_space(3))) void lds_void;

// Issue the asynchronous global -> LDS copies of one chunk's operands; the
// NW waves of the workgroup split the 56 one-KiB pieces between them.
template <int NU>
__device__ __forceinline__ int swzu(int row, int blk)
{
    if constexpr (NU == 1)
        return blk;  // 64-byte rows: the 16 banks they span are read 4 rows at a time anyway
    else
        return blk ^ (2 * ((row >> 2) & 3));
}

template <int NW, int NU>
__device__ __forceinline__ void issue_chunk_copy(ChunkImage<NU> &img, const PrefillParams &p, int chunk,
                                                 int h, int kh, int dvw, int wave, int lane)
{
    const int Hv = p.hc.Hv, Hk = p.hc.Hk;
    const unsigned char *wg = reinterpret_cast<const unsigned char *>(p.wmat + ((int64_t)chunk * Hv + h) * C * DH);
    const unsigned char *qg = reinterpret_cast<const unsigned char *>(p.qn + ((int64_t)chunk * Hk + kh) * C * DH);
    const unsigned char *kg = reinterpret_cast<const unsigned char *>(p.knT + ((int64_t)chunk * Hk + kh) * DH * C);
    const unsigned char *ag = reinterpret_cast<const unsigned char *>(p.aqk + ((int64_t)chunk * Hv + h) * C * C);
    // W and Q: 16 pieces each of 4 rows x 256 B; K^T: 16 pieces and Aqk: 8
    // pieces of 8 rows x 128 B. Each lane fetches the global block that the
    // swizzle places at its 16-byte slot of the piece.
    static_assert(16 % NW == 0 && 8 % NW == 0, "pieces split evenly");
#pragma unroll
    for (int k = 0; k < 16 / NW; ++k) {
        const int q = k * NW + wave;
        const int row = 4 * q + (lane >> 4), slot = lane & 15;
        const int goff = row * 256 + 16 * (slot ^ (row & 15));
        __builtin_amdgcn_global_load_lds(wg + goff, (lds_void *)(img.w + q * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(qg + goff, (lds_void *)(img.q + q * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 16 / NW; ++k) {
        const int q = k * NW + wave;
        const int row = 8 * q + (lane >> 3), slot = lane & 7;
        __builtin_amdgcn_global_load_lds(kg + row * 128 + 16 * (slot ^ ((row >> 1) & 7)),
                                         (lds_void *)(img.kt + q * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 8 / NW; ++k) {
        const int q = k * NW + wave;
        const int row = 8 * q + (lane >> 3), slot = lane & 7;
        __builtin_amdgcn_global_load_lds(ag + row * 128 + 16 * (slot ^ ((row >> 1) & 7)),
                                         (lds_void *)(img.aq + q * 1024), 16, 0, 0);
    }
    // U columns [dvw, dvw + 16 NU): rows of 64 NU bytes (4 NU blocks)
    constexpr int UB = 4 * NU, UROWS = 64 / UB;  // blocks per row, rows per piece
    static_assert((4 * NU) % NW == 0, "U pieces split evenly");
    const unsigned char *ug = reinterpret_cast<const unsigned char *>(
        p.umat + ((int64_t)chunk * Hv + h) * C * DH + dvw);
#pragma unroll
    for (int k = 0; k < (4 * NU) / NW; ++k) {
        const int q = k * NW + wave;
        const int row = UROWS * q + lane / UB, slot = lane % UB;
        const int goff = row * (DH * 4) + 16 * swzu<NU>(row, slot);
        unsigned char *dst = reinterpret_cast<unsigned char *>(&img.u[0][0]) + q * 1024;
        __builtin_amdgcn_global_load_lds(ug + goff, (lds_void *)dst, 16, 0, 0);
    }
    if (wave == 0) {  // 512 bytes of decay factors (lanes 32..63 repeat them)
        const unsigned char *gg = reinterpret_cast<const unsigned char *>(p.gcum + ((int64_t)chunk * Hv + h) * 2 * C);
        __builtin_amdgcn_global_load_lds(gg + 16 * (lane & 31), (lds_void *)img.gd, 16, 0, 0);
    }
}

__device__ __forceinline__ half8 img_read(const unsigned char *base, int off)
{
    return *reinterpret_cast<const half8 *>(base + off);
}

// Carry: one workgroup of 4 waves per (sequence, v-head, 16-row slice of dv),
// sequential over the sequence's chunks. The state slice S[dv0..dv0+16)[:] lives
// in MFMA accumulators (f32; wave w holds dk columns 32w..32w+31) with an f16
// copy in LDS as the B operand of W S^T and Q S^T. Per chunk, wave w owns token
// rows 16w..16w+15:
//   P  = W S^T, QS = Q S^T
//   D  = U - P,  D~ = D exp(G_last - G_t)            (to LDS, token index permuted)
//   O  = scale (gamma QS + Aqk D)
//   S <- gamma_last S + D~^T K                       (D~ as an f16 hi + lo pair)
// The chunk's operands (W, Q, K^T, Aqk, U slice, decay factors) arrive in LDS by
// asynchronous global->LDS copies issued one chunk ahead into a two-slot ring;
// outputs are stored one chunk late. Two barriers per chunk.
template <int OUT>
__global__ __launch_bounds__(256, 1) void carry_kernel(PrefillParams p)
{
    constexpr int NW = 4;
    __shared__ __attribute__((aligned(16))) ChunkImage<1> img[2];
    __shared__ __attribute__((aligned(16))) _Float16 Sh[2][DT][KP];   // f16 state slice, dk permuted
    __shared__ __attribute__((aligned(16))) _Float16 DTl[DT][TP];     // D^T, token permuted
    __shared__ __attribute__((aligned(16))) _Float16 DsH[DT][TP];     // (decayed D)^T, hi part
    __shared__ __attribute__((aligned(16))) _Float16 DsL[DT][TP];     // (decayed D)^T, lo part

    const HeadCfg &hc = p.hc;
    const int Hv = hc.Hv;
    constexpr int NT = DH / DT;  // dv slices per head
    // XCD-aware order: the NT slices of one (sequence, head) share id % 8
    const int id = blockIdx.x;
    const int group = (id & 7) + 8 * (id / (8 * NT));
    const int slice = (id >> 3) % NT;
    if (group >= p.N * Hv)
        return;
    const int seq = group / Hv, h = group % Hv;
    const int kh = k_head_of(hc.head_map, h, hc.Hk, Hv);
    const int dv0 = slice * DT;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int start = p.cu[seq];
    const int len = p.cu[seq + 1] - start;
    const int nch = (len + C - 1) / C;
    if (nch == 0)
        return;  // empty sequence: state untouched
    const int c0 = p.seq_chunk0[seq];

    // state slice: wave w holds dk columns 32w .. 32w+31 as two 16x16 tiles
    float *Sg = p.state + ((int64_t)seq * Hv + h) * DH * DH;
    f32x4 S[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int dk = wave * 32 + nt * 16 + li;
            S[nt][r] = Sg[(int64_t)(dv0 + lg * 4 + r) * DH + dk];
            Sh[0][lg * 4 + r][perm_pos(dk)] = (_Float16)S[nt][r];
        }

    issue_chunk_copy<NW, 1>(img[0], p, c0, h, kh, dv0, wave, lane);
    f32x4 Oprev = {0.f, 0.f, 0.f, 0.f};
    int prev_tok0 = 0, prev_n = 0;

    for (int ci = 0; ci < nch; ++ci) {
        // this chunk's copies (issued one iteration ago), older stores, LDS writes
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        if (ci > 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = wave * 16 + lg * 4 + r;
                if (t < prev_n)
                    store_out<OUT>(p, ((int64_t)(prev_tok0 + t) * Hv + h) * DH + dv0 + li,
                                   hc.scale * Oprev[r]);
            }
        }
        if (ci + 1 < nch)
            issue_chunk_copy<NW, 1>(img[(ci + 1) & 1], p, c0 + ci + 1, h, kh, dv0, wave, lane);
        const ChunkImage<1> &cur = img[ci & 1];
        const int sb = ci & 1;

        // P = W S0^T and QS = Q S0^T for token rows 16w..16w+15
        f32x4 P = {0.f, 0.f, 0.f, 0.f}, QS = {0.f, 0.f, 0.f, 0.f};
        const int trow = wave * 16 + li;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const half8 b = lds_half8(&Sh[sb][li][ks * 32 + lg * 8]);
            P = mfma16(img_read(cur.w, swz256(trow, 4 * ks + lg)), b, P);
            QS = mfma16(img_read(cur.q, swz256(trow, 4 * ks + lg)), b, QS);
        }
        // D = U - P; the decayed D as an f16 hi + lo pair; gamma QS
        f32x4 O;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = wave * 16 + lg * 4 + r;
            const float d = cur.u[t][li] - P[r];
            const float ds = d * cur.gd[C + t];
            const _Float16 dh = (_Float16)ds;
            const int tp = perm_pos(t);
            DTl[li][tp] = (_Float16)d;
            DsH[li][tp] = dh;
            DsL[li][tp] = (_Float16)(ds - (float)dh);
            O[r] = cur.gd[t] * QS[r];
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();

        // O += Aqk D (only the token blocks at or below this wave's rows)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            if (2 * ks <= wave)
                O = mfma16(img_read(cur.aq, swz128(trow, 4 * ks + lg)),
                           lds_half8(&DTl[li][ks * 32 + lg * 8]), O);
        // S_n = gamma_last S0 + D~^T K
        const float gn = cur.gd[C - 1];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            S[nt] *= gn;
            const int krow = wave * 32 + nt * 16 + li;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const half8 kb = img_read(cur.kt, swz128(krow, 4 * ks + lg));
                S[nt] = mfma16(lds_half8(&DsH[li][ks * 32 + lg * 8]), kb, S[nt]);
                S[nt] = mfma16(lds_half8(&DsL[li][ks * 32 + lg * 8]), kb, S[nt]);
            }
        }
        Oprev = O;
        prev_tok0 = start + ci * C;
        prev_n = min(C, len - ci * C);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Sh[sb ^ 1][lg * 4 + r][perm_pos(wave * 32 + nt * 16 + li)] = (_Float16)S[nt][r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = wave * 16 + lg * 4 + r;
        if (t < prev_n)
            store_out<OUT>(p, ((int64_t)(prev_tok0 + t) * Hv + h) * DH + dv0 + li,
                           hc.scale * Oprev[r]);
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Sg[(int64_t)(dv0 + lg * 4 + r) * DH + wave * 32 + nt * 16 + li] = S[nt][r];
}

// ---------------------------------------------------------------- 4. gated norm

__global__ __launch_bounds__(256) void norm_kernel(PrefillParams p)
{
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (token, v-head)
    if (row >= (int64_t)p.total * p.hc.Hv)
        return;
    const int lane = threadIdx.x & 63;
    const float *o = p.onorm + row * DH;
    const float o0 = o[lane], o1 = o[lane + 64];
    const float ss = group_sum<64>(o0 * o0 + o1 * o1);
    const float inv = rsqrtf(ss / (float)DH + p.hc.norm_eps);
    const float z0 = load_act(p.in.z, row * DH + lane, p.in.z_dt);
    const float z1 = load_act(p.in.z, row * DH + lane + 64, p.in.z_dt);
    store_act(p.out, row * DH + lane, p.out_dt, o0 * inv * p.in.norm_w[lane] * silu_f(z0));
    store_act(p.out, row * DH + lane + 64, p.out_dt, o1 * inv * p.in.norm_w[lane + 64] * silu_f(z1));
}

}  // namespace

bool prefill_supported(int dk, int dv) { return dk == DH && dv == DH; }

size_t prefill_workspace_bytes(int Hk, int Hv, int dk, int dv, int64_t max_chunks, int N,
                               int64_t total_tokens, bool norm)
{
    (void)dk;
    (void)dv;
    return ws_layout(Hk, Hv, max_chunks, N, total_tokens, norm).total;
}

void prefill_carve(PrefillParams &p, void *ws, int64_t max_chunks)
{
    const WsLayout L = ws_layout(p.hc.Hk, p.hc.Hv, max_chunks, p.N, p.total,
                                 (p.hc.flags & F_GATED_NORM) != 0);
    unsigned char *b = static_cast<unsigned char *>(ws);
    p.chunk_seq = reinterpret_cast<int32_t *>(b + L.chunk_seq);
    p.chunk_start = reinterpret_cast<int32_t *>(b + L.chunk_start);
    p.chunk_len = reinterpret_cast<int32_t *>(b + L.chunk_len);
    p.seq_chunk0 = reinterpret_cast<int32_t *>(b + L.seq_chunk0);
    p.qn = reinterpret_cast<uint16_t *>(b + L.qn);
    p.knT = reinterpret_cast<uint16_t *>(b + L.knT);
    p.wmat = reinterpret_cast<uint16_t *>(b + L.wmat);
    p.umat = reinterpret_cast<float *>(b + L.umat);
    p.aqk = reinterpret_cast<uint16_t *>(b + L.aqk);
    p.gcum = reinterpret_cast<float *>(b + L.gcum);
    p.onorm = reinterpret_cast<float *>(b + L.onorm);
}

hipError_t launch_prefill(const PrefillParams &p, hipStream_t s)
{
    if (p.num_chunks == 0)
        return hipSuccess;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, s, p);
    const dim3 pgrid((unsigned)((int64_t)p.num_chunks * p.hc.Hv));
    switch (p.in.qkv_dt) {
    case DT_F32: hipLaunchKernelGGL((prep_kernel<DT_F32>), pgrid, dim3(256), 0, s, p); break;
    case DT_F16: hipLaunchKernelGGL((prep_kernel<DT_F16>), pgrid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((prep_kernel<DT_BF16>), pgrid, dim3(256), 0, s, p); break;
    }
    const int64_t groups = (int64_t)p.N * p.hc.Hv;
    const dim3 cgrid((unsigned)((groups + 7) / 8 * 8 * (DH / DT)));
    const int omode = (p.hc.flags & F_GATED_NORM) ? kOutNorm : p.out_dt;
    switch (omode) {
    case kOutNorm: hipLaunchKernelGGL((carry_kernel<kOutNorm>), cgrid, dim3(256), 0, s, p); break;
    case DT_F32: hipLaunchKernelGGL((carry_kernel<DT_F32>), cgrid, dim3(256), 0, s, p); break;
    case DT_F16: hipLaunchKernelGGL((carry_kernel<DT_F16>), cgrid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((carry_kernel<DT_BF16>), cgrid, dim3(256), 0, s, p); break;
    }
    if (p.hc.flags & F_GATED_NORM) {
        const int64_t rows = (int64_t)p.total * p.hc.Hv;
        hipLaunchKernelGGL(norm_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace gdn
